/*
 * kpage.h -- C ABI of a gfx950 (MI355X) implementation of KPage-style
 * block-sparse attention over flattened T x H x W video token layouts.
 *
 * Source: "KPage: Cross-Block Page Compaction for Hardware-Efficient Sparse
 * Attention" (arXiv 2610.28096).  Section numbers below refer to that paper.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are caller-owned device buffers, bf16 (bfloat16), contiguous
 *    [batch, heads, rows, head_dim], 16-byte aligned:
 *      Q, O, dO, dQ : rows = seq_q  (= 128 * n_q_blocks; query block q owns
 *                                    rows [128 q, 128 q + 128), valid rows first)
 *      K, V, dK, dV : rows = seq_kv (K/V block k owns rows
 *                                    [kv_offset[k], kv_offset[k] + kv_valid[k]))
 *    LSE is fp32 [batch, heads, seq_q] (natural log).
 *  - Every row of K and V that lies inside a block's 16-row page footprint
 *    must hold finite values, padded rows included (section 3.2.4: padding is
 *    masked before the row maximum; the paper zeroes it, a finite value is
 *    enough for exact results).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    device work is asynchronous on that stream; kernel faults surface at the
 *    caller's next synchronisation.
 *  - No exception crosses the ABI.  A non-OK status leaves a thread-local
 *    message readable with kpage_last_error().  Descriptor errors are reported
 *    before any device work is enqueued.
 */
#ifndef KPAGE_H
#define KPAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KPAGE_OK = 0,
  KPAGE_ERR_INVALID = 1,      /* malformed descriptor, pointer or size           */
  KPAGE_ERR_UNSUPPORTED = 2,  /* well formed but outside what is implemented     */
  KPAGE_ERR_OOM = 3,          /* host or device allocation failed                */
  KPAGE_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed      */
} kpage_status;

typedef struct kpage_plan kpage_plan_t;

/*
 * Problem descriptor (host memory, read only during kpage_plan()).
 * Section 3.4.1: per-head Q block sizes c^Q, K/V block sizes c^K and
 * Page16-aligned offsets o^K with disjoint page footprints, and the ordered
 * per-query-block lists K_q of selected K/V blocks.  The shared blk128 layout
 * is the special case n_q = n_kv, c^Q = c^K, o^K = 128 k.
 *
 * G = 1 graph slot when per_head == 0 (one layout and graph for every
 * (batch, head)), G = batch * heads when per_head == 1 (slot b * heads + h).
 */
typedef struct {
  int32_t batch, heads, head_dim;   /* head_dim in {64, 128}                         */
  int32_t n_q_blocks, n_kv_blocks;  /* >= 1                                          */
  int64_t seq_q, seq_kv;            /* seq_q == 128 * n_q_blocks; seq_kv % 16 == 0    */
  int32_t per_head;                 /* 0 or 1                                        */
  const int32_t *q_valid;           /* [G][n_q]  valid rows per Q block, in [0,128]  */
  const int32_t *kv_valid;          /* [G][n_kv] valid rows per K/V block, in [0,128]*/
  const int64_t *kv_offset;         /* [G][n_kv] first row, % 16 == 0; NULL: 128 k   */
  const int64_t *q2k_ptr;           /* [G][n_q + 1] offsets into q2k_idx (CSR rows)  */
  const int32_t *q2k_idx;           /* K/V block ids in [0, n_kv), unique per row    */
} kpage_problem;

/*
 * Planner options (NULL = defaults).  Section 3.2.2: the Q64 path consumes 16
 * pages per iteration and the Q128 path 8, so walks are padded with dummy pages
 * to a multiple of align_q64 / align_q128 (defaults 16 / 8; multiples of those
 * values are accepted).  q_group is the Q-group size of section 3.3.2, in Q
 * blocks: 0 = one group; n > 0 bounds the serial Q work of a backward work item
 * at n Q blocks: an owner whose reverse neighbourhood holds more than n Q blocks
 * is split into the groups [g n, (g + 1) n) of Q blocks, one work item per
 * non-empty (owner, group); an owner with at most n keeps its whole list in
 * group 0 (one item, no partials).  An owner split over several items sums fp32
 * partials of dK/dV (in group order, deterministic) in the backward workspace.
 * Negative values are KPAGE_ERR_INVALID.
 *
 * ungrouped = 0 (default) lets kpage_plan() run query blocks of the Q64 route with
 * at most 32 valid rows in group items: up to four such blocks whose K/V walks
 * overlap share one M128 x N128 work item of the forward and dQ passes over the
 * union of their walks (each block's rows mask the pages it did not select), so a
 * page they share is gathered once.  This is a launch-level choice outside the
 * paper's tables (section 3.2.2 routes such blocks to M64 x N256 one at a time):
 * the exported tables, queues and pair counts do not change, and each row's result
 * is the same attention up to fp32 summation order.  ungrouped = 1 runs every
 * block as its own item.  kpage_plan_device() builds the same groups as kpage_plan()
 * (with ungrouped = 1, none).  Grouping applies where the page bitsets fit the GPU
 * planner: seq_kv up to 2^21 rows, at most 16384 candidate blocks per graph slot, and
 * all slots' candidate bitsets together at most 2^25 64-bit words (both planners use
 * these limits).
 */
typedef struct {
  int32_t q_group;
  int32_t align_q128;
  int32_t align_q64;
  int32_t ungrouped;
} kpage_plan_opts;

/* Section 4.4 pair-capacity accounting, summed over batch, heads and non-empty
 * query blocks (see kpage_plan_stats). */
typedef struct {
  uint64_t useful;            /* sum over edges of c_q * c_k                         */
  uint64_t whole_block;       /* 128 * 128 per selected block                        */
  uint64_t paged_m128;        /* 128 * 16 * pages of the selected blocks              */
  uint64_t nominal;           /* M_q * 16 * pages, M_q = 64 or 128 by route           */
  uint64_t scheduled;         /* M_q * 16 * walk length including dummy pages        */
  uint64_t bwd_physical;      /* 128 * 128 per backward step (lazy; 0 until built)   */
  uint64_t bwd_useful_check;  /* valid pairs visited by backward; equals useful      */
} kpage_pair_stats;

/*
 * Build the forward metadata (section 3.4): Page16 walks of every query block
 * (full pages of K_q in order, then one tail page per partial block, then dummy
 * pages), Q64/Q128 routes (section 3.2.2), per-route work queues ordered by
 * descending walk length, validity words (two 16-bit page masks per uint32,
 * section 3.2.4) and the index of the end of the fully valid prefix.
 * Host-only: no device memory is touched here; tables are copied to the device
 * on first use (kpage_plan_upload or the first attention call).
 * Returns KPAGE_ERR_INVALID for a malformed descriptor, KPAGE_ERR_UNSUPPORTED
 * for head_dim not in {64,128}.  *out is owned by the caller
 * and released with kpage_plan_destroy().
 */
kpage_status kpage_plan(const kpage_problem *problem, const kpage_plan_opts *opts,
                        kpage_plan_t **out);

/*
 * The same forward metadata as kpage_plan(), built on the GPU (section 3.4: the
 * metadata depends only on the graph and the sizes, so a block selector that runs
 * on the device can hand its graph to the planner without a host round trip).
 * The descriptor struct is host memory; its arrays q_valid, kv_valid, kv_offset
 * (or NULL), q2k_ptr and q2k_idx are DEVICE pointers to the same layouts as for
 * kpage_plan(), and q2k_idx holds q2k_nnz entries (every q2k_ptr value must lie in
 * [0, q2k_nnz]).  The plan keeps its own copies of the arrays, so the caller may
 * reuse them once this returns.  Tables, queues and pair counts are identical to
 * those of kpage_plan() on the same descriptor.  The descriptor is validated on
 * the device with the same rules (KPAGE_ERR_INVALID, nothing left allocated).
 * Work runs on `stream` (hipStream_t as void*), which is synchronised twice
 * (table sizes, then queue lengths and pair counts).  The backward metadata
 * (section 3.3: owners, reverse-Q lists compacted from an owner x query-block
 * bitmap, Q-page walks, adjacency words, work order) is built on the device too,
 * lazily by the first kpage_attn_bwd() on that call's stream (synchronised twice),
 * or by the first kpage_plan_export() of a backward table (on the null stream);
 * it is identical to kpage_plan()'s.  kpage_plan_export() copies device tables to
 * the host on first use; the descriptor itself never leaves the device.
 */
kpage_status kpage_plan_device(const kpage_problem *problem, int64_t q2k_nnz, const kpage_plan_opts *opts,
                               void *stream, kpage_plan_t **out);

/* Copy the forward tables to the current HIP device on `stream` (idempotent). */
kpage_status kpage_plan_upload(kpage_plan_t *plan, void *stream);

/*
 * Forward attention, section 3.2: for every (b, h) and query block q with
 * c_q > 0, O = softmax(scale * Q K_J^T) V_J over exactly the valid key rows J
 * of the selected blocks (masking before the row maximum, eq. 3), and
 * LSE = log sum exp.  K/V pages are gathered straight into LDS tiles; no
 * compacted copy is written to device memory.  Rows outside the valid prefix
 * of a block, blocks with c_q = 0 and rows with no valid key get O = 0 and
 * LSE = -inf.  q, k, v, o: bf16 device pointers; lse: fp32 device pointer.
 * Two launches on `stream`: the fixed-maximum pass, then an exact re-run of the
 * items it marked, the mark being a NaN written into the item's first LSE row
 * (overwritten by the re-run).  A plan holds no per-call state, so calls on one
 * plan may run concurrently on several streams as long as their o and lse
 * buffers differ.
 */
kpage_status kpage_attn_fwd(kpage_plan_t *plan, const void *q, const void *k, const void *v,
                            void *o, float *lse, float softmax_scale, void *stream);

/* Bytes of device workspace kpage_attn_bwd needs: two fp32 values per query row
 * (LSE * log2(e) and rowsum(dO * O)), i.e. 8 * batch * heads * seq_q; with
 * q_group > 0, rounded up to 256 and followed by 2 * 128 * head_dim fp32 values
 * per work item of an owner split over several Q groups (this call then builds
 * the backward metadata, on the host). */
kpage_status kpage_bwd_workspace_size(kpage_plan_t *plan, size_t *bytes);

/*
 * Backward attention, section 3.3: gradients of sum(O * dO) under the forward
 * definition.  dK and dV are computed over K/V-owned tiles (owners of 8 Page16
 * slots, no logical block crossing an owner), their reverse-Q neighbourhoods
 * packed into 8-page Q steps, and one 64-bit page-pair adjacency word per step
 * that restores the original graph.  dQ is computed by a Q-owned pass over the
 * forward page walks (each query block recomputes its scores), so every output
 * row is written by exactly one workgroup and all three gradients are
 * deterministic.  The backward metadata is built on the first call (lazily,
 * section 3.4).  o and lse are the forward outputs; query rows past c_q of
 * their block (the plan's query sizes, section 3.4.1) are ignored whatever o,
 * lse and dO hold there, and a valid row with LSE = -inf (no valid key)
 * contributes nothing.  Every row of Q and dO must hold finite values, padded
 * rows included (they meet zero weights inside the products).
 * workspace is a caller-owned device buffer of at least
 * kpage_bwd_workspace_size() bytes, 4-byte aligned (16-byte aligned when
 * q_group > 0); at most 2^29 query rows
 * (batch * heads * seq_q) per call.
 * Invalid rows of dQ (by Q sizes) and of dK/dV (by K/V sizes), and rows of
 * blocks with no edge, are written as 0.
 */
kpage_status kpage_attn_bwd(kpage_plan_t *plan, const void *q, const void *k, const void *v,
                            const void *o, const float *lse, const void *dO,
                            void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes,
                            float softmax_scale, void *stream);

/*
 * kpage_attn_bwd without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same kernels and results
 * (bit for bit) as kpage_attn_bwd; the workspace is a static device array of
 * KPAGE_NOALLOC_SCRATCH_BYTES (32 MiB) inside the library, one per device the
 * library runs on, held until the process ends.  Its device address is looked
 * up on the first call on each device (the current device must be the
 * stream's); later calls make no allocation of any kind.
 * Preconditions: the plan's device tables exist, i.e. kpage_attn_bwd has run
 * once on this plan (it builds and uploads them); otherwise KPAGE_ERR_INVALID.
 * A problem whose workspace (kpage_bwd_workspace_size) exceeds 32 MiB, e.g.
 * more than 4,194,304 query rows (batch * heads * seq_q) with one Q group, is
 * rejected with KPAGE_ERR_INVALID before any device work.
 * Every call on one device shares the array and leaves its contents behind
 * (every byte a call reads it first writes): calls that overlap on one device,
 * on any streams, race and must be serialised by the caller.
 */
#define KPAGE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
kpage_status kpage_attn_bwd_noalloc(kpage_plan_t *plan, const void *q, const void *k, const void *v,
                                    const void *o, const float *lse, const void *dO,
                                    void *dq, void *dk, void *dv, float softmax_scale, void *stream);

/* Pair statistics (host memory).  Backward fields are filled once the backward
 * metadata exists (after kpage_attn_bwd or an export of a backward table). */
kpage_status kpage_plan_stats(const kpage_plan_t *plan, kpage_pair_stats *out);

/* Plan tables for offline comparison.  Element types: */
enum {
  KPAGE_T_FWD_ROUTE = 0,      /* int32 [G][n_q]: 0, 64 or 128                         */
  KPAGE_T_FWD_WALK_PTR = 1,   /* int64 [G][n_q + 1]: offsets into FWD_WALK            */
  KPAGE_T_FWD_WALK = 2,       /* int32 page ids (row / 16), -1 = dummy                */
  KPAGE_T_FWD_NFULL = 3,      /* int32 [G][n_q]: length of the fully valid prefix     */
  KPAGE_T_FWD_VALID = 4,      /* uint32: word i of a walk at FWD_WALK_PTR / 2 + i     */
  KPAGE_T_Q64_QUEUE = 5,      /* int32 [n][2]: (b * heads + h, q)                     */
  KPAGE_T_Q128_QUEUE = 6,     /* int32 [n][2]                                         */
  KPAGE_T_OWNER_PTR = 7,      /* int64 [G + 1]: offsets into OWNERS                   */
  KPAGE_T_OWNERS = 8,         /* int32 [n_own][8]: K/V page ids, -1 = empty slot      */
  KPAGE_T_OWNER_ALIGNED = 9,  /* uint8 [n_own]: one block of 8 contiguous pages (plan
                                 metadata only: the kernels read owners page by page) */
  KPAGE_T_REVQ_PTR = 10,      /* int64 [n_own + 1]                                    */
  KPAGE_T_REVQ = 11,          /* int32 Q block ids, ascending per owner               */
  KPAGE_T_QWALK_PTR = 12,     /* int64 [n_own + 1]: offsets into QWALK (multiple of 8)*/
  KPAGE_T_QWALK = 13,         /* int32 Q page ids (8 q + j), -1 = dummy               */
  KPAGE_T_ADJ = 14,           /* uint64: step s of owner t at QWALK_PTR[t] / 8 + s    */
  KPAGE_T_BWD_QUEUE = 15,     /* int32 [n][2]: (b * heads + h, owner within its slot) */
  KPAGE_T_UNCOVERED_PTR = 16, /* int64 [G + 1]: offsets into UNCOVERED                */
  KPAGE_T_UNCOVERED = 17,     /* int32 K/V pages outside every block footprint, ascending */
  /* group items of kpage_plan() (see kpage_plan_opts.ungrouped; empty otherwise) */
  KPAGE_T_GROUP_PTR = 18,     /* int64 [G + 1]: offsets into the group list            */
  KPAGE_T_GROUP_MEMBERS = 19, /* int32 [n_groups][4]: query blocks, -1 = none          */
  KPAGE_T_GROUP_WALK_PTR = 20,/* int64 [n_groups + 1]: offsets into GROUP_WALK (x4)    */
  KPAGE_T_GROUP_WALK = 21,    /* int32 union walk page ids, -1 = dummy (at the end)    */
  KPAGE_T_GROUP_NFULL = 22,   /* int32 [n_groups]: leading pages full in every member  */
  KPAGE_T_GROUP_VALID = 23,   /* uint32: member w of group i, word j at
                                 2 GROUP_WALK_PTR[i] + w len_i / 2 + j (page masks of
                                 the member's own selection, 0 for other pages)        */
  KPAGE_T_COUNT = 24
};

/*
 * Copy table `table_id` into host_buf.  With host_buf == NULL, *bytes receives
 * the size.  Otherwise *bytes must be at least that size (KPAGE_ERR_INVALID if
 * not) and receives the number of bytes written.  Backward tables trigger the
 * host part of the lazy backward build.
 */
kpage_status kpage_plan_export(kpage_plan_t *plan, int table_id, void *host_buf, size_t *bytes);

/* Release a plan and its device tables (NULL is ignored).  Synchronises the
 * device before freeing device memory that kernels may still read. */
void kpage_plan_destroy(kpage_plan_t *plan);

/*
 * Kernel timing.  With timing enabled on a plan, every kernel launch the plan
 * makes is bracketed by a pair of HIP events recorded on the launch stream.
 * kpage_timing_read() waits for those events, returns the summed milliseconds
 * and the number of launches of one kernel since the last read, and resets that
 * kernel's record.  Kernel ids below.  Disabled by default; enable = 1 adds two
 * event records per launch and nothing else.  enable = 2 is a profiling mode that
 * also splits the forward and dQ launches by route: the pass runs its full launch
 * twice, once with only the M128 x N128 items (timed under the pass's own id) and
 * once with only the M64 x N256 items and the empty-block cleanup (timed as
 * KPAGE_K_FWD_Q64 / KPAGE_K_BWD_DQ_Q64); each item keeps its launch position and
 * the other route's workgroups exit at once, so a route is timed without the
 * other one running beside it.
 */
enum {
  KPAGE_K_FWD = 0,       /* forward, both routes in one launch (M128 x N128 items, */
                         /* then M64 x N256 items and empty-block cleanup)         */
  KPAGE_K_FWD_EXACT = 1, /* forward re-run with online rescaling of the items the  */
                         /* fixed-maximum pass marked (one launch, both routes)    */
  KPAGE_K_BWD_PRE = 2,   /* reserved: rowsum(dO * O) and LSE * log2(e) per query   */
                         /* row run inside the dQ pass; no launch, reads 0         */
  KPAGE_K_BWD_ZERO = 3,  /* dK/dV pages outside every block footprint              */
  KPAGE_K_BWD_KV = 4,    /* K/V-owned pass: dK, dV                                  */
  KPAGE_K_BWD_DQ = 5,    /* Q-owned pass over the forward walks (both routes): dQ, */
                         /* and rowsum(dO * O), LSE * log2(e) of every query row   */
  KPAGE_K_BWD_REDUCE = 6,/* sum of the fp32 dK/dV partials of owners split over Q groups */
  KPAGE_K_FWD_Q64 = 7,   /* timing mode 2 only: the forward's M64 x N256 launch      */
  KPAGE_K_BWD_DQ_Q64 = 8,/* timing mode 2 only: the dQ pass's M64 x N256 launch      */
  KPAGE_K_COUNT = 9
};
kpage_status kpage_timing_enable(kpage_plan_t *plan, int enable);
kpage_status kpage_timing_read(kpage_plan_t *plan, int kernel_id, double *total_ms, int64_t *launches);

/* Message of the last non-OK status on this thread ("" if none). */
const char *kpage_last_error(void);

/*
 * Block selection prelude (the selector in front of KPage; KPage paper, sections 1
 * and 2: VSA-style dynamic selection over 3D video blocks, SSTA's top-k selection).
 * It produces the per-(b, h) sparse graph that kpage_plan_device() consumes, on the
 * GPU, so that selection, planning and attention need no host round trip.
 *
 * One block layout shared by all (b, h): Q block q holds rows [128 q, 128 q + c_q)
 * of Q, K block k rows [kv_offset_k, kv_offset_k + c_k) of K (kv_offset NULL: 128 k).
 * q_valid, kv_valid and kv_offset are DEVICE arrays with the rules of kpage_problem;
 * the kernels clamp rows to the tensors, and a layout that breaks the rules gives
 * unspecified lists (kpage_plan_device rejects it).  n_kv_blocks <= 4096;
 * batch * heads <= 65535.
 */
typedef struct {
  int32_t batch, heads, head_dim;  /* head_dim in {64, 128} */
  int32_t n_q_blocks, n_kv_blocks;
  int64_t seq_q, seq_kv;           /* seq_q = 128 * n_q_blocks */
  const int32_t *q_valid;          /* DEVICE [n_q_blocks] in [0, 128] */
  const int32_t *kv_valid;         /* DEVICE [n_kv_blocks] in [0, 128] */
  const int64_t *kv_offset;        /* DEVICE [n_kv_blocks] or NULL */
} kpage_select_layout;

/* Device workspace of kpage_select_topk(): the fp64 block means and block scores,
 * 8 * batch * heads * (head_dim * (n_q + n_kv) + n_q * n_kv) bytes plus a few KiB. */
kpage_status kpage_select_workspace_size(const kpage_select_layout *layout, size_t *bytes);

/*
 * Top-k block selection: for every (b, h) and query block q with c_q > 0,
 *   qbar_q, kbar_k = fp64 means of the valid rows (rows added in ascending order),
 *   s_qk = qbar_q . kbar_k (fp64 products added over ascending columns, each
 *          operation rounded on its own),
 *   K_q  = the min(top_k, n_live) key blocks with c_k > 0 of largest s_qk (ties to
 *          the lower block), in ascending block order; n_live = blocks with c_k > 0.
 * A query block with c_q = 0 selects nothing.  q, k: bf16 [batch, heads, seq, d]
 * contiguous, 16-byte aligned, DEVICE.  Outputs, DEVICE, caller-owned:
 *   q2k_ptr  int64 [batch * heads][n_q + 1], absolute offsets into q2k_idx
 *            (the per_head = 1 layout of kpage_problem, slot = b * heads + h);
 *   q2k_idx  int32, capacity batch * heads * n_q * top_k.
 * The fixed operation order makes the lists a function of the inputs alone.
 * Asynchronous on `stream`; workspace >= kpage_select_workspace_size(), 256-byte
 * aligned.  KPAGE_ERR_INVALID / UNSUPPORTED for bad arguments before any GPU work.
 */
kpage_status kpage_select_topk(const kpage_select_layout *layout, const void *q, const void *k, int32_t top_k,
                               int64_t *q2k_ptr, int32_t *q2k_idx, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * Cluster selection for independent Q/K partitions (SVG2-style: Q and K tokens
 * clustered and permuted so each cluster occupies contiguous blocks; KPage paper,
 * sections 3.4.1 and 4.6).  Per (b, h) slot g = b * heads + h, DEVICE arrays:
 *   q_centroids  fp32 [G][n_q_clusters][head_dim], kv_centroids fp32 [G][n_kv_clusters][head_dim]
 *   q_cluster_size, kv_cluster_size  int32 [G][n_clusters]: tokens per cluster
 *   q_block_cluster int32 [G][n_q_blocks], kv_block_cluster int32 [G][n_kv_blocks]:
 *                the cluster each block belongs to, -1 for none (out-of-range ids count as none)
 * n_kv_clusters <= 4096; batch * heads <= 65535.
 */
typedef struct {
  int32_t batch, heads, head_dim;  /* head_dim in {64, 128} */
  int32_t n_q_clusters, n_kv_clusters, n_q_blocks, n_kv_blocks;
  const float *q_centroids, *kv_centroids;
  const int32_t *q_cluster_size, *kv_cluster_size;
  const int32_t *q_block_cluster, *kv_block_cluster;
} kpage_select_clusters;

/* Device workspace of kpage_select_top_p(): fp64 centroids and cluster scores,
 * a keep mask and per-row counts, about 8 * G * (head_dim * (n_qc + n_kc) + n_qc * n_kc
 * + n_q_blocks) bytes. */
kpage_status kpage_select_top_p_workspace_size(const kpage_select_clusters *c, size_t *bytes);

/*
 * Top-p cluster selection: for every slot and Q cluster with tokens,
 *   s_k   = scale * (qcent . kcent_k) for every K cluster with tokens (fp64; the dot
 *           product over ascending columns, each operation rounded on its own),
 *   order = s descending, ties to the lower cluster; softmax p = exp(s - s_max) / sum,
 *   keep  = the shortest prefix of that order whose cumulative p reaches top_p (all of
 *           them if rounding never reaches it);
 * a Q block of that cluster selects every K block of a kept cluster, in ascending block
 * order; a Q block without a cluster selects nothing.  Outputs, DEVICE, caller-owned:
 *   q2k_ptr int64 [G][n_q_blocks + 1], absolute offsets into q2k_idx;
 *   q2k_idx int32, capacity G * n_q_blocks * n_kv_blocks.
 * 0 < top_p <= 1, scale > 0.  Asynchronous on `stream`; workspace 256-byte aligned.
 */
kpage_status kpage_select_top_p(const kpage_select_clusters *c, double top_p, double scale, int64_t *q2k_ptr,
                                int32_t *q2k_idx, void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KPAGE_H */
