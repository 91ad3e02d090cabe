// Device-side work descriptors and kernel launchers shared by the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace kpage {

// One forward work item: a query block of one (batch, head) and its page walk.
struct FwdItem {
  int64_t walk_off;  // first entry of the walk in the device page table (multiple of the step size)
  int32_t bh;        // b * heads + h
  int32_t q;         // query block
  int32_t walk_len;  // pages, a multiple of the pages per step (0: nothing selected)
  int32_t n_full;    // pages of the fully valid prefix
  int32_t c_q;       // valid query rows (0 only for cleanup items of empty blocks)
  int32_t n_pages;   // real pages of the walk (the rest are dummies, which the kernels skip
                     // past the last 4-page tile holding a real page)
};

// A group item: up to four query blocks of one (batch, head), each with at most 32 valid
// rows, run as one M128 x N128 work item over the union of their page walks.  Wave w
// holds the rows of member w and masks the pages of the union that its own block did not
// select; the item writes the 128 output rows of every member block.  Group items are
// M128 items whose q field is ~(index into the group table).
struct FwdGroup {
  int32_t q[4];        // member block of wave w (-1: no member, the wave computes nothing)
  int32_t c_q[4];      // its valid rows (1..32; 0 without a member)
  int64_t valid_off;   // wave w's validity words start at valid_off + w * (walk_len / 2)
  int64_t pad;
};

// The 32 query rows of query group qg (one wave's rows in the M128 route) of a work item.
struct WaveRows {
  int32_t block;       // query block holding them (never -1: an absent member names member 0)
  int32_t row0;        // first of them inside the block
  int32_t rows;        // how many are valid (0: the wave computes nothing)
  int64_t valid_off;   // first validity word of this wave's walk
};

__device__ __forceinline__ WaveRows wave_rows(const FwdItem &it, const FwdGroup *groups, int qg) {
  WaveRows r;
  if (it.q >= 0) {
    const int left = it.c_q - 32 * qg;
    r.block = it.q;
    r.row0 = 32 * qg;
    r.rows = left < 0 ? 0 : (left > 32 ? 32 : left);
    r.valid_off = it.walk_off >> 1;
  } else {
    const FwdGroup &gr = groups[~it.q];
    const int32_t b = gr.q[qg];
    r.block = b >= 0 ? b : gr.q[0];
    r.row0 = 0;
    r.rows = b >= 0 ? gr.c_q[qg] : 0;
    r.valid_off = gr.valid_off + int64_t(qg) * (it.walk_len / 2);
  }
  return r;
}

// First output row of a work item (the row that carries the forward's re-run mark).
__device__ __forceinline__ int32_t item_block0(const FwdItem &it, const FwdGroup *groups) {
  return it.q >= 0 ? it.q : groups[~it.q].q[0];
}

struct FwdArgs {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const FwdItem *items;
  const FwdGroup *groups;   // member tables of the group items (NULL when there are none)
  // launch order of a launch holding both routes: workgroup b runs M128 item order[b]
  // when order[b] >= 0, else M64 item ~order[b]; NULL: the M128 items, then the M64 items
  const int32_t *order;
  int32_t route_only;       // timing mode: 128 or 64 runs only that route's items (the other
                            // route's workgroups exit at once); 0 runs both
  const int32_t *pages;     // walk entries; dummy slots point at a real page of the same walk
  const uint32_t *valid;    // two 16-bit row masks per word, indexed by walk position / 2
  int64_t seq_q, seq_kv;
  int32_t n_items;
  float scale;              // softmax scale
  float scale_log2;         // softmax scale * log2(e)
};

// One backward work item: a K/V owner of one (batch, head) and its Q-page steps.
struct BwdItem {
  int64_t qwalk_off;   // first Q page entry (multiple of 8)
  int32_t bh;
  int32_t owner;       // global owner index (row of the owner table)
  int32_t n_steps;
  int32_t partial;     // -1: write dK/dV (bf16) directly; >= 0: fp32 partial slot of
                       // an owner split over several Q groups (summed by the reduce pass)
  int32_t pad[2];
};

// One owner whose Q groups were split over `count` work items: partial slots
// [part0, part0 + count) are summed in group order and written as bf16.
struct BwdReduce {
  int32_t bh, owner, part0, count;
};

struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  const int32_t *q_valid;     // [slots][n_q] valid rows per query block (rows past them are padding)
  float *lse2;                // fp32 [BH, seq_q]: LSE * log2(e); +inf for rows without keys and rows
                              // past c_q, so that exp2(x - lse2) = 0 there
  float *delta;               // fp32 [BH, seq_q]: rowsum(dO * O)
  // K/V-owned pass (dK, dV)
  const BwdItem *items;
  const int32_t *owners;      // [n_own][8] page ids, -1 empty
  const uint32_t *owner_kmask;// [n_own][8] 16-bit row masks of the owner pages (0 for empty slots)
  const int32_t *qpages;      // Q-page walk entries, dummy slots point at a real page
  const uint64_t *adj;        // adjacency word per step
  const int32_t *uncovered;   // K/V pages outside every footprint, per slot
  const int64_t *uncovered_ptr;
  float *part;                // fp32 [n_partials][2][128][d]: unscaled dK, then dV, per owner row
  const BwdReduce *reduce;
  int32_t n_reduce;
  // Q-owned pass (dQ): the forward work items and page walks of both routes
  const FwdItem *fitems128, *fitems64;
  const FwdGroup *fgroups;    // as FwdArgs::groups
  const int32_t *forder;      // launch order of the dQ pass, as FwdArgs::order
  int32_t froute_only;        // as FwdArgs::route_only
  const int32_t *pages;
  const uint32_t *valid;
  int32_t n_fitems128, n_fitems64;
  int64_t seq_q, seq_kv;
  int32_t n_items, heads, n_q, per_head, bh_count;
  int32_t max_uncovered;      // largest count of uncovered K/V pages over the graph slots
  float scale, scale_log2;
};

// Launch order for MI355X's 8 XCDs.  The dispatcher hands workgroup i to XCD i % 8, and
// each XCD has its own 4 MB L2.  Entry p of a work list (head-major, spatially ordered)
// goes to launch position launch_position(p, n, chunk), a bijection onto [0, n) in which
// XCD x receives exactly the positions with p % 8 == x:
//  - chunk <= 0: XCD x takes the x-th contiguous eighth of the list, so each XCD works
//    through its own run of heads and its workgroups gather neighbouring blocks' pages
//    from its L2; 8 heads (one per XCD) are live at a time.
//  - chunk > 0: the list is dealt to the XCDs in chunks of `chunk` consecutive entries
//    (the entries after the last full round of 8 chunks are split into 8 contiguous
//    shares), so all XCDs stay within the same one or two heads.
// The first keeps more L2 locality, the second keeps the live K/V small enough for the
// memory-side cache when 8 heads of it would not fit (xcd_chunk_for).
constexpr int kXcds = 8;
constexpr int64_t kMemCacheBytes = int64_t(256) << 20;  // MI355X Infinity Cache

__host__ __device__ inline int64_t launch_position(int64_t p, int64_t n, int64_t chunk) {
  const int64_t round = kXcds * chunk;
  const int64_t full = chunk > 0 ? n / round : 0;
  if (p < full * round) {
    const int64_t k = p / chunk, o = p % chunk;
    return ((k / kXcds) * chunk + o) * kXcds + k % kXcds;
  }
  const int64_t m = n - full * round, q = p - full * round;
  const int64_t per = m / kXcds, extra = m % kXcds;
  int64_t x, j;
  if (q < extra * (per + 1)) {
    x = q / (per + 1);
    j = q % (per + 1);
  } else {
    x = extra + (q - extra * (per + 1)) / per;
    j = (q - extra * (per + 1)) % per;
  }
  return (full * chunk + j) * kXcds + x;
}

// Entries at the end of each XCD's backward launch sequence that run longest-first
// (5%, at most kMaxBwdTail): owners differ in step count by up to 4x, and an XCD that
// ends on a long one idles the rest of its CUs.
constexpr int64_t kMaxBwdTail = 1024;
__host__ __device__ inline int64_t bwd_tail_len(int64_t count) {
  const int64_t t = count / 20;
  return t < kMaxBwdTail ? t : kMaxBwdTail;
}

// Entries at the end of each XCD's forward (and dQ) launch sequence that run
// longest-first: two per workgroup slot of an XCD (64 slots), so that the XCD's last
// round does not end on a long item.  Cost of an item: its 4-page stages, weighted 3
// for the M128 route and 2 for the M64 route (a measured per-stage time ratio of about
// 2 : 3); ties keep their launch order.
constexpr int kFwdTail = 128;
__host__ __device__ inline int32_t fwd_tail_cost(int route, int n_pages) {
  return (route == 128 ? 3 : 2) * ((n_pages + 3) / 4);
}

// Chunk length of a plan's launch order: whole-head runs per XCD (0) while one head's
// pair of gathered tensors (K and V, or Q and dO) times 8 fits the memory-side cache,
// else 64 entries (one XCD's two workgroups per CU).
inline int64_t xcd_chunk_for(int64_t seq_q, int64_t seq_kv, int head_dim) {
  const int64_t rows = seq_q > seq_kv ? seq_q : seq_kv;
  const int64_t head_bytes = rows * head_dim * 2 * 2;
  return kXcds * head_bytes > kMemCacheBytes ? 64 : 0;
}

// Optional per-launch timing: called right before and right after each kernel launch.
struct LaunchTimer {
  virtual void before(int kernel_id, hipStream_t stream) = 0;
  virtual void after(int kernel_id, hipStream_t stream) = 0;
  // profiling mode: the forward and dQ passes launch their two routes separately
  // (M128 items under the pass's own id, M64 items under KPAGE_K_FWD_Q64 / KPAGE_K_BWD_DQ_Q64)
  virtual bool split_routes() const { return false; }
  virtual ~LaunchTimer() = default;
};

// Forward over both routes in one launch (M128 items first, then M64 items), then the
// exact re-run launch over the items the first marked in their LSE; timer ids 0 and 1.
hipError_t launch_fwd(const FwdArgs &a128, const FwdArgs &a64, int head_dim, hipStream_t stream, LaunchTimer *timer);
hipError_t launch_bwd(const BwdArgs &a, int head_dim, hipStream_t stream, LaunchTimer *timer);

}  // namespace kpage
