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
  int32_t pad;
};

struct FwdArgs {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const FwdItem *items;
  const int32_t *pages;     // walk entries; dummy slots point at a real page of the same walk
  const uint32_t *valid;    // two 16-bit row masks per word, indexed by walk position / 2
  int64_t seq_q, seq_kv;
  int32_t *redo;            // per workgroup of the launch: 1 when its item needs the exact rescaling pass
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
  int32_t aligned;     // 1: the owner is one block of 8 contiguous pages
  int32_t partial;     // -1: write dK/dV (bf16) directly; >= 0: fp32 partial slot of
                       // an owner split over several Q groups (summed by the reduce pass)
  int32_t pad;
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
  float *lse2;                // fp32 [BH, seq_q]: LSE * log2(e), 0 for rows without keys
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
  const int32_t *pages;
  const uint32_t *valid;
  int32_t n_fitems128, n_fitems64;
  int64_t seq_q, seq_kv;
  int32_t n_items, heads, n_q, per_head, bh_count;
  int32_t max_uncovered;      // largest count of uncovered K/V pages over the graph slots
  float scale, scale_log2;
};

// Optional per-launch timing: called right before and right after each kernel launch.
struct LaunchTimer {
  virtual void before(int kernel_id, hipStream_t stream) = 0;
  virtual void after(int kernel_id, hipStream_t stream) = 0;
  virtual ~LaunchTimer() = default;
};

// Forward over both routes in one launch (M128 items first, then M64 items), then the
// exact re-run launch; timer ids 0 and 1.  The redo flags hold n128 + n64 entries.
hipError_t launch_fwd(const FwdArgs &a128, const FwdArgs &a64, int head_dim, hipStream_t stream, LaunchTimer *timer);
hipError_t launch_bwd(const BwdArgs &a, int head_dim, hipStream_t stream, LaunchTimer *timer);

}  // namespace kpage
