// GPU-side construction of the page tables (KPage paper, sections 3.2.1-3.2.4, 3.3 and
// 3.4): the same walks, routes, validity words, queues, owners, reverse-Q lists,
// adjacency words and pair statistics as the host planner, built by kernels from a
// descriptor whose arrays live in device memory, so that a block selector running on
// the GPU feeds the planner without a round trip through host memory.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <functional>
#include <string>

#include "device.hpp"
#include "kpage.h"
#include "plan.hpp"

namespace kpage {

// The descriptor with device pointers (kv_offset may be NULL: block k at row 128 k).
struct DevProblem {
  int batch = 0, heads = 0, n_q = 0, n_kv = 0, slots = 0;
  int64_t seq_q = 0, seq_kv = 0;
  bool per_head = false;
  const int32_t *q_valid = nullptr, *kv_valid = nullptr, *q2k_idx = nullptr;
  const int64_t *kv_offset = nullptr, *q2k_ptr = nullptr;
  int64_t nnz = 0;  // entries of q2k_idx
  int64_t xcd_chunk = 0;  // launch-order chunk (launch_position)
};

// Device forward tables (every array allocated through the caller's allocator).
struct DevFwdTables {
  int32_t *route = nullptr, *nfull = nullptr, *unpadded = nullptr;  // [slots][n_q]
  int64_t *walk_ptr = nullptr;                                       // [slots][n_q + 1]
  int32_t *walk = nullptr;    // page ids, -1 = dummy (as exported)
  int32_t *pages = nullptr;   // the same with dummies pointed at the walk's first page
  uint32_t *valid = nullptr;  // two 16-bit page masks per word
  int32_t *q64_queue = nullptr, *q128_queue = nullptr;  // (bh, q) pairs, queue order
  FwdItem *items128 = nullptr, *items64 = nullptr;      // (bh, q) order per route; cleanup items last
  int32_t *order = nullptr;  // launch position -> item: i >= 0 M128 item i, ~j M64 item j
  int32_t *page_block = nullptr;  // [slots][seq_kv / 16] block whose footprint holds the page, -1 none
  int64_t walk_total = 0;
  int n_q64 = 0, n_q128 = 0, n_zero = 0;  // queue entries, empty query blocks
  PairStats stats;
  // Group items (plan.hpp, GroupTables), the same groups as the host planner's.  The
  // union walks follow the plan's walks in `pages` and their validity words follow the
  // plan's words in `valid`; g_walk / g_valid hold the exported copies.
  FwdGroup *groups = nullptr;                       // [n_groups], shared by a slot's (b, h)s
  int32_t *g_members = nullptr;                     // [n_groups][4] query blocks, -1 none
  int32_t *g_nfull = nullptr, *g_npages = nullptr;  // [n_groups]
  int32_t *g_walk = nullptr;                        // union walks, -1 dummies
  uint32_t *g_valid = nullptr;                      // member validity words
  std::vector<int64_t> g_group_ptr, g_walk_ptr;     // host copies: [slots + 1], [n_groups + 1]
  int64_t n_groups = 0, n_gitems = 0, n_members = 0;  // groups, group items over (b, h), member items
};

// Device backward tables (section 3.3), same contents and order as BwdTables.
struct DevBwdTables {
  int64_t *owner_ptr = nullptr;      // [slots + 1]
  int32_t *owners = nullptr;         // [n_own][8] page ids, -1 = empty slot
  uint32_t *kmask = nullptr;         // [n_own][8] row masks of the owner pages
  uint8_t *aligned = nullptr;        // [n_own]
  int64_t *revq_ptr = nullptr;       // [n_own * n_groups + 1], per (owner, group), owner-major
  int32_t *revq = nullptr;
  int64_t *qwalk_ptr = nullptr;      // [n_own * n_groups + 1]
  int32_t *qwalk = nullptr;          // Q page ids (8 q + j), -1 = dummy
  int32_t *qpages = nullptr;         // the same with dummies pointed at the walk's first page
  uint64_t *adj = nullptr;           // one word per 8-page step
  int32_t *bwd_queue = nullptr;      // (bh, owner within slot * n_groups + group) pairs, queue order
  BwdItem *items = nullptr;          // launch order (bh, owner, group), XCD-interleaved
  BwdReduce *reduce = nullptr;       // owners split over several items, (bh, owner) order
  int64_t *uncovered_ptr = nullptr;  // [slots + 1]
  int32_t *uncovered = nullptr;
  int64_t n_own = 0, revq_total = 0, qwalk_total = 0, n_items = 0, uncovered_total = 0;
  int n_groups = 1;
  int64_t n_partials = 0, n_reduce = 0;  // fp32 partial slots and reduce entries (Q groups)
  int max_uncovered = 0;
  uint64_t bwd_physical = 0, bwd_useful_check = 0;
};

using DevAlloc = std::function<void *(size_t)>;

// Builds the forward tables on `stream`.  Validates the descriptor on the device first
// (KPAGE_ERR_INVALID with `err` set on a malformed one).  Synchronises `stream` twice:
// once for the table sizes, once at the end for the queue lengths and pair counts; with
// `grouped`, twice more for the group items (candidate counts, then group sizes).
kpage_status build_forward_device(const DevProblem &p, int align64, int align128, bool grouped, hipStream_t stream,
                                  const DevAlloc &alloc, DevFwdTables *t, std::string *err);

// Builds the backward tables on `stream` from a descriptor already validated by
// build_forward_device and that call's page_block table, with Q groups of q_group Q
// blocks (0: one group) as the host planner builds them.  Synchronises `stream` twice
// (table sizes, then pair counts).
kpage_status build_backward_device(const DevProblem &p, const int32_t *page_block, int q_group, hipStream_t stream,
                                   const DevAlloc &alloc, DevBwdTables *t, std::string *err);

}  // namespace kpage
