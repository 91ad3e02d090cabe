// GPU-side construction of the forward page tables (KPage paper, sections 3.2.1-3.2.4
// and 3.4): the same walks, routes, validity words, queues and pair statistics as the
// host planner, built by kernels from a descriptor whose arrays live in device memory,
// so that a block selector running on the GPU feeds the planner without a round trip
// through host memory.
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
};

// Device forward tables (every array allocated through the caller's allocator).
struct DevFwdTables {
  int32_t *route = nullptr, *nfull = nullptr, *unpadded = nullptr;  // [slots][n_q]
  int64_t *walk_ptr = nullptr;                                       // [slots][n_q + 1]
  int32_t *walk = nullptr;    // page ids, -1 = dummy (as exported)
  int32_t *pages = nullptr;   // the same with dummies pointed at the walk's first page
  uint32_t *valid = nullptr;  // two 16-bit page masks per word
  int32_t *q64_queue = nullptr, *q128_queue = nullptr;  // (bh, q) pairs, queue order
  FwdItem *items128 = nullptr, *items64 = nullptr;      // launch order (see api.hip)
  int32_t *redo = nullptr;
  int64_t walk_total = 0;
  int n_q64 = 0, n_q128 = 0, n_zero = 0;  // queue entries, empty query blocks
  PairStats stats;
};

using DevAlloc = std::function<void *(size_t)>;

// Builds the forward tables on `stream`.  Validates the descriptor on the device first
// (KPAGE_ERR_INVALID with `err` set on a malformed one).  Synchronises `stream` twice:
// once for the table sizes, once at the end for the queue lengths and pair counts.
kpage_status build_forward_device(const DevProblem &p, int align64, int align128, hipStream_t stream,
                                  const DevAlloc &alloc, DevFwdTables *t, std::string *err);

}  // namespace kpage
