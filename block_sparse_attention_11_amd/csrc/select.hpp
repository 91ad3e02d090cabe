// Block selection prelude: arguments, workspace layout and launcher.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace kpage {

constexpr int kSelectMaxKv = 4096;  // key blocks sorted in one workgroup's LDS

struct SelectArgs {
  const int32_t *q_valid, *kv_valid;  // device [n_q], [n_kv]
  const int64_t *kv_offset;           // device [n_kv] or NULL (block k at row 128 k)
  int64_t seq_q, seq_kv;
  int32_t n_q, n_kv, bh_count;
};

// byte offsets inside the caller's workspace
struct SelectWorkspace {
  size_t counts, pre, qbar, kbar, total;
};

inline SelectWorkspace select_workspace(const SelectArgs &a, int head_dim) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  SelectWorkspace w;
  w.counts = 0;
  w.pre = up(4 * sizeof(int32_t));
  w.qbar = w.pre + up(size_t(a.n_q) * sizeof(int32_t));
  w.kbar = w.qbar + up(size_t(a.bh_count) * a.n_q * head_dim * sizeof(double));
  w.total = w.kbar + up(size_t(a.bh_count) * a.n_kv * head_dim * sizeof(double));
  return w;
}

hipError_t launch_select(const SelectArgs &a, int head_dim, int32_t top_k, const void *q, const void *k, void *ws,
                         int64_t *q2k_ptr, int32_t *q2k_idx, hipStream_t stream);

}  // namespace kpage
