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
  size_t counts, pre, qbar, kbar, scores, total;
};

inline SelectWorkspace select_workspace(const SelectArgs &a, int head_dim) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  SelectWorkspace w;
  w.counts = 0;
  w.pre = up(4 * sizeof(int32_t));
  w.qbar = w.pre + up(size_t(a.n_q) * sizeof(int32_t));
  w.kbar = w.qbar + up(size_t(a.bh_count) * a.n_q * head_dim * sizeof(double));
  w.scores = w.kbar + up(size_t(a.bh_count) * a.n_kv * head_dim * sizeof(double));
  w.total = w.scores + up(size_t(a.bh_count) * a.n_q * a.n_kv * sizeof(double));
  return w;
}

hipError_t launch_select(const SelectArgs &a, int head_dim, int32_t top_k, const void *q, const void *k, void *ws,
                         int64_t *q2k_ptr, int32_t *q2k_idx, hipStream_t stream);

// Cluster top-p selection (independent Q/K partitions).
struct ClusterArgs {
  const float *q_cent, *k_cent;                    // device [BH][n_qc][d], [BH][n_kc][d]
  const int32_t *q_size, *k_size;                  // device [BH][n_qc], [BH][n_kc]
  const int32_t *q_block_cluster, *k_block_cluster;  // device [BH][n_q], [BH][n_kv], -1 none
  int32_t n_qc, n_kc, n_q, n_kv, bh_count;
  double top_p, scale;
};

struct ClusterWorkspace {
  size_t qc, kc, scores, keep, counts, total;
};

inline ClusterWorkspace cluster_workspace(const ClusterArgs &a, int head_dim) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t bh = size_t(a.bh_count);
  ClusterWorkspace w;
  w.qc = 0;
  w.kc = up(bh * a.n_qc * head_dim * sizeof(double));
  w.scores = w.kc + up(bh * a.n_kc * head_dim * sizeof(double));
  w.keep = w.scores + up(bh * a.n_qc * a.n_kc * sizeof(double));
  w.counts = w.keep + up(bh * a.n_qc * a.n_kc);
  w.total = w.counts + up(bh * a.n_q * sizeof(int64_t));
  return w;
}

hipError_t launch_select_top_p(const ClusterArgs &a, int head_dim, void *ws, int64_t *q2k_ptr, int32_t *q2k_idx,
                               hipStream_t stream);

}  // namespace kpage
