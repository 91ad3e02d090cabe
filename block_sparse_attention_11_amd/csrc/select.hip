// Block selection in front of KPage (the selector whose graph KPage consumes; KPage
// paper, sections 1 and 2: VSA-style dynamic selection over 3D video blocks, SSTA's
// top-k selection).  For one block layout shared by all heads:
//   block means   fp64 mean of the valid rows of every Q and K block, rows added in
//                 ascending order (one thread per 8 columns of a block)
//   block scores  s_qk = qbar_q . kbar_k in fp64, products added over ascending
//                 columns, every operation rounded on its own (no fused multiply-add),
//                 64 x 64 tiles per workgroup into an fp64 score matrix
//   top-k         per query block with c_q > 0: the min(top_k, n_live) key blocks with
//                 c_k > 0 of largest score, ties to the lower block, in ascending order
// and, for independent Q/K partitions (SVG2-style clusters, sections 3.4.1 and 4.6):
//   top-p         per Q cluster with tokens: K clusters with tokens by scale * centroid
//                 score descending, the shortest prefix reaching top_p of the softmax;
//                 each Q block of the cluster selects the K blocks of those clusters
// The fixed operation order makes the selected sets a function of the inputs alone.
// Means and scores are HBM- and latency-bound side work (a few hundred microseconds on
// a 40-head 21x45x80 layout), next to the attention they feed.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "select.hpp"

namespace kpage {
namespace {

constexpr int kBlockRows = 128;
constexpr int kSelThreads = 256;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// valid rows of block b clamped to [0, 128] and to the tensor (a malformed layout is
// rejected later by the planner; these kernels only stay inside their buffers)
__device__ __forceinline__ int clamp_rows(int c, int64_t off, int64_t seq) {
  if (c < 0 || off < 0 || off >= seq) return 0;
  c = c > kBlockRows ? kBlockRows : c;
  return (int)((int64_t)c < seq - off ? (int64_t)c : seq - off);
}

__device__ __forceinline__ int64_t kv_row0(const SelectArgs &a, int k) {
  return a.kv_offset ? a.kv_offset[k] : (int64_t)kBlockRows * k;
}

// Means of one tensor: 8 columns per thread, D / 8 threads per block, 256 / (D / 8)
// blocks per workgroup; grid (block groups, B * H).  out: [BH][n][D] or, transposed,
// [BH][D][n] (the key side, read column by column by the score loop).
template <int D, bool KEYS>
__global__ __launch_bounds__(kSelThreads) void k_sel_means(SelectArgs a, const __bf16 *x, double *out) {
  constexpr int CPB = D / 8;
  constexpr int BPW = kSelThreads / CPB;
  const int n = KEYS ? a.n_kv : a.n_q;
  const int64_t seq = KEYS ? a.seq_kv : a.seq_q;
  const int blk = blockIdx.x * BPW + threadIdx.x / CPB;
  const int col = (threadIdx.x % CPB) * 8;
  const int64_t bh = blockIdx.y;
  if (blk >= n) return;
  const int64_t off = KEYS ? kv_row0(a, blk) : (int64_t)kBlockRows * blk;
  const int c = clamp_rows(KEYS ? a.kv_valid[blk] : a.q_valid[blk], off, seq);
  const bf16x8_t *src = (const bf16x8_t *)(x + (bh * seq + off) * D + col);
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 4
  for (int r = 0; r < c; ++r) {
    const bf16x8_t v = src[(int64_t)r * (D / 8)];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = acc[i] + (double)(float)v[i];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double m = c ? acc[i] / (double)c : 0.0;
    if (KEYS) out[(bh * D + col + i) * n + blk] = m;
    else out[(bh * n + blk) * D + col + i] = m;
  }
}

// Per-layout counts, one workgroup: live key blocks, kk = min(top_k, n_live), and the
// number of valid query blocks before each query block.
__global__ __launch_bounds__(1024) void k_sel_counts(SelectArgs a, int32_t top_k, int32_t *pre, int32_t *counts) {
  __shared__ int32_t lds[1024];
  __shared__ int32_t live;
  if (threadIdx.x == 0) live = 0;
  __syncthreads();
  int mine = 0;
  for (int k = threadIdx.x; k < a.n_kv; k += 1024) mine += clamp_rows(a.kv_valid[k], kv_row0(a, k), a.seq_kv) > 0;
  atomicAdd(&live, mine);
  int carry = 0;
  for (int base = 0; base < a.n_q; base += 1024) {
    const int q = base + threadIdx.x;
    const int v = q < a.n_q && clamp_rows(a.q_valid[q], (int64_t)kBlockRows * q, a.seq_q) > 0 ? 1 : 0;
    lds[threadIdx.x] = v;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int t = threadIdx.x >= o ? lds[threadIdx.x - o] : 0;
      __syncthreads();
      lds[threadIdx.x] += t;
      __syncthreads();
    }
    if (q < a.n_q) pre[q] = carry + lds[threadIdx.x] - v;
    carry += lds[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    counts[0] = live;
    counts[1] = live < top_k ? live : top_k;  // kk
    counts[2] = carry;                        // valid query blocks
  }
}

// order-preserving map of a double onto uint64 (+0 and -0 both map to +0's image)
__device__ __forceinline__ uint64_t ordered_bits(double s) {
  s = s + 0.0;
  const uint64_t u = __builtin_bit_cast(uint64_t, s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Block scores s[bh][q][k], 64 x 64 per workgroup, 4 x 4 per thread, the columns staged
// through LDS 16 at a time.  Every score is the fixed-order sum over ascending columns
// with each product and each sum rounded on its own (no fused multiply-add), so the
// tiling only decides who computes it.
constexpr int kScoreTile = 64, kScoreCols = 16;

template <int D>
__global__ __launch_bounds__(kSelThreads) void k_sel_scores(SelectArgs a, const double *qbar, const double *kbar_t,
                                                            double *scores) {
#pragma clang fp contract(off)
  __shared__ double qs[kScoreCols][kScoreTile + 1];
  __shared__ double ks[kScoreCols][kScoreTile + 1];
  const int64_t bh = blockIdx.z;
  const int q0 = blockIdx.y * kScoreTile, k0 = blockIdx.x * kScoreTile;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  double acc[4][4] = {};
  for (int j0 = 0; j0 < D; j0 += kScoreCols) {
    for (int e = threadIdx.x; e < kScoreCols * kScoreTile; e += kSelThreads) {
      const int jq = e % kScoreCols, rq = e / kScoreCols;  // q tile: consecutive threads along columns
      const int q = q0 + rq;
      qs[jq][rq] = q < a.n_q ? qbar[(bh * a.n_q + q) * D + j0 + jq] : 0.0;
      const int rk = e % kScoreTile, jk = e / kScoreTile;  // k tile: consecutive threads along blocks
      const int k = k0 + rk;
      ks[jk][rk] = k < a.n_kv ? kbar_t[(bh * D + j0 + jk) * (int64_t)a.n_kv + k] : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int j = 0; j < kScoreCols; ++j) {
      double qv[4], kv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qv[i] = qs[j][4 * ty + i];
        kv[i] = ks[j][4 * tx + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int l = 0; l < 4; ++l) acc[i][l] = acc[i][l] + qv[i] * kv[l];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = q0 + 4 * ty + i;
    if (q >= a.n_q) continue;
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const int k = k0 + 4 * tx + l;
      if (k < a.n_kv) scores[(bh * a.n_q + q) * (int64_t)a.n_kv + k] = acc[i][l];
    }
  }
}

// Ascending bitonic sort of np (a power of two) (key, id) pairs in LDS by the whole
// workgroup; pairs compare by key, then id.  Ends with a barrier.
__device__ void bitonic_sort(uint64_t *key, int32_t *id, int np) {
  for (int size = 2; size <= np; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < np / 2; i += kSelThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t kl = key[lo], kh = key[hi];
        const int il = id[lo], ih = id[hi];
        const bool greater = kl > kh || (kl == kh && il > ih);
        if (greater == up) {
          key[lo] = kh;
          key[hi] = kl;
          id[lo] = ih;
          id[hi] = il;
        }
      }
      __syncthreads();
    }
  }
}

// One workgroup per (query block, b * H + h): its row of scores, a bitonic sort on
// (score descending, block ascending) in LDS, the first kk blocks written in ascending
// block order.  Also writes the row's CSR offset.
__global__ __launch_bounds__(kSelThreads) void k_sel_topk(SelectArgs a, const double *scores, const int32_t *pre,
                                                          const int32_t *counts, int64_t *q2k_ptr, int32_t *q2k_idx,
                                                          int np) {
  // LDS sized for this layout (np = smallest power of two >= max(n_kv, 2)), so that
  // small layouts keep many workgroups per CU
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  uint64_t *key = (uint64_t *)lds_raw;
  int32_t *id = (int32_t *)(lds_raw + 8 * np);
  int32_t *scan = (int32_t *)(lds_raw + 12 * np);
  uint8_t *pick = (uint8_t *)(lds_raw + 12 * np + 4 * kSelThreads);
  const int q = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int kk = counts[1], n_vq = counts[2];
  const bool active = clamp_rows(a.q_valid[q], (int64_t)kBlockRows * q, a.seq_q) > 0 && kk > 0;
  const int64_t base = (bh * n_vq + pre[q]) * (int64_t)kk;
  if (threadIdx.x == 0) {
    q2k_ptr[bh * (a.n_q + 1) + q] = base;
    if (q == a.n_q - 1) q2k_ptr[bh * (a.n_q + 1) + a.n_q] = base + (active ? kk : 0);
  }
  if (!active) return;
  const double *srow = scores + (bh * a.n_q + q) * (int64_t)a.n_kv;
  for (int k = threadIdx.x; k < np; k += kSelThreads) {
    uint64_t kv = ~0ull;
    if (k < a.n_kv && clamp_rows(a.kv_valid[k], kv_row0(a, k), a.seq_kv) > 0) kv = ~ordered_bits(srow[k]);
    key[k] = kv;
    id[k] = k;
    if (k < a.n_kv) pick[k] = 0;
  }
  __syncthreads();
  bitonic_sort(key, id, np);
  for (int i = threadIdx.x; i < kk; i += kSelThreads) pick[id[i]] = 1;
  __syncthreads();
  // ascending compaction: thread t scans a contiguous range of blocks
  const int per = (a.n_kv + kSelThreads - 1) / kSelThreads;
  const int k0 = threadIdx.x * per, k1 = min(a.n_kv, k0 + per);
  int cnt = 0;
  for (int k = k0; k < k1; ++k) cnt += pick[k];
  scan[threadIdx.x] = cnt;
  __syncthreads();
  for (int o = 1; o < kSelThreads; o <<= 1) {
    const int t = threadIdx.x >= o ? scan[threadIdx.x - o] : 0;
    __syncthreads();
    scan[threadIdx.x] += t;
    __syncthreads();
  }
  int pos = scan[threadIdx.x] - cnt;
  for (int k = k0; k < k1; ++k)
    if (pick[k]) q2k_idx[base + pos++] = k;
}

// ---- cluster top-p selection (independent Q/K partitions) ----

// fp32 centroids widened to fp64: Q row-major [BH][n_qc][D], K transposed [BH][D][n_kc]
template <int D>
__global__ __launch_bounds__(kSelThreads) void k_cent_prep(ClusterArgs a, double *qc, double *kc_t) {
  const int64_t bh = blockIdx.y;
  const int64_t e = (int64_t)blockIdx.x * kSelThreads + threadIdx.x;
  if (e < (int64_t)a.n_qc * D) qc[bh * a.n_qc * D + e] = (double)a.q_cent[bh * a.n_qc * D + e];
  if (e < (int64_t)a.n_kc * D) {
    const int64_t k = e / D, j = e % D;
    kc_t[(bh * D + j) * a.n_kc + k] = (double)a.k_cent[bh * a.n_kc * D + e];
  }
}

__device__ __forceinline__ double from_ordered(uint64_t o) {
  const uint64_t u = (o >> 63) ? (o & 0x7FFFFFFFFFFFFFFFull) : ~o;
  return __builtin_bit_cast(double, u);
}

// One workgroup per (Q cluster, b * H + h): scale * scores of the K clusters with tokens
// sorted descending (ties to the lower cluster), softmax in sorted order, the shortest
// prefix whose cumulative probability reaches top_p marked in keep[bh][c][k].
__global__ __launch_bounds__(kSelThreads) void k_sel_topp(ClusterArgs a, const double *scores, uint8_t *keep, int np) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  uint64_t *key = (uint64_t *)lds_raw;
  int32_t *id = (int32_t *)(lds_raw + 8 * np);
  __shared__ int n_live, m_keep;
  __shared__ double x0;
  const int c = blockIdx.x;
  const int64_t bh = blockIdx.y;
  uint8_t *row = keep + (bh * a.n_qc + c) * (int64_t)a.n_kc;
  for (int k = threadIdx.x; k < a.n_kc; k += kSelThreads) row[k] = 0;
  if (a.q_size[bh * a.n_qc + c] <= 0) return;
  if (threadIdx.x == 0) n_live = 0;
  __syncthreads();
  const double *srow = scores + (bh * a.n_qc + c) * (int64_t)a.n_kc;
  int mine = 0;
  for (int k = threadIdx.x; k < np; k += kSelThreads) {
    uint64_t kv = ~0ull;
    if (k < a.n_kc && a.k_size[bh * a.n_kc + k] > 0) {
      kv = ~ordered_bits(a.scale * srow[k]);
      ++mine;
    }
    key[k] = kv;
    id[k] = k;
  }
  atomicAdd(&n_live, mine);
  __syncthreads();
  bitonic_sort(key, id, np);
  const int nl = n_live;
  if (nl == 0) return;
  if (threadIdx.x == 0) x0 = from_ordered(~key[0]);
  __syncthreads();
  for (int i = threadIdx.x; i < nl; i += kSelThreads)  // exp(x_i - x_max), in place of the key
    key[i] = __builtin_bit_cast(uint64_t, exp(from_ordered(~key[i]) - x0));
  __syncthreads();
  if (threadIdx.x == 0) {
    const double *e = (const double *)key;
    double total = 0.0;
    for (int i = 0; i < nl; ++i) total += e[i];
    double cum = 0.0;
    int m = nl;
    for (int i = 0; i < nl; ++i) {
      cum += e[i] / total;
      if (cum >= a.top_p) {
        m = i + 1;
        break;
      }
    }
    m_keep = m;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < m_keep; i += kSelThreads) row[id[i]] = 1;
}

__device__ __forceinline__ bool block_kept(const ClusterArgs &a, const uint8_t *keep, int64_t bh, int c, int k) {
  const int kc = a.k_block_cluster[bh * a.n_kv + k];
  return kc >= 0 && kc < a.n_kc && keep[(bh * a.n_qc + c) * (int64_t)a.n_kc + kc];
}

__device__ __forceinline__ int q_cluster(const ClusterArgs &a, int64_t bh, int q) {
  const int c = a.q_block_cluster[bh * a.n_q + q];
  return c >= 0 && c < a.n_qc ? c : -1;
}

// per (bh, Q block): number of selected K blocks
__global__ __launch_bounds__(kSelThreads) void k_topp_count(ClusterArgs a, const uint8_t *keep, int64_t *counts) {
  const int64_t i = (int64_t)blockIdx.x * kSelThreads + threadIdx.x;
  if (i >= (int64_t)a.bh_count * a.n_q) return;
  const int64_t bh = i / a.n_q;
  const int c = q_cluster(a, bh, int(i % a.n_q));
  int64_t n = 0;
  if (c >= 0)
    for (int k = 0; k < a.n_kv; ++k) n += block_kept(a, keep, bh, c, k);
  counts[i] = n;
}

// CSR offsets over all (bh, Q block) rows, one workgroup: q2k_ptr[bh][q], absolute
__global__ __launch_bounds__(1024) void k_topp_ptr(ClusterArgs a, const int64_t *counts, int64_t *q2k_ptr) {
  __shared__ int64_t lds[1024];
  const int64_t n = (int64_t)a.bh_count * a.n_q;
  int64_t carry = 0;
  for (int64_t base = 0; base < n; base += 1024) {
    const int64_t i = base + threadIdx.x;
    const int64_t v = i < n ? counts[i] : 0;
    lds[threadIdx.x] = v;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int64_t t = threadIdx.x >= o ? lds[threadIdx.x - o] : 0;
      __syncthreads();
      lds[threadIdx.x] += t;
      __syncthreads();
    }
    if (i < n) {
      const int64_t bh = i / a.n_q, q = i % a.n_q;
      q2k_ptr[bh * (a.n_q + 1) + q] = carry + lds[threadIdx.x] - v;
      if (q == a.n_q - 1) q2k_ptr[bh * (a.n_q + 1) + a.n_q] = carry + lds[threadIdx.x];
    }
    carry += lds[1023];
    __syncthreads();
  }
}

// per (bh, Q block): its selected K blocks in ascending order
__global__ __launch_bounds__(kSelThreads) void k_topp_fill(ClusterArgs a, const uint8_t *keep, const int64_t *q2k_ptr,
                                                           int32_t *q2k_idx) {
  const int64_t i = (int64_t)blockIdx.x * kSelThreads + threadIdx.x;
  if (i >= (int64_t)a.bh_count * a.n_q) return;
  const int64_t bh = i / a.n_q;
  const int q = int(i % a.n_q);
  const int c = q_cluster(a, bh, q);
  if (c < 0) return;
  int64_t pos = q2k_ptr[bh * (a.n_q + 1) + q];
  for (int k = 0; k < a.n_kv; ++k)
    if (block_kept(a, keep, bh, c, k)) q2k_idx[pos++] = k;
}

template <int D>
hipError_t launch_top_p_d(const ClusterArgs &a, double *qc, double *kc_t, double *scores, uint8_t *keep,
                          int64_t *counts, int64_t *q2k_ptr, int32_t *q2k_idx, hipStream_t st) {
  const unsigned bh = (unsigned)a.bh_count;
  const int64_t prep = (int64_t)(a.n_qc > a.n_kc ? a.n_qc : a.n_kc) * D;
  hipLaunchKernelGGL(k_cent_prep<D>, dim3((unsigned)((prep + kSelThreads - 1) / kSelThreads), bh), dim3(kSelThreads), 0,
                     st, a, qc, kc_t);
  SelectArgs sa{};
  sa.n_q = a.n_qc;
  sa.n_kv = a.n_kc;
  sa.bh_count = a.bh_count;
  hipLaunchKernelGGL(k_sel_scores<D>,
                     dim3((a.n_kc + kScoreTile - 1) / kScoreTile, (a.n_qc + kScoreTile - 1) / kScoreTile, bh),
                     dim3(kSelThreads), 0, st, sa, qc, kc_t, scores);
  int np = 2;
  while (np < a.n_kc) np <<= 1;
  hipLaunchKernelGGL(k_sel_topp, dim3(a.n_qc, bh), dim3(kSelThreads), size_t(12) * np, st, a, scores, keep, np);
  const int64_t rows = (int64_t)a.bh_count * a.n_q;
  const unsigned grid = (unsigned)((rows + kSelThreads - 1) / kSelThreads);
  hipLaunchKernelGGL(k_topp_count, dim3(grid), dim3(kSelThreads), 0, st, a, keep, counts);
  hipLaunchKernelGGL(k_topp_ptr, dim3(1), dim3(1024), 0, st, a, counts, q2k_ptr);
  hipLaunchKernelGGL(k_topp_fill, dim3(grid), dim3(kSelThreads), 0, st, a, keep, q2k_ptr, q2k_idx);
  return hipGetLastError();
}

template <int D>
hipError_t launch_select_d(const SelectArgs &a, int32_t top_k, const void *q, const void *k, double *qbar,
                           double *kbar_t, double *scores, int32_t *pre, int32_t *counts, int64_t *q2k_ptr,
                           int32_t *q2k_idx, hipStream_t st) {
  constexpr int BPW = kSelThreads / (D / 8);
  const unsigned bh = (unsigned)a.bh_count;
  hipLaunchKernelGGL(k_sel_counts, dim3(1), dim3(1024), 0, st, a, top_k, pre, counts);
  hipLaunchKernelGGL((k_sel_means<D, false>), dim3((a.n_q + BPW - 1) / BPW, bh), dim3(kSelThreads), 0, st, a,
                     (const __bf16 *)q, qbar);
  hipLaunchKernelGGL((k_sel_means<D, true>), dim3((a.n_kv + BPW - 1) / BPW, bh), dim3(kSelThreads), 0, st, a,
                     (const __bf16 *)k, kbar_t);
  hipLaunchKernelGGL(k_sel_scores<D>,
                     dim3((a.n_kv + kScoreTile - 1) / kScoreTile, (a.n_q + kScoreTile - 1) / kScoreTile, bh),
                     dim3(kSelThreads), 0, st, a, qbar, kbar_t, scores);
  int np = 2;
  while (np < a.n_kv) np <<= 1;
  const size_t lds = size_t(12) * np + 4 * kSelThreads + size_t(a.n_kv + 15) / 16 * 16;
  hipLaunchKernelGGL(k_sel_topk, dim3(a.n_q, bh), dim3(kSelThreads), lds, st, a, scores, pre, counts, q2k_ptr,
                     q2k_idx, np);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select_top_p(const ClusterArgs &a, int head_dim, void *ws, int64_t *q2k_ptr, int32_t *q2k_idx,
                               hipStream_t stream) {
  const ClusterWorkspace w = cluster_workspace(a, head_dim);
  char *base = static_cast<char *>(ws);
  double *qc = reinterpret_cast<double *>(base + w.qc);
  double *kc_t = reinterpret_cast<double *>(base + w.kc);
  double *scores = reinterpret_cast<double *>(base + w.scores);
  uint8_t *keep = reinterpret_cast<uint8_t *>(base + w.keep);
  int64_t *counts = reinterpret_cast<int64_t *>(base + w.counts);
  if (head_dim == 128) return launch_top_p_d<128>(a, qc, kc_t, scores, keep, counts, q2k_ptr, q2k_idx, stream);
  if (head_dim == 64) return launch_top_p_d<64>(a, qc, kc_t, scores, keep, counts, q2k_ptr, q2k_idx, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_select(const SelectArgs &a, int head_dim, int32_t top_k, const void *q, const void *k, void *ws,
                         int64_t *q2k_ptr, int32_t *q2k_idx, hipStream_t stream) {
  const SelectWorkspace w = select_workspace(a, head_dim);
  char *base = static_cast<char *>(ws);
  int32_t *counts = reinterpret_cast<int32_t *>(base + w.counts);
  int32_t *pre = reinterpret_cast<int32_t *>(base + w.pre);
  double *qbar = reinterpret_cast<double *>(base + w.qbar);
  double *kbar_t = reinterpret_cast<double *>(base + w.kbar);
  double *scores = reinterpret_cast<double *>(base + w.scores);
  if (head_dim == 128)
    return launch_select_d<128>(a, top_k, q, k, qbar, kbar_t, scores, pre, counts, q2k_ptr, q2k_idx, stream);
  if (head_dim == 64)
    return launch_select_d<64>(a, top_k, q, k, qbar, kbar_t, scores, pre, counts, q2k_ptr, q2k_idx, stream);
  return hipErrorInvalidValue;
}

}  // namespace kpage
