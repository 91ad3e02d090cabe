// Block selection in front of KPage (the selector whose graph KPage consumes; KPage
// paper, sections 1 and 2: VSA-style dynamic selection over 3D video blocks, SSTA's
// top-k selection).  For one block layout shared by all heads:
//   block means   fp64 mean of the valid rows of every Q and K block, rows added in
//                 ascending order (one thread per 8 columns of a block)
//   block scores  s_qk = qbar_q . kbar_k in fp64, products added over ascending
//                 columns, every operation rounded on its own (no fused multiply-add)
//   top-k         per query block with c_q > 0: the min(top_k, n_live) key blocks with
//                 c_k > 0 of largest score, ties to the lower block, in ascending order
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

// The fixed-order dot product: every product and every sum rounded separately.
template <int D>
__device__ __forceinline__ double dot_in_order(const double *qs, const double *kcol, int64_t stride) {
#pragma clang fp contract(off)
  double s = 0.0;
#pragma unroll 8
  for (int j = 0; j < D; ++j) s = s + qs[j] * kcol[(int64_t)j * stride];
  return s;
}

// One workgroup per (query block, b * H + h): scores of all key blocks, a bitonic sort
// on (score descending, block ascending) in LDS, the first kk blocks written in
// ascending block order.  Also writes the row's CSR offset.
template <int D>
__global__ __launch_bounds__(kSelThreads) void k_sel_topk(SelectArgs a, const double *qbar, const double *kbar_t,
                                                          const int32_t *pre, const int32_t *counts, int64_t *q2k_ptr,
                                                          int32_t *q2k_idx) {
  __shared__ double qs[D];
  __shared__ uint64_t key[kSelectMaxKv];
  __shared__ int32_t id[kSelectMaxKv];
  __shared__ uint8_t pick[kSelectMaxKv];
  __shared__ int32_t scan[kSelThreads];
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
  int np = 2;
  while (np < a.n_kv) np <<= 1;
  for (int j = threadIdx.x; j < D; j += kSelThreads) qs[j] = qbar[(bh * a.n_q + q) * D + j];
  __syncthreads();
  for (int k = threadIdx.x; k < np; k += kSelThreads) {
    uint64_t kv = ~0ull;
    if (k < a.n_kv && clamp_rows(a.kv_valid[k], kv_row0(a, k), a.seq_kv) > 0)
      kv = ~ordered_bits(dot_in_order<D>(qs, kbar_t + bh * D * (int64_t)a.n_kv + k, a.n_kv));
    key[k] = kv;
    id[k] = k;
    if (k < a.n_kv) pick[k] = 0;
  }
  __syncthreads();
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

template <int D>
hipError_t launch_select_d(const SelectArgs &a, int32_t top_k, const void *q, const void *k, double *qbar,
                           double *kbar_t, int32_t *pre, int32_t *counts, int64_t *q2k_ptr, int32_t *q2k_idx,
                           hipStream_t st) {
  constexpr int BPW = kSelThreads / (D / 8);
  const unsigned bh = (unsigned)a.bh_count;
  hipLaunchKernelGGL(k_sel_counts, dim3(1), dim3(1024), 0, st, a, top_k, pre, counts);
  hipLaunchKernelGGL((k_sel_means<D, false>), dim3((a.n_q + BPW - 1) / BPW, bh), dim3(kSelThreads), 0, st, a,
                     (const __bf16 *)q, qbar);
  hipLaunchKernelGGL((k_sel_means<D, true>), dim3((a.n_kv + BPW - 1) / BPW, bh), dim3(kSelThreads), 0, st, a,
                     (const __bf16 *)k, kbar_t);
  hipLaunchKernelGGL(k_sel_topk<D>, dim3(a.n_q, bh), dim3(kSelThreads), 0, st, a, qbar, kbar_t, pre, counts,
                     q2k_ptr, q2k_idx);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const SelectArgs &a, int head_dim, int32_t top_k, const void *q, const void *k, void *ws,
                         int64_t *q2k_ptr, int32_t *q2k_idx, hipStream_t stream) {
  const SelectWorkspace w = select_workspace(a, head_dim);
  char *base = static_cast<char *>(ws);
  int32_t *counts = reinterpret_cast<int32_t *>(base + w.counts);
  int32_t *pre = reinterpret_cast<int32_t *>(base + w.pre);
  double *qbar = reinterpret_cast<double *>(base + w.qbar);
  double *kbar_t = reinterpret_cast<double *>(base + w.kbar);
  if (head_dim == 128)
    return launch_select_d<128>(a, top_k, q, k, qbar, kbar_t, pre, counts, q2k_ptr, q2k_idx, stream);
  if (head_dim == 64) return launch_select_d<64>(a, top_k, q, k, qbar, kbar_t, pre, counts, q2k_ptr, q2k_idx, stream);
  return hipErrorInvalidValue;
}

}  // namespace kpage
