// GPU-side forward planner (KPage paper, sections 3.2.1-3.2.4 and 3.4; pair accounting
// of section 4.4).  Same tables, in the same order, as the host planner in plan.cpp:
//   walk of query block q: the full pages of every selected block in selection order,
//   then the partial tail page of every partial block in selection order, then dummy
//   pages up to a multiple of the route's pages per step (16 for Q64, 8 for Q128);
//   two 16-bit page masks per validity word; route Q64 for 1..64 valid rows, Q128 above;
//   per-route queues ordered by descending unpadded walk length, then (bh, q).
// One thread per (slot, query block) builds that block's walk; scans run in one
// workgroup; the queues are sorted with a device radix sort on
// (unpadded length descending, bh * n_q + q) keys.
#include "plan_dev.hpp"

#include <hipcub/hipcub.hpp>

#include <vector>

namespace kpage {
namespace {

enum : uint32_t {
  kErrQValid = 1u << 0,
  kErrKvValid = 1u << 1,
  kErrPtr = 1u << 2,
  kErrIdx = 1u << 3,
  kErrDup = 1u << 4,
  kErrOffset = 1u << 5,
  kErrFootprint = 1u << 6,
  kErrOverlap = 1u << 7,
};

// device -> host summary
struct Summary {
  uint32_t err;
  int32_t pad0;
  int64_t walk_total;
  int32_t n_q128, n_q64, n_zero, pad1;  // over all (b, h)
  unsigned long long useful, whole_block, paged_m128, nominal, scheduled;
};

constexpr int kScanThreads = 1024;

__device__ __forceinline__ int pages_of(int c) { return (c + kPageRows - 1) / kPageRows; }
__device__ __forceinline__ uint32_t tail_mask(int c) { return (1u << (c % kPageRows)) - 1u; }
__device__ __forceinline__ int64_t kv_off(const DevProblem &p, int g, int k) {
  return p.kv_offset ? p.kv_offset[int64_t(g) * p.n_kv + k] : int64_t(kBlockRows) * k;
}

__global__ void k_fill_i32(int32_t *p, int64_t n, int32_t v) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// K/V blocks: sizes, page-aligned offsets, footprints inside seq_kv and pairwise
// disjoint (each page claimed by one block: compare-and-swap on a page-owner table)
__global__ void k_check_kv(DevProblem p, int32_t *page_owner, Summary *sum) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(p.slots) * p.n_kv) return;
  const int g = int(i / p.n_kv), k = int(i % p.n_kv);
  const int c = p.kv_valid[i];
  if (c < 0 || c > kBlockRows) {
    atomicOr(&sum->err, kErrKvValid);
    return;
  }
  const int64_t off = kv_off(p, g, k);
  if (off < 0 || off % kPageRows) {
    atomicOr(&sum->err, kErrOffset);
    return;
  }
  const int np = pages_of(c);
  if (off + int64_t(kPageRows) * np > p.seq_kv) {
    atomicOr(&sum->err, kErrFootprint);
    return;
  }
  const int64_t n_pages = p.seq_kv / kPageRows;
  for (int j = 0; j < np; ++j) {
    const int old = atomicCAS(&page_owner[int64_t(g) * n_pages + off / kPageRows + j], -1, k);
    if (old != -1) atomicOr(&sum->err, kErrOverlap);
  }
}

// per (slot, query block): validation, route, walk lengths and pair counts
__global__ void k_count(DevProblem p, int align64, int align128, int32_t *route, int32_t *nfull, int32_t *unpadded,
                        int64_t *len, Summary *sum) {
  __shared__ unsigned long long st[5];
  __shared__ int cnt[3];
  if (threadIdx.x < 5) st[threadIdx.x] = 0;
  if (threadIdx.x < 3) cnt[threadIdx.x] = 0;
  __syncthreads();
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < int64_t(p.slots) * p.n_q) {
    const int g = int(i / p.n_q), q = int(i % p.n_q);
    const int mult = p.per_head ? 1 : p.batch * p.heads;  // (b, h) sharing this slot
    const int cq = p.q_valid[i];
    const int64_t a = p.q2k_ptr[int64_t(g) * (p.n_q + 1) + q], b = p.q2k_ptr[int64_t(g) * (p.n_q + 1) + q + 1];
    int r = 0, nf = 0, unp = 0;
    int64_t l = 0;
    bool ok = true;
    if (cq < 0 || cq > kBlockRows) {
      atomicOr(&sum->err, kErrQValid);
      ok = false;
    }
    if (a < 0 || b < a || b > p.nnz) {
      atomicOr(&sum->err, kErrPtr);
      ok = false;
    }
    if (ok) {
      unsigned long long useful = 0, psum = 0;
      int tails = 0;
      for (int64_t e = a; e < b; ++e) {
        const int k = p.q2k_idx[e];
        if (k < 0 || k >= p.n_kv) {
          atomicOr(&sum->err, kErrIdx);
          ok = false;
          continue;
        }
        for (int64_t e2 = a; e2 < e; ++e2)
          if (p.q2k_idx[e2] == k) {
            atomicOr(&sum->err, kErrDup);
            ok = false;
          }
        const int ck = min(max(p.kv_valid[int64_t(g) * p.n_kv + k], 0), kBlockRows);
        nf += ck / kPageRows;
        tails += (ck % kPageRows) ? 1 : 0;
        useful += (unsigned long long)cq * (unsigned long long)ck;
        psum += (unsigned long long)pages_of(ck);
      }
      if (ok && cq > 0) {
        r = cq <= 64 ? 64 : 128;
        const int per_step = r == 64 ? align64 : align128;
        unp = nf + tails;
        l = (unp + per_step - 1) / per_step * per_step;
        const unsigned long long M = (unsigned long long)r;
        atomicAdd(&st[0], mult * useful);
        atomicAdd(&st[1], mult * (unsigned long long)kBlockRows * kBlockRows * (unsigned long long)(b - a));
        atomicAdd(&st[2], mult * (unsigned long long)kBlockRows * kPageRows * psum);
        atomicAdd(&st[3], mult * M * kPageRows * psum);
        atomicAdd(&st[4], mult * M * kPageRows * (unsigned long long)l);
        atomicAdd(&cnt[r == 128 ? 0 : 1], mult);
      } else if (ok) {
        atomicAdd(&cnt[2], mult);
        nf = 0;
      }
    }
    route[i] = r;
    nfull[i] = r ? nf : 0;
    unpadded[i] = r ? unp : 0;
    len[i] = l;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(&sum->useful, st[0]);
    atomicAdd(&sum->whole_block, st[1]);
    atomicAdd(&sum->paged_m128, st[2]);
    atomicAdd(&sum->nominal, st[3]);
    atomicAdd(&sum->scheduled, st[4]);
    atomicAdd(&sum->n_q128, cnt[0]);
    atomicAdd(&sum->n_q64, cnt[1]);
    atomicAdd(&sum->n_zero, cnt[2]);
  }
}

// exclusive scan of v over a workgroup of kScanThreads; returns this thread's prefix
__device__ int64_t block_scan(int64_t v, int64_t *lds, int64_t *total) {
  const int t = threadIdx.x;
  lds[t] = v;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int64_t x = t >= off ? lds[t - off] : 0;
    __syncthreads();
    lds[t] += x;
    __syncthreads();
  }
  *total = lds[kScanThreads - 1];
  const int64_t excl = lds[t] - v;
  __syncthreads();
  return excl;
}

// walk_ptr[g][q] = global start of walk (g, q); walk_ptr[g][n_q] = end of slot g
__global__ __launch_bounds__(kScanThreads) void k_scan_walks(DevProblem p, const int64_t *len, int64_t *walk_ptr,
                                                             Summary *sum) {
  __shared__ int64_t lds[kScanThreads];
  const int64_t n = int64_t(p.slots) * p.n_q;
  int64_t carry = 0;
  for (int64_t base = 0; base < n; base += kScanThreads) {
    const int64_t i = base + threadIdx.x;
    const int64_t v = i < n ? len[i] : 0;
    int64_t total;
    const int64_t pre = carry + block_scan(v, lds, &total);
    if (i < n) {
      const int g = int(i / p.n_q), q = int(i % p.n_q);
      walk_ptr[int64_t(g) * (p.n_q + 1) + q] = pre;
      if (q == p.n_q - 1) walk_ptr[int64_t(g) * (p.n_q + 1) + p.n_q] = pre + v;
    }
    carry += total;
  }
  if (threadIdx.x == 0) sum->walk_total = carry;
}

// walk, redirected page table and validity words of (slot, query block)
__global__ void k_fill_walks(DevProblem p, const int32_t *route, const int32_t *nfull, const int64_t *walk_ptr,
                             int32_t *walk, int32_t *pages, uint32_t *valid) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(p.slots) * p.n_q || route[i] == 0) return;
  const int g = int(i / p.n_q), q = int(i % p.n_q);
  const int64_t base = walk_ptr[int64_t(g) * (p.n_q + 1) + q], end = walk_ptr[int64_t(g) * (p.n_q + 1) + q + 1];
  if (end <= base) return;
  const int64_t a = p.q2k_ptr[int64_t(g) * (p.n_q + 1) + q], b = p.q2k_ptr[int64_t(g) * (p.n_q + 1) + q + 1];
  int64_t pos = base;
  uint32_t lo = 0;
  int32_t first = -1;
  auto emit = [&](int32_t page, uint32_t mask) {
    if (first < 0) first = page;
    walk[pos] = page;
    pages[pos] = page >= 0 ? page : first;
    if ((pos - base) & 1) valid[pos >> 1] = lo | (mask << 16);
    else lo = mask;
    ++pos;
  };
  for (int64_t e = a; e < b; ++e) {  // full pages, selection order
    const int k = p.q2k_idx[e];
    const int ck = p.kv_valid[int64_t(g) * p.n_kv + k];
    const int32_t pg0 = int32_t(kv_off(p, g, k) / kPageRows);
    for (int j = 0; j < ck / kPageRows; ++j) emit(pg0 + j, kFullMask);
  }
  for (int64_t e = a; e < b; ++e) {  // partial tails, selection order
    const int k = p.q2k_idx[e];
    const int ck = p.kv_valid[int64_t(g) * p.n_kv + k];
    if (ck % kPageRows) emit(int32_t(kv_off(p, g, k) / kPageRows) + ck / kPageRows, tail_mask(ck));
  }
  while (pos < end) emit(-1, 0u);  // dummies (a walk that has any page starts with a real one)
  (void)nfull;
}

// queue sort keys: (unpadded descending, bh * n_q + q ascending); other routes sort last
__global__ void k_queue_keys(DevProblem p, const int32_t *route, const int32_t *unpadded, unsigned long long *k64,
                             unsigned long long *k128) {
  const int64_t f = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t n = int64_t(p.batch) * p.heads * p.n_q;
  if (f >= n) return;
  const int bh = int(f / p.n_q), q = int(f % p.n_q);
  const int64_t i = int64_t(p.per_head ? bh : 0) * p.n_q + q;
  const unsigned long long key =
      ((unsigned long long)(0x7FFFFFFF - unpadded[i]) << 32) | (unsigned long long)(uint32_t)f;
  k64[f] = route[i] == 64 ? key : ~0ull;
  k128[f] = route[i] == 128 ? key : ~0ull;
}

__global__ void k_queue_out(const unsigned long long *keys, int n, int n_q, int32_t *queue) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t f = uint32_t(keys[i] & 0xFFFFFFFFull);
  queue[2 * i] = int32_t(f / uint32_t(n_q));
  queue[2 * i + 1] = int32_t(f % uint32_t(n_q));
}

// Launch position of entry p of a list of n: workgroup i goes to XCD i % 8, so XCD x
// takes the x-th contiguous eighth of the list in order (see the host planner glue).
__device__ __forceinline__ int64_t xcd_position(int64_t pidx, int64_t n) {
  const int64_t m = n / 8, r = n % 8;
  int64_t x, j;
  if (pidx < r * (m + 1)) {
    x = pidx / (m + 1);
    j = pidx % (m + 1);
  } else {
    x = r + (pidx - r * (m + 1)) / m;
    j = (pidx - r * (m + 1)) % m;
  }
  return j * 8 + x;
}

// launch items in (bh, q) order per route; the Q64 list also carries the cleanup items
// of empty query blocks after its own items
__global__ __launch_bounds__(kScanThreads) void k_items(DevProblem p, const int32_t *route, const int32_t *nfull,
                                                        const int64_t *walk_ptr, const Summary *sum, FwdItem *items128,
                                                        FwdItem *items64) {
  __shared__ int64_t lds[kScanThreads];
  const int64_t n = int64_t(p.batch) * p.heads * p.n_q;
  const int64_t n128 = sum->n_q128, n64 = sum->n_q64, nall64 = sum->n_q64 + sum->n_zero;
  int64_t c128 = 0, c64 = 0, cz = 0;
  for (int64_t base = 0; base < n; base += kScanThreads) {
    const int64_t f = base + threadIdx.x;
    int r = -1, cq = 0;
    int64_t i = 0;
    int bh = 0, q = 0;
    if (f < n) {
      bh = int(f / p.n_q);
      q = int(f % p.n_q);
      i = int64_t(p.per_head ? bh : 0) * p.n_q + q;
      r = route[i];
      cq = p.q_valid[i];
    }
    int64_t t128, t64, tz;
    const int64_t p128 = c128 + block_scan(r == 128 ? 1 : 0, lds, &t128);
    const int64_t p64 = c64 + block_scan(r == 64 ? 1 : 0, lds, &t64);
    const int64_t pz = cz + block_scan(f < n && r == 0 && cq == 0 ? 1 : 0, lds, &tz);
    if (f < n && (r != 0 || cq == 0)) {
      FwdItem x{};
      const int64_t wp = int64_t(p.per_head ? bh : 0) * (p.n_q + 1) + q;
      x.walk_off = walk_ptr[wp];
      x.walk_len = int32_t(walk_ptr[wp + 1] - x.walk_off);
      x.bh = bh;
      x.q = q;
      x.n_full = nfull[i];
      x.c_q = cq;
      if (r == 128) items128[xcd_position(p128, n128)] = x;
      else if (r == 64) items64[xcd_position(p64, nall64)] = x;
      else items64[xcd_position(n64 + pz, nall64)] = x;
    }
    c128 += t128;
    c64 += t64;
    cz += tz;
  }
}

int blocks_for(int64_t n, int threads) { return int((n + threads - 1) / threads); }

}  // namespace

kpage_status build_forward_device(const DevProblem &p, int align64, int align128, hipStream_t st,
                                  const DevAlloc &alloc, DevFwdTables *t, std::string *err) {
  const int64_t GQ = int64_t(p.slots) * p.n_q, GK = int64_t(p.slots) * p.n_kv;
  const int64_t BHQ = int64_t(p.batch) * p.heads * p.n_q;
  const int64_t n_pages = p.seq_kv / kPageRows;
  auto a32 = [&](int64_t n) { return static_cast<int32_t *>(alloc(size_t(std::max<int64_t>(n, 1)) * 4)); };
  auto a64 = [&](int64_t n) { return static_cast<int64_t *>(alloc(size_t(std::max<int64_t>(n, 1)) * 8)); };
  Summary *d_sum = static_cast<Summary *>(alloc(sizeof(Summary)));
  int32_t *owner = a32(int64_t(p.slots) * n_pages);
  int64_t *len = a64(GQ);
  t->route = a32(GQ);
  t->nfull = a32(GQ);
  t->unpadded = a32(GQ);
  t->walk_ptr = a64(int64_t(p.slots) * (p.n_q + 1));
  if (!d_sum || !owner || !len || !t->route || !t->nfull || !t->unpadded || !t->walk_ptr) {
    *err = "device allocation failed while planning";
    return KPAGE_ERR_OOM;
  }
  hipError_t e;
#define KP_CHECK(call)                                                   \
  do {                                                                   \
    if ((e = (call)) != hipSuccess) {                                    \
      *err = std::string(#call) + ": " + hipGetErrorString(e);           \
      return KPAGE_ERR_HIP;                                              \
    }                                                                    \
  } while (0)
  const int TB = 256;
  KP_CHECK(hipMemsetAsync(d_sum, 0, sizeof(Summary), st));
  hipLaunchKernelGGL(k_fill_i32, dim3(blocks_for(int64_t(p.slots) * n_pages, TB)), dim3(TB), 0, st, owner,
                     int64_t(p.slots) * n_pages, -1);
  hipLaunchKernelGGL(k_check_kv, dim3(blocks_for(GK, TB)), dim3(TB), 0, st, p, owner, d_sum);
  hipLaunchKernelGGL(k_count, dim3(blocks_for(GQ, TB)), dim3(TB), 0, st, p, align64, align128, t->route, t->nfull,
                     t->unpadded, len, d_sum);
  hipLaunchKernelGGL(k_scan_walks, dim3(1), dim3(kScanThreads), 0, st, p, len, t->walk_ptr, d_sum);
  KP_CHECK(hipGetLastError());
  Summary h{};
  KP_CHECK(hipMemcpyAsync(&h, d_sum, sizeof(Summary), hipMemcpyDeviceToHost, st));
  KP_CHECK(hipStreamSynchronize(st));
  if (h.err) {
    const char *msg = (h.err & kErrQValid)      ? "q_valid outside [0,128]"
                      : (h.err & kErrKvValid)   ? "kv_valid outside [0,128]"
                      : (h.err & kErrPtr)       ? "q2k_ptr must be non-negative, non-decreasing and within nnz"
                      : (h.err & kErrIdx)       ? "q2k_idx entry outside [0, n_kv)"
                      : (h.err & kErrDup)       ? "duplicate K/V block in a selection list"
                      : (h.err & kErrOffset)    ? "kv_offset must be a non-negative multiple of 16"
                      : (h.err & kErrFootprint) ? "a K/V block footprint exceeds seq_kv"
                                                : "K/V block page footprints overlap";
    *err = msg;
    return KPAGE_ERR_INVALID;
  }
  t->walk_total = h.walk_total;
  t->n_q128 = h.n_q128;
  t->n_q64 = h.n_q64;
  t->n_zero = h.n_zero;
  t->walk = a32(h.walk_total);
  t->pages = a32(h.walk_total);
  t->valid = static_cast<uint32_t *>(alloc(size_t(std::max<int64_t>(h.walk_total / 2, 1)) * 4));
  t->q64_queue = a32(2 * int64_t(h.n_q64));
  t->q128_queue = a32(2 * int64_t(h.n_q128));
  t->items128 = static_cast<FwdItem *>(alloc(size_t(std::max(h.n_q128, 1)) * sizeof(FwdItem)));
  t->items64 = static_cast<FwdItem *>(alloc(size_t(std::max(h.n_q64 + h.n_zero, 1)) * sizeof(FwdItem)));
  const int n_redo = std::max(std::max(h.n_q128, h.n_q64 + h.n_zero), 1);
  t->redo = a32(n_redo);
  unsigned long long *keys = static_cast<unsigned long long *>(alloc(size_t(std::max<int64_t>(BHQ, 1)) * 8 * 3));
  if (!t->walk || !t->pages || !t->valid || !t->q64_queue || !t->q128_queue || !t->items128 || !t->items64 ||
      !t->redo || !keys) {
    *err = "device allocation failed while planning";
    return KPAGE_ERR_OOM;
  }
  hipLaunchKernelGGL(k_fill_walks, dim3(blocks_for(GQ, TB)), dim3(TB), 0, st, p, t->route, t->nfull, t->walk_ptr,
                     t->walk, t->pages, t->valid);
  hipLaunchKernelGGL(k_fill_i32, dim3(blocks_for(n_redo, TB)), dim3(TB), 0, st, t->redo, int64_t(n_redo), 0);
  // queues: one radix sort per route over all (bh, q) keys
  unsigned long long *k64 = keys, *k128 = keys + BHQ, *ksorted = keys + 2 * BHQ;
  hipLaunchKernelGGL(k_queue_keys, dim3(blocks_for(BHQ, TB)), dim3(TB), 0, st, p, t->route, t->unpadded, k64, k128);
  size_t tmp_bytes = 0;
  KP_CHECK(hipcub::DeviceRadixSort::SortKeys(nullptr, tmp_bytes, k64, ksorted, int(BHQ), 0, 64, st));
  void *tmp = alloc(std::max<size_t>(tmp_bytes, 16));
  if (!tmp) {
    *err = "device allocation failed while planning";
    return KPAGE_ERR_OOM;
  }
  if (h.n_q64 > 0) {
    KP_CHECK(hipcub::DeviceRadixSort::SortKeys(tmp, tmp_bytes, k64, ksorted, int(BHQ), 0, 64, st));
    hipLaunchKernelGGL(k_queue_out, dim3(blocks_for(h.n_q64, TB)), dim3(TB), 0, st, ksorted, h.n_q64, p.n_q,
                       t->q64_queue);
  }
  if (h.n_q128 > 0) {
    KP_CHECK(hipcub::DeviceRadixSort::SortKeys(tmp, tmp_bytes, k128, ksorted, int(BHQ), 0, 64, st));
    hipLaunchKernelGGL(k_queue_out, dim3(blocks_for(h.n_q128, TB)), dim3(TB), 0, st, ksorted, h.n_q128, p.n_q,
                       t->q128_queue);
  }
  hipLaunchKernelGGL(k_items, dim3(1), dim3(kScanThreads), 0, st, p, t->route, t->nfull, t->walk_ptr, d_sum,
                     t->items128, t->items64);
  KP_CHECK(hipGetLastError());
  KP_CHECK(hipMemcpyAsync(&h, d_sum, sizeof(Summary), hipMemcpyDeviceToHost, st));
  KP_CHECK(hipStreamSynchronize(st));
#undef KP_CHECK
  t->stats = PairStats();
  t->stats.useful = h.useful;
  t->stats.whole_block = h.whole_block;
  t->stats.paged_m128 = h.paged_m128;
  t->stats.nominal = h.nominal;
  t->stats.scheduled = h.scheduled;
  return KPAGE_OK;
}

}  // namespace kpage
