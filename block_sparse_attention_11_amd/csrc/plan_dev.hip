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
constexpr int kOwnersLdsMax = 48 * 1024;  // dynamic LDS of the owner packing (about 390,000 blocks)

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
// `seen` (optional): one bit per K/V block for every (slot, query block), so the
// duplicate check of a selection list is linear; without it the check is quadratic.
__global__ void k_count(DevProblem p, int align64, int align128, int32_t *route, int32_t *nfull, int32_t *unpadded,
                        int64_t *len, Summary *sum, uint32_t *seen) {
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
    uint32_t *row = nullptr;
    if (seen) {
      const int nkw = (p.n_kv + 31) / 32;
      row = seen + i * nkw;
      for (int w = 0; w < nkw; ++w) row[w] = 0u;
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
        if (row) {  // this thread's own row: plain read-modify-write
          const uint32_t bit = 1u << (k & 31);
          if (row[k >> 5] & bit) {
            atomicOr(&sum->err, kErrDup);
            ok = false;
          }
          row[k >> 5] |= bit;
        } else {
          for (int64_t e2 = a; e2 < e; ++e2)
            if (p.q2k_idx[e2] == k) {
              atomicOr(&sum->err, kErrDup);
              ok = false;
            }
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
__global__ void k_fill_walks(DevProblem p, const int32_t *route, const int64_t *walk_ptr, int32_t *walk,
                             int32_t *pages, uint32_t *valid) {
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

// Launch items in (bh, q) order per route; the Q64 list also carries the cleanup items
// of empty query blocks after its own items.  Launch order (the host planner's, in the
// same closed form): one list of both routes, head-major, each head's M128 items before
// its M64 items, cleanup items last; list position L of M128 item i of head bh is
// i + (M64 items of heads < bh), of M64 item j is j + (M128 items of heads <= bh), of
// cleanup item z is n128 + n64 + z; workgroup launch_position(L) runs that item
// (order[] = i, or ~(index in the M64 list)).  hs128 / hs64 [BH + 1]: items of each
// route in the heads before bh.
// With group items (in_group: members; hsg [BH + 1]: group items of the heads before bh,
// NULL without groups): a head's group items follow its other M128 items (k_group_items
// writes them), member blocks are no M64 items, and every later position shifts by the
// group items before it.
__global__ __launch_bounds__(kScanThreads) void k_items(DevProblem p, const int32_t *route, const int32_t *nfull,
                                                        const int32_t *unpadded, const int64_t *walk_ptr,
                                                        const Summary *sum, const uint8_t *in_group,
                                                        const int64_t *hsg, int64_t n_members, FwdItem *items128,
                                                        FwdItem *items64, int64_t *hs128, int64_t *hs64,
                                                        int32_t *order) {
  __shared__ int64_t lds[kScanThreads];
  const int64_t n = int64_t(p.batch) * p.heads * p.n_q;
  const int BH = p.batch * p.heads;
  const int64_t n_gi = hsg ? hsg[BH] : 0;
  const int64_t n128 = sum->n_q128, n64 = sum->n_q64 - n_members, n_all = n128 + n_gi + n64 + sum->n_zero;
  auto gb = [&](int bh) -> int64_t { return hsg ? hsg[bh] : 0; };
  for (int pass = 0; pass < 2; ++pass) {
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
        if (r == 64 && in_group && in_group[i]) r = -1;  // runs inside its group item
      }
      int64_t t128, t64, tz;
      const int64_t p128 = c128 + block_scan(r == 128 ? 1 : 0, lds, &t128);
      const int64_t p64 = c64 + block_scan(r == 64 ? 1 : 0, lds, &t64);
      const int64_t pz = cz + block_scan(f < n && r == 0 && cq == 0 ? 1 : 0, lds, &tz);
      if (pass == 0 && f < n && q == 0) {
        hs128[bh] = p128;
        hs64[bh] = p64;
      }
      if (f < n && r >= 0 && (r != 0 || cq == 0)) {
        if (pass == 0) {
          FwdItem x{};
          const int64_t wp = int64_t(p.per_head ? bh : 0) * (p.n_q + 1) + q;
          x.walk_off = walk_ptr[wp];
          x.walk_len = int32_t(walk_ptr[wp + 1] - x.walk_off);
          x.bh = bh;
          x.q = q;
          x.n_full = nfull[i];
          x.n_pages = unpadded[i];
          x.c_q = cq;
          if (r == 128) items128[p128 + gb(bh)] = x;
          else if (r == 64) items64[p64] = x;
          else items64[n64 + pz] = x;
        } else {
          int64_t L;
          int32_t tag;
          if (r == 128) {
            L = p128 + gb(bh) + hs64[bh];
            tag = int32_t(p128 + gb(bh));
          } else if (r == 64) {
            L = p64 + hs128[bh + 1] + gb(bh + 1);
            tag = ~int32_t(p64);
          } else {
            L = n128 + n_gi + n64 + pz;
            tag = ~int32_t(n64 + pz);
          }
          order[launch_position(L, n_all, p.xcd_chunk)] = tag;
        }
      }
      c128 += t128;
      c64 += t64;
      cz += tz;
    }
    if (pass == 0 && threadIdx.x == 0) {
      hs128[BH] = c128;
      hs64[BH] = c64;
    }
    __syncthreads();  // head starts visible to the second pass
  }
}

// The last kFwdTail entries of each XCD's launch sequence (positions 8 j + x) in
// descending fwd_tail_cost, ties in launch order: one workgroup per XCD sorts them in
// LDS (bitonic), the same order as the host planner's.
__global__ __launch_bounds__(kFwdTail) void k_fwd_tails(int32_t *order, const FwdItem *items128,
                                                        const FwdItem *items64, int64_t n) {
  __shared__ unsigned long long key[kFwdTail];
  __shared__ int32_t tag[kFwdTail];
  const int x = int(blockIdx.x);
  const int64_t cnt = n > x ? (n - x + kXcds - 1) / kXcds : 0;
  const int64_t t = cnt < kFwdTail ? cnt : kFwdTail;
  const int64_t j0 = cnt - t;
  const int i = int(threadIdx.x);
  if (i < t) {
    const int32_t tg = order[(j0 + i) * kXcds + x];
    const int32_t c = tg >= 0 ? fwd_tail_cost(128, items128[tg].n_pages) : fwd_tail_cost(64, items64[~tg].n_pages);
    tag[i] = tg;
    key[i] = ((unsigned long long)(uint32_t)(0x7FFFFFFF - c) << 32) | (unsigned long long)(uint32_t)i;
  } else {
    key[i] = ~0ull;
  }
  __syncthreads();
  for (int k = 2; k <= kFwdTail; k <<= 1)
    for (int h = k >> 1; h > 0; h >>= 1) {
      const int l = i ^ h;
      if (l > i) {
        const unsigned long long a = key[i], b = key[l];
        if ((a > b) == ((i & k) == 0)) {
          key[i] = b;
          key[l] = a;
        }
      }
      __syncthreads();
    }
  if (i < t) order[(j0 + i) * kXcds + x] = tag[uint32_t(key[i])];
}

// ---------------------------------------------------------------------------------
// Group items (the host planner's build_groups: same rule, same groups, same union walks).
// Candidates of a slot: the query blocks of the Q64 route with 1..32 valid rows and a
// non-empty walk, in block order, each held as a bitset of its walk's pages.  One
// workgroup per slot makes the greedy choice (the opening blocks in order; each pick a
// parallel argmax over the free candidates, ties to the lower block); one workgroup per
// group then writes its union walk, in the same order as the host, and the validity
// words of its four waves.
constexpr int kGroupThreads = 256;

// row mask of page pg of slot g (a page of a walk lies in a selected block's footprint)
__device__ __forceinline__ uint32_t dev_page_mask(const DevProblem &p, const int32_t *page_block, int g, int32_t pg) {
  const int64_t n_pg = p.seq_kv / kPageRows;
  const int b = page_block[int64_t(g) * n_pg + pg];
  const int ck = p.kv_valid[int64_t(g) * p.n_kv + b];
  const int j = pg - int(kv_off(p, g, b) / kPageRows);
  return (j + 1) * kPageRows <= ck ? kFullMask : tail_mask(ck);
}

// candidates of slot blockIdx.x in block order; their count
__global__ __launch_bounds__(kScanThreads) void k_group_cands(DevProblem p, const int32_t *route,
                                                              const int32_t *unpadded, int32_t *cand,
                                                              int32_t *n_cand) {
  __shared__ int64_t lds[kScanThreads];
  const int g = int(blockIdx.x);
  int64_t c = 0;
  for (int base = 0; base < p.n_q; base += kScanThreads) {
    const int q = base + int(threadIdx.x);
    bool f = false;
    if (q < p.n_q) {
      const int64_t i = int64_t(g) * p.n_q + q;
      const int cq = p.q_valid[i];
      f = route[i] == 64 && cq > 0 && cq <= kGroupMaxRows && unpadded[i] > 0;
    }
    int64_t tot;
    const int64_t pos = c + block_scan(f ? 1 : 0, lds, &tot);
    if (f) cand[int64_t(g) * p.n_q + pos] = q;
    c += tot;
  }
  if (threadIdx.x == 0) n_cand[g] = int32_t(c);
}

// slot of global index i with ptr[g] <= i < ptr[g + 1] (ptr non-decreasing, ptr[0] = 0)
__device__ __forceinline__ int slot_of_index(const int64_t *ptr, int slots, int64_t i) {
  int lo = 0, hi = slots;
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (ptr[mid] <= i) lo = mid;
    else hi = mid;
  }
  return lo;
}

// page bitset of candidate blockIdx.x (global candidate index; bits zeroed beforehand)
__global__ void k_group_bits(DevProblem p, const int64_t *walk_ptr, const int32_t *walk, const int32_t *unpadded,
                             const int32_t *cand, const int64_t *cand_off, int W, unsigned long long *bits) {
  const int64_t ci = blockIdx.x;
  const int g = slot_of_index(cand_off, p.slots, ci);
  const int q = cand[int64_t(g) * p.n_q + (ci - cand_off[g])];
  const int64_t a = walk_ptr[int64_t(g) * (p.n_q + 1) + q];
  const int n = unpadded[int64_t(g) * p.n_q + q];
  unsigned long long *b = bits + ci * W;
  for (int i = int(threadIdx.x); i < n; i += int(blockDim.x)) {
    const int32_t pg = walk[a + i];
    atomicOr(&b[pg >> 6], 1ull << (pg & 63));
  }
}

// the greedy choice of slot blockIdx.x; group gi of the slot: members (candidate
// indices, -1 none) at gmem[(cand_off + gi) * 4 ..], union size at gunion[cand_off + gi]
__global__ __launch_bounds__(kGroupThreads) void k_group_greedy(DevProblem p, const int32_t *unpadded,
                                                                const int32_t *cand, const int32_t *n_cand,
                                                                const int64_t *cand_off, int W,
                                                                const unsigned long long *bits, int32_t *gmem,
                                                                int32_t *gunion, int32_t *gcount, int32_t *gmembers) {
  extern __shared__ unsigned long long gl[];  // union [W], intersection [W], taken flags [n_cand]
  unsigned long long *uni = gl, *inter = gl + W;
  uint8_t *taken = reinterpret_cast<uint8_t *>(gl + 2 * W);
  __shared__ int64_t r_in[kGroupThreads], r_n[kGroupThreads];
  __shared__ int32_t r_c[kGroupThreads];
  __shared__ int32_t mem[kGroupMembers];
  const int g = int(blockIdx.x), tid = int(threadIdx.x);
  const int nc = n_cand[g];
  const int64_t off = cand_off[g];
  const unsigned long long *B = bits + off * W;
  for (int c = tid; c < nc; c += kGroupThreads) taken[c] = 0;
  int ng = 0, nmem = 0;
  for (int c0 = 0; c0 < nc; ++c0) {
    __syncthreads();
    const bool skip = taken[c0] != 0;
    __syncthreads();  // every wave has read the flag before thread 0 may set it
    if (skip) continue;
    if (tid == 0) {
      taken[c0] = 1;
      mem[0] = c0;
      mem[1] = mem[2] = mem[3] = -1;
    }
    for (int w = tid; w < W; w += kGroupThreads) uni[w] = inter[w] = B[int64_t(c0) * W + w];
    __syncthreads();
    int m = 1;
    while (m < kGroupMembers) {
      int64_t bi = 0, bn = 1;
      int32_t bc = -1;
      for (int c = c0 + 1 + tid; c < nc; c += kGroupThreads) {
        if (taken[c]) continue;
        const unsigned long long *bb = B + int64_t(c) * W;
        // one pass over the words (independent loads): pages shared with every member, and
        // pages already in the union
        unsigned long long sh = 0;
        int64_t in = 0;
#pragma unroll 8
        for (int w = 0; w < W; ++w) {
          const unsigned long long x = bb[w];
          sh |= inter[w] & x;
          in += __popcll(uni[w] & x);
        }
        if (sh == 0) continue;  // no page selected by every member and by c
        const int64_t n = unpadded[int64_t(g) * p.n_q + cand[int64_t(g) * p.n_q + c]];
        if (bc < 0 || in * bn > bi * n) {
          bi = in;
          bn = n;
          bc = c;
        }
      }
      r_in[tid] = bi;
      r_n[tid] = bn;
      r_c[tid] = bc;
      __syncthreads();
      for (int h = kGroupThreads / 2; h > 0; h >>= 1) {
        if (tid < h) {
          const int32_t c1 = r_c[tid + h], c0b = r_c[tid];
          if (c1 >= 0) {
            const int64_t i1 = r_in[tid + h], n1 = r_n[tid + h], i0 = r_in[tid], n0 = r_n[tid];
            if (c0b < 0 || i1 * n0 > i0 * n1 || (i1 * n0 == i0 * n1 && c1 < c0b)) {
              r_in[tid] = i1;
              r_n[tid] = n1;
              r_c[tid] = c1;
            }
          }
        }
        __syncthreads();
      }
      const int32_t best = r_c[0];
      const int64_t best_in = r_in[0], best_n = r_n[0];
      __syncthreads();  // the next round rewrites r_*
      if (best < 0 || 2 * best_in < best_n) break;
      if (tid == 0) {
        taken[best] = 1;
        mem[m] = best;
      }
      for (int w = tid; w < W; w += kGroupThreads) {
        const unsigned long long x = B[int64_t(best) * W + w];
        uni[w] |= x;
        inter[w] &= x;
      }
      ++m;
      __syncthreads();
    }
    if (m >= 2) {
      int cnt = 0;
      for (int w = tid; w < W; w += kGroupThreads) cnt += __popcll(uni[w]);
      r_c[tid] = cnt;
      __syncthreads();
      for (int h = kGroupThreads / 2; h > 0; h >>= 1) {
        if (tid < h) r_c[tid] += r_c[tid + h];
        __syncthreads();
      }
      if (tid == 0) {
        for (int j = 0; j < kGroupMembers; ++j) gmem[(off + ng) * kGroupMembers + j] = mem[j];
        gunion[off + ng] = r_c[0];
      }
      ++ng;
      nmem += m;
    }
  }
  if (tid == 0) {
    gcount[g] = ng;
    gmembers[g] = nmem;
  }
}

// union walk, validity words and member table of group blockIdx.x (global group index)
__global__ __launch_bounds__(kScanThreads) void k_group_walks(
    DevProblem p, const int32_t *page_block, const int64_t *walk_ptr, const int32_t *walk, const int32_t *unpadded,
    const int32_t *cand, const int64_t *cand_off, int W, const unsigned long long *bits, const int32_t *gmem,
    const int64_t *group_ptr, const int64_t *gwalk_ptr, int64_t walk_base, int64_t valid_base, FwdGroup *groups,
    int32_t *members, int32_t *nfull, int32_t *npages, int32_t *gwalk, int32_t *pages, uint32_t *valid,
    uint32_t *gvalid, uint8_t *in_group) {
  extern __shared__ unsigned long long used[];  // [W]: pages already in the union walk
  __shared__ int64_t lds[kScanThreads];
  const int64_t i = blockIdx.x;
  const int tid = int(threadIdx.x);
  const int g = slot_of_index(group_ptr, p.slots, i);
  const int64_t k = i - group_ptr[g], off = cand_off[g];
  int32_t mc[kGroupMembers], mq[kGroupMembers];
  int nm = 0;
  for (int j = 0; j < kGroupMembers; ++j) {
    mc[j] = gmem[(off + k) * kGroupMembers + j];
    mq[j] = mc[j] >= 0 ? cand[int64_t(g) * p.n_q + mc[j]] : -1;
    nm += mc[j] >= 0 ? 1 : 0;
  }
  for (int w = tid; w < W; w += kScanThreads) used[w] = 0;
  __syncthreads();
  const int64_t o0 = gwalk_ptr[i], len = gwalk_ptr[i + 1] - o0;
  auto in_member = [&](int j, int32_t pg) -> bool {
    return (bits[(off + mc[j]) * W + (pg >> 6)] >> (pg & 63)) & 1ull;
  };
  int64_t pos = 0;
  // phase 0: full pages every member selected, 1: the other shared pages (both in the
  // first member's walk order), 2: a member's pages not yet in the walk
  auto pass = [&](int j, int phase) {
    const int q = mq[j];
    const int64_t a = walk_ptr[int64_t(g) * (p.n_q + 1) + q];
    const int n = unpadded[int64_t(g) * p.n_q + q];
    for (int base = 0; base < n; base += kScanThreads) {
      const int e = base + tid;
      int32_t pg = -1;
      bool f = false;
      if (e < n) {
        pg = walk[a + e];
        if (phase < 2) {
          bool all = true;
          for (int jj = 1; jj < nm; ++jj) all = all && in_member(jj, pg);
          const bool full = dev_page_mask(p, page_block, g, pg) == kFullMask;
          f = all && (phase == 0 ? full : !full);
        } else {
          f = !((used[pg >> 6] >> (pg & 63)) & 1ull);
        }
      }
      int64_t tot;
      const int64_t x = block_scan(f ? 1 : 0, lds, &tot);
      if (f && pos + x < len) {  // the union size bounds the walk (the guard only keeps stores in range)
        gwalk[o0 + pos + x] = pg;
        atomicOr(&used[pg >> 6], 1ull << (pg & 63));
      }
      pos += tot;
      __syncthreads();
    }
  };
  pass(0, 0);
  const int64_t n_full = pos;
  pass(0, 1);
  for (int j = 0; j < nm; ++j) pass(j, 2);
  for (int64_t e = pos + tid; e < len; e += kScanThreads) gwalk[o0 + e] = -1;
  __syncthreads();  // the walk, written by this workgroup, is read back below
  const int32_t first = gwalk[o0];
  for (int64_t e = tid; e < len; e += kScanThreads) {
    const int32_t pg = gwalk[o0 + e];
    pages[walk_base + o0 + e] = pg >= 0 ? pg : first;
  }
  const int64_t half = len / 2;
  for (int64_t e = tid; e < kGroupMembers * half; e += kScanThreads) {
    const int w = int(e / half);
    const int64_t j = e % half;
    uint32_t word = 0;
    if (mc[w] >= 0)
      for (int h = 0; h < 2; ++h) {
        const int32_t pg = gwalk[o0 + 2 * j + h];
        if (pg >= 0 && in_member(w, pg)) word |= dev_page_mask(p, page_block, g, pg) << (16 * h);
      }
    valid[valid_base + 2 * o0 + e] = word;
    gvalid[2 * o0 + e] = word;
  }
  if (tid < kGroupMembers) {
    FwdGroup &gr = groups[i];
    gr.q[tid] = mq[tid];
    gr.c_q[tid] = mq[tid] >= 0 ? p.q_valid[int64_t(g) * p.n_q + mq[tid]] : 0;
    members[i * kGroupMembers + tid] = mq[tid];
    if (mq[tid] >= 0) in_group[int64_t(g) * p.n_q + mq[tid]] = 1;
    if (tid == 0) {
      gr.valid_off = valid_base + 2 * o0;
      gr.pad = 0;
      nfull[i] = int32_t(n_full);
      npages[i] = int32_t(pos);
    }
  }
}

// group item k of head bh: M128 item hs128[bh + 1] + hsg[bh] + k (after the head's other
// M128 items), list position that + hs64[bh]; one thread per group item
__global__ void k_group_items(DevProblem p, const int64_t *group_ptr, const int64_t *gwalk_ptr,
                              const int32_t *nfull, const int32_t *npages, int64_t walk_base, const int64_t *hs128,
                              const int64_t *hs64, const int64_t *hsg, int64_t n_all, FwdItem *items128,
                              int32_t *order) {
  const int BH = p.batch * p.heads;
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= hsg[BH]) return;
  const int bh = slot_of_index(hsg, BH, t);
  const int g = p.per_head ? bh : 0;
  const int64_t k = t - hsg[bh], gi = group_ptr[g] + k;
  FwdItem x{};
  x.walk_off = walk_base + gwalk_ptr[gi];
  x.walk_len = int32_t(gwalk_ptr[gi + 1] - gwalk_ptr[gi]);
  x.bh = bh;
  x.q = ~int32_t(gi);
  x.n_full = nfull[gi];
  x.n_pages = npages[gi];
  x.c_q = kBlockRows;
  const int64_t idx = hs128[bh + 1] + hsg[bh] + k;
  items128[idx] = x;
  order[launch_position(idx + hs64[bh], n_all, p.xcd_chunk)] = int32_t(idx);
}

int blocks_for(int64_t n, int threads) { return int((n + threads - 1) / threads); }

}  // namespace

kpage_status build_forward_device(const DevProblem &p, int align64, int align128, bool grouped, hipStream_t st,
                                  const DevAlloc &alloc, DevFwdTables *t, std::string *err) {
  const int64_t GQ = int64_t(p.slots) * p.n_q, GK = int64_t(p.slots) * p.n_kv;
  const int64_t BHQ = int64_t(p.batch) * p.heads * p.n_q;
  const int64_t n_pages = p.seq_kv / kPageRows;
  auto a32 = [&](int64_t n) { return static_cast<int32_t *>(alloc(size_t(std::max<int64_t>(n, 1)) * 4)); };
  auto a64 = [&](int64_t n) { return static_cast<int64_t *>(alloc(size_t(std::max<int64_t>(n, 1)) * 8)); };
  Summary *d_sum = static_cast<Summary *>(alloc(sizeof(Summary)));
  int32_t *owner = a32(int64_t(p.slots) * n_pages);
  t->page_block = owner;
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
  // duplicate-check bitmap, when it fits in 256 MiB (else the quadratic check)
  const int64_t seen_words = GQ * ((p.n_kv + 31) / 32);
  uint32_t *seen = seen_words * 4 <= (int64_t(256) << 20) ? static_cast<uint32_t *>(alloc(size_t(seen_words) * 4)) : nullptr;
  hipLaunchKernelGGL(k_count, dim3(blocks_for(GQ, TB)), dim3(TB), 0, st, p, align64, align128, t->route, t->nfull,
                     t->unpadded, len, d_sum, seen);
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
  int64_t *head_starts = static_cast<int64_t *>(alloc(size_t(2) * (size_t(p.batch) * p.heads + 1) * 8));
  unsigned long long *keys = static_cast<unsigned long long *>(alloc(size_t(std::max<int64_t>(BHQ, 1)) * 8 * 3));
  if (!t->walk || !t->pages || !t->valid || !t->q64_queue || !t->q128_queue || !head_starts || !keys) {
    *err = "device allocation failed while planning";
    return KPAGE_ERR_OOM;
  }
  hipLaunchKernelGGL(k_fill_walks, dim3(blocks_for(GQ, TB)), dim3(TB), 0, st, p, t->route, t->walk_ptr, t->walk,
                     t->pages, t->valid);
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
  // group items (the host planner's build_groups)
  const int BH = p.batch * p.heads;
  const int64_t W = (n_pages + 63) / 64;
  uint8_t *in_group = nullptr;
  int64_t *d_hsg = nullptr, *d_gptr = nullptr, *d_gwptr = nullptr;
  t->g_group_ptr.assign(size_t(p.slots) + 1, 0);
  t->g_walk_ptr.assign(1, 0);
  if (grouped && W <= kGroupMaxWords) {
    int32_t *cand = a32(GQ), *n_cand = a32(p.slots);
    if (!cand || !n_cand) {
      *err = "device allocation failed while planning";
      return KPAGE_ERR_OOM;
    }
    hipLaunchKernelGGL(k_group_cands, dim3(p.slots), dim3(kScanThreads), 0, st, p, t->route, t->unpadded, cand,
                       n_cand);
    std::vector<int32_t> hc(static_cast<size_t>(p.slots));
    KP_CHECK(hipMemcpyAsync(hc.data(), n_cand, hc.size() * 4, hipMemcpyDeviceToHost, st));
    KP_CHECK(hipStreamSynchronize(st));
    // slots with fewer than 2 or more than kGroupMaxCands candidates form no group
    std::vector<int64_t> coff(size_t(p.slots) + 1, 0);
    int max_nc = 0;
    for (int g = 0; g < p.slots; ++g) {
      if (hc[size_t(g)] < 2 || hc[size_t(g)] > kGroupMaxCands) hc[size_t(g)] = 0;
      coff[size_t(g) + 1] = coff[size_t(g)] + hc[size_t(g)];
      max_nc = std::max(max_nc, hc[size_t(g)]);
    }
    const int64_t n_cand_all = coff[size_t(p.slots)];
    // no slot groups when all the page bitsets together pass the limit (as on the host)
    if (n_cand_all > 0 && n_cand_all * W <= kGroupMaxBitsetWords) {
      int64_t *d_coff = a64(p.slots + 1);
      int32_t *d_nc = a32(p.slots);
      unsigned long long *bits = static_cast<unsigned long long *>(alloc(size_t(n_cand_all * W) * 8));
      int32_t *gmem = a32(n_cand_all * kGroupMembers), *gunion = a32(n_cand_all);
      int32_t *gcount = a32(p.slots), *gmembers = a32(p.slots);
      if (!d_coff || !d_nc || !bits || !gmem || !gunion || !gcount || !gmembers) {
        *err = "device allocation failed while planning";
        return KPAGE_ERR_OOM;
      }
      KP_CHECK(hipMemcpyAsync(d_coff, coff.data(), coff.size() * 8, hipMemcpyHostToDevice, st));
      KP_CHECK(hipMemcpyAsync(d_nc, hc.data(), hc.size() * 4, hipMemcpyHostToDevice, st));
      KP_CHECK(hipMemsetAsync(bits, 0, size_t(n_cand_all * W) * 8, st));
      hipLaunchKernelGGL(k_group_bits, dim3(unsigned(n_cand_all)), dim3(256), 0, st, p, t->walk_ptr, t->walk,
                         t->unpadded, cand, d_coff, int(W), bits);
      const size_t lds = size_t(2 * W) * 8 + size_t((max_nc + 7) / 8) * 8;
      hipLaunchKernelGGL(k_group_greedy, dim3(p.slots), dim3(kGroupThreads), lds, st, p, t->unpadded, cand, d_nc,
                         d_coff, int(W), bits, gmem, gunion, gcount, gmembers);
      KP_CHECK(hipGetLastError());
      std::vector<int32_t> hgc(static_cast<size_t>(p.slots)), hgm(static_cast<size_t>(p.slots)),
          hgu(static_cast<size_t>(n_cand_all));
      KP_CHECK(hipMemcpyAsync(hgc.data(), gcount, hgc.size() * 4, hipMemcpyDeviceToHost, st));
      KP_CHECK(hipMemcpyAsync(hgm.data(), gmembers, hgm.size() * 4, hipMemcpyDeviceToHost, st));
      KP_CHECK(hipMemcpyAsync(hgu.data(), gunion, hgu.size() * 4, hipMemcpyDeviceToHost, st));
      KP_CHECK(hipStreamSynchronize(st));
      int64_t n_mem_slot = 0;
      for (int g = 0; g < p.slots; ++g) {
        t->g_group_ptr[size_t(g) + 1] = t->g_group_ptr[size_t(g)] + hgc[size_t(g)];
        for (int k = 0; k < hgc[size_t(g)]; ++k)
          t->g_walk_ptr.push_back(t->g_walk_ptr.back() + (int64_t(hgu[size_t(coff[size_t(g)] + k)]) + 3) / 4 * 4);
      }
      t->n_groups = t->g_group_ptr[size_t(p.slots)];
      if (t->n_groups > 0) {
        const int64_t gw_total = t->g_walk_ptr.back();
        std::vector<int64_t> hsg(size_t(BH) + 1, 0);
        for (int bh = 0; bh < BH; ++bh) {
          const int g = p.per_head ? bh : 0;
          hsg[size_t(bh) + 1] = hsg[size_t(bh)] + (t->g_group_ptr[size_t(g) + 1] - t->g_group_ptr[size_t(g)]);
          n_mem_slot += hgm[size_t(g)];
        }
        t->n_gitems = hsg[size_t(BH)];
        t->n_members = n_mem_slot;
        d_gptr = a64(p.slots + 1);
        d_gwptr = a64(t->n_groups + 1);
        d_hsg = a64(BH + 1);
        t->groups = static_cast<FwdGroup *>(alloc(size_t(t->n_groups) * sizeof(FwdGroup)));
        t->g_members = a32(t->n_groups * kGroupMembers);
        t->g_nfull = a32(t->n_groups);
        t->g_npages = a32(t->n_groups);
        t->g_walk = a32(gw_total);
        t->g_valid = static_cast<uint32_t *>(alloc(size_t(2 * gw_total) * 4));
        in_group = static_cast<uint8_t *>(alloc(size_t(GQ)));
        // the union walks and their words follow the plan's walks and words
        int32_t *pages2 = a32(h.walk_total + gw_total);
        uint32_t *valid2 = static_cast<uint32_t *>(alloc(size_t(h.walk_total / 2 + 2 * gw_total) * 4));
        if (!d_gptr || !d_gwptr || !d_hsg || !t->groups || !t->g_members || !t->g_nfull || !t->g_npages ||
            !t->g_walk || !t->g_valid || !in_group || !pages2 || !valid2) {
          *err = "device allocation failed while planning";
          return KPAGE_ERR_OOM;
        }
        KP_CHECK(hipMemcpyAsync(d_gptr, t->g_group_ptr.data(), t->g_group_ptr.size() * 8, hipMemcpyHostToDevice, st));
        KP_CHECK(hipMemcpyAsync(d_gwptr, t->g_walk_ptr.data(), t->g_walk_ptr.size() * 8, hipMemcpyHostToDevice, st));
        KP_CHECK(hipMemcpyAsync(d_hsg, hsg.data(), hsg.size() * 8, hipMemcpyHostToDevice, st));
        KP_CHECK(hipMemsetAsync(in_group, 0, size_t(GQ), st));
        if (h.walk_total > 0) {
          KP_CHECK(hipMemcpyAsync(pages2, t->pages, size_t(h.walk_total) * 4, hipMemcpyDeviceToDevice, st));
          KP_CHECK(hipMemcpyAsync(valid2, t->valid, size_t(h.walk_total / 2) * 4, hipMemcpyDeviceToDevice, st));
        }
        t->pages = pages2;
        t->valid = valid2;
        hipLaunchKernelGGL(k_group_walks, dim3(unsigned(t->n_groups)), dim3(kScanThreads), size_t(W) * 8, st, p,
                           t->page_block, t->walk_ptr, t->walk, t->unpadded, cand, d_coff, int(W), bits, gmem, d_gptr,
                           d_gwptr, h.walk_total, h.walk_total / 2, t->groups, t->g_members, t->g_nfull,
                           t->g_npages, t->g_walk, t->pages, t->valid, t->g_valid, in_group);
        KP_CHECK(hipGetLastError());
      }
    }
  }
  const int64_t n_items128 = int64_t(h.n_q128) + t->n_gitems;
  const int64_t n_items64 = int64_t(h.n_q64) - t->n_members + h.n_zero;
  const int64_t n_all = n_items128 + n_items64;
  t->items128 = static_cast<FwdItem *>(alloc(size_t(std::max<int64_t>(n_items128, 1)) * sizeof(FwdItem)));
  t->items64 = static_cast<FwdItem *>(alloc(size_t(std::max<int64_t>(n_items64, 1)) * sizeof(FwdItem)));
  t->order = a32(n_all);
  if (!t->items128 || !t->items64 || !t->order) {
    *err = "device allocation failed while planning";
    return KPAGE_ERR_OOM;
  }
  int64_t *hs128 = head_starts, *hs64 = head_starts + (int64_t(BH) + 1);
  hipLaunchKernelGGL(k_items, dim3(1), dim3(kScanThreads), 0, st, p, t->route, t->nfull, t->unpadded, t->walk_ptr, d_sum,
                     in_group, d_hsg, t->n_members, t->items128, t->items64, hs128, hs64, t->order);
  if (t->n_gitems > 0)
    hipLaunchKernelGGL(k_group_items, dim3(blocks_for(t->n_gitems, TB)), dim3(TB), 0, st, p, d_gptr,
                       d_gwptr, t->g_nfull, t->g_npages, h.walk_total, hs128, hs64, d_hsg, n_all,
                       t->items128, t->order);
  hipLaunchKernelGGL(k_fwd_tails, dim3(kXcds), dim3(kFwdTail), 0, st, t->order, t->items128, t->items64, n_all);
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


// ---------------------------------------------------------------------------------
// Backward tables (section 3.3).  Per graph slot: owners (3.3.1), the owner x Q-block
// bitmap compacted into reverse-Q lists, Q-page walks with dummies to a multiple of 8
// pages (3.3.2), one 64-bit adjacency word per step (3.3.3, eq. 6), the work order of
// section 3.4 (descending step count, then (bh, owner)) and the pages outside every
// block footprint.  Bitmaps: edge[slot][q][n_kv / 32] (a selected pair with c_q > 0
// and c_k > 0), own_q[slot][owner][n_q / 32] (the owner holds a page of a block that q
// selects).
namespace {

struct BwdSummary {
  int64_t n_own, revq_total, qwalk_total, uncovered_total;
  int32_t max_uncovered, pad;
  unsigned long long useful_check;
  int64_t n_witems, n_part, n_red;  // per slot (shared graph) or in all: items, partial slots, reduces
};

// Q groups (section 3.3.2): the query blocks [lo, hi) of group grp of an owner.  An
// owner whose reverse neighbourhood holds more than gsz query blocks is cut into the
// ranges [grp gsz, (grp + 1) gsz); a smaller one keeps its whole list in group 0.
__device__ __forceinline__ void group_range(bool split, int grp, int gsz, int n_q, int *lo, int *hi) {
  if (split) {
    *lo = grp * gsz;
    *hi = min(n_q, (grp + 1) * gsz);
  } else {
    *lo = grp == 0 ? 0 : n_q;
    *hi = n_q;
  }
}

// bits [lo, hi) of word w of a query-block bitset
__device__ __forceinline__ uint32_t range_word(int w, int lo, int hi) {
  const int a = max(lo - 32 * w, 0), b = min(hi - 32 * w, 32);
  if (b <= a) return 0u;
  const uint32_t upto = b == 32 ? ~0u : (1u << b) - 1u;
  return upto & ~((1u << a) - 1u);
}

__device__ __forceinline__ uint32_t page_mask(int c, int j) {
  return (j + 1) * kPageRows <= c ? kFullMask : tail_mask(c);
}

// own_info packing: blocks in the owner | pages in the owner << 16
__device__ __forceinline__ int32_t pack_info(int blocks, int pages) { return blocks | (pages << 16); }

// Reverse neighbourhood of every K/V block: the query blocks with c_q > 0 that select it,
// as a bitset of nqw words per (slot, block); one thread per (slot, query block).
__global__ void k_block_revq(DevProblem p, int nqw, uint32_t *rev_k) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(p.slots) * p.n_q) return;
  const int g = int(i / p.n_q), q = int(i % p.n_q);
  if (p.q_valid[i] == 0) return;
  const int64_t a = p.q2k_ptr[int64_t(g) * (p.n_q + 1) + q], b = p.q2k_ptr[int64_t(g) * (p.n_q + 1) + q + 1];
  for (int64_t e = a; e < b; ++e) {
    const int k = p.q2k_idx[e];
    if (p.kv_valid[int64_t(g) * p.n_kv + k] == 0) continue;
    atomicOr(&rev_k[(int64_t(g) * p.n_kv + k) * nqw + (q >> 5)], 1u << (q & 31));
  }
}

__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) {
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned lo = __shfl_xor((unsigned)v, off), hi = __shfl_xor((unsigned)(v >> 32), off);
    const unsigned long long o = ((unsigned long long)hi << 32) | lo;
    v = o < v ? o : v;
  }
  return v;
}

// Owners of slot blockIdx.x: every full block is an owner of its own, in block order.
// The partial blocks then fill owners one at a time: the smallest unplaced one opens an
// owner, and while one fits, the fitting block that adds the fewest query blocks to the
// owner's reverse neighbourhood joins it (ties to the smaller index).  The candidates of
// each choice are scored in parallel, one or more per thread, and the choice is the
// minimum of (new query blocks, block index) over the workgroup.  Dynamic LDS: the
// owner's covered query blocks (nqw words), then one placed bit per block (nkw words).
__global__ __launch_bounds__(kScanThreads) void k_owners(DevProblem p, const uint32_t *rev_k, int nqw, int nkw,
                                                         int32_t *owner_of, int32_t *pos_of, int32_t *own_info,
                                                         int32_t *n_own) {
  __shared__ int64_t lds[kScanThreads];
  __shared__ unsigned long long s_min[kScanThreads / 64];
  __shared__ int s_pick;
  extern __shared__ uint32_t s_dyn[];
  uint32_t *covered = s_dyn;
  uint32_t *placed = s_dyn + nqw;
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t gb = int64_t(g) * p.n_kv;
  const int32_t *ck = p.kv_valid + gb;
  const uint32_t *rk = rev_k + gb * nqw;
  for (int i = tid; i < nkw; i += kScanThreads) placed[i] = 0;
  int64_t carry = 0;
  for (int base = 0; base < p.n_kv; base += kScanThreads) {
    const int k = base + tid;
    const int c = k < p.n_kv ? ck[k] : 0;
    int64_t total;
    const int64_t pre = carry + block_scan(c == kBlockRows ? 1 : 0, lds, &total);
    if (k < p.n_kv && c == kBlockRows) {
      owner_of[gb + k] = int32_t(pre);
      pos_of[gb + k] = 0;
      own_info[gb + pre] = pack_info(1, kOwnerSlots);
    } else if (k < p.n_kv && c == 0) {
      owner_of[gb + k] = -1;
      pos_of[gb + k] = 0;
    }
    carry += total;
  }
  auto is_partial = [&](int k) { const int c = ck[k]; return c > 0 && c < kBlockRows; };
  auto is_placed = [&](int k) { return (placed[k >> 5] >> (k & 31)) & 1u; };
  int n = int(carry);
  int scan = 0;  // every partial block below it is placed
  for (;;) {
    __syncthreads();
    if (tid == 0) {
      while (scan < p.n_kv && !(is_partial(scan) && !is_placed(scan))) ++scan;
      s_pick = scan < p.n_kv ? scan : -1;
    }
    __syncthreads();
    const int seed = s_pick;
    if (seed < 0) break;
    scan = seed + 1;
    const int cur = n++;
    int used = 0, blocks = 0;
    for (int i = tid; i < nqw; i += kScanThreads) covered[i] = 0;
    __syncthreads();
    int k = seed;
    for (;;) {  // place k, then look for the next block
      if (tid == 0) {
        owner_of[gb + k] = cur;
        pos_of[gb + k] = used;
        placed[k >> 5] |= 1u << (k & 31);
      }
      for (int i = tid; i < nqw; i += kScanThreads) covered[i] |= rk[int64_t(k) * nqw + i];
      used += pages_of(ck[k]);
      ++blocks;
      __syncthreads();
      const int free_slots = kOwnerSlots - used;
      unsigned long long best = ~0ull;
      if (free_slots > 0) {
        for (int j = seed + 1 + tid; j < p.n_kv; j += kScanThreads) {
          if (!is_partial(j) || is_placed(j) || pages_of(ck[j]) > free_slots) continue;
          unsigned new_q = 0;
          for (int i = 0; i < nqw; ++i) new_q += __popc(rk[int64_t(j) * nqw + i] & ~covered[i]);
          const unsigned long long key = ((unsigned long long)new_q << 32) | unsigned(j);
          best = key < best ? key : best;
        }
      }
      best = wave_min_u64(best);
      if ((tid & 63) == 0) s_min[tid >> 6] = best;
      __syncthreads();
      if (tid == 0) {
        unsigned long long m = ~0ull;
        for (int w = 0; w < kScanThreads / 64; ++w) m = s_min[w] < m ? s_min[w] : m;
        s_pick = m == ~0ull ? -1 : int(m & 0xFFFFFFFFu);
      }
      __syncthreads();
      if (s_pick < 0) break;
      k = s_pick;
    }
    if (tid == 0) own_info[gb + cur] = pack_info(blocks, used);
  }
  if (tid == 0) n_own[g] = n;
}

// pages of slot blockIdx.x outside every block footprint: count, or (unc != NULL)
// write them in page order from unc_ptr[slot]
__global__ __launch_bounds__(kScanThreads) void k_uncovered(DevProblem p, const int32_t *page_block, int32_t *count,
                                                            const int64_t *unc_ptr, int32_t *unc) {
  __shared__ int64_t lds[kScanThreads];
  const int g = blockIdx.x;
  const int64_t n_pages = p.seq_kv / kPageRows;
  const int32_t *pb = page_block + int64_t(g) * n_pages;
  int64_t carry = unc ? unc_ptr[g] : 0;
  for (int64_t base = 0; base < n_pages; base += kScanThreads) {
    const int64_t pg = base + threadIdx.x;
    const int hole = pg < n_pages && pb[pg] < 0 ? 1 : 0;
    int64_t total;
    const int64_t pre = carry + block_scan(hole, lds, &total);
    if (unc && hole) unc[pre] = int32_t(pg);
    carry += total;
  }
  if (!unc && threadIdx.x == 0) count[g] = int32_t(carry);
}

// owner_ptr and uncovered_ptr over slots
__global__ __launch_bounds__(kScanThreads) void k_slot_scans(int G, const int32_t *n_own, const int32_t *n_unc,
                                                             int64_t *owner_ptr, int64_t *unc_ptr, BwdSummary *s) {
  __shared__ int64_t lds[kScanThreads];
  int64_t c1 = 0, c2 = 0;
  int mx = 0;
  for (int base = 0; base < G; base += kScanThreads) {
    const int g = base + threadIdx.x;
    const int64_t a = g < G ? n_own[g] : 0, b = g < G ? n_unc[g] : 0;
    int64_t t1, t2;
    const int64_t p1 = c1 + block_scan(a, lds, &t1);
    const int64_t p2 = c2 + block_scan(b, lds, &t2);
    if (g < G) {
      owner_ptr[g] = p1;
      unc_ptr[g] = p2;
    }
    mx = max(mx, int(b));
    c1 += t1;
    c2 += t2;
  }
  atomicMax(&s->max_uncovered, mx);
  if (threadIdx.x == 0) {
    owner_ptr[G] = c1;
    unc_ptr[G] = c2;
    s->n_own = c1;
    s->uncovered_total = c2;
  }
}

// per (slot, query block): edge bits of its row, its bit in the owner x Q bitmap of
// every owner it reaches, and its bit in the slot's full-query-block mask
__global__ void k_edges(DevProblem p, const int32_t *owner_of, int nkw, int nqw, uint32_t *edge, uint32_t *own_q,
                        uint32_t *fullq) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(p.slots) * p.n_q) return;
  const int g = int(i / p.n_q), q = int(i % p.n_q);
  const int cq = p.q_valid[i];
  const uint32_t qbit = 1u << (q & 31);
  if (cq == kBlockRows) atomicOr(&fullq[int64_t(g) * nqw + (q >> 5)], qbit);
  if (cq == 0) return;
  const int64_t a = p.q2k_ptr[int64_t(g) * (p.n_q + 1) + q], b = p.q2k_ptr[int64_t(g) * (p.n_q + 1) + q + 1];
  uint32_t *row = edge + i * nkw;  // written by this thread only
  for (int64_t e = a; e < b; ++e) {
    const int k = p.q2k_idx[e];
    if (p.kv_valid[int64_t(g) * p.n_kv + k] == 0) continue;
    row[k >> 5] |= 1u << (k & 31);
    const int t = owner_of[int64_t(g) * p.n_kv + k];
    atomicOr(&own_q[(int64_t(g) * p.n_kv + t) * nqw + (q >> 5)], qbit);
  }
}

// per (slot, owner): for each Q group, the reverse-Q count and the Q-walk length (full
// query blocks first, 8 pages each, then the pages of partial ones, padded to a multiple
// of 8), at (owner, group) = tg * ng + group; the owner's slot, whether it is split into
// groups, its alignment flag and the empty page slots of the owner table
__global__ void k_owner_counts(DevProblem p, const int64_t *owner_ptr, const int32_t *n_own, const int32_t *own_info,
                               const uint32_t *own_q, const uint32_t *fullq, int nqw, int gsz, int ng, int64_t *rcount,
                               int64_t *qlen, int32_t *owner_slot, uint8_t *split_of, uint8_t *aligned,
                               int32_t *owners, uint32_t *kmask) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(p.slots) * p.n_kv) return;
  const int g = int(i / p.n_kv), t = int(i % p.n_kv);
  if (t >= n_own[g]) return;
  const int64_t tg = owner_ptr[g] + t;
  const uint32_t *bm = own_q + i * nqw;
  const uint32_t *fm = fullq + int64_t(g) * nqw;
  int64_t r_all = 0;
  for (int w = 0; w < nqw; ++w) r_all += __popc(bm[w]);
  const bool split = r_all > gsz;
  for (int grp = 0; grp < ng; ++grp) {
    int lo, hi;
    group_range(split, grp, gsz, p.n_q, &lo, &hi);
    int64_t r = 0, pages = 0;
    for (int w = lo >> 5; w < nqw && 32 * w < hi; ++w) {
      const uint32_t bits = bm[w] & range_word(w, lo, hi);
      r += __popc(bits);
      pages += int64_t(kOwnerSlots) * __popc(bits & fm[w]);
      uint32_t part = bits & ~fm[w];
      while (part) {
        const int b = __ffs(part) - 1;
        part &= part - 1;
        pages += pages_of(p.q_valid[int64_t(g) * p.n_q + 32 * w + b]);
      }
    }
    rcount[tg * ng + grp] = r;
    qlen[tg * ng + grp] = (pages + kOwnerSlots - 1) / kOwnerSlots * kOwnerSlots;
  }
  owner_slot[tg] = g;
  split_of[tg] = split ? 1 : 0;
  const int32_t info = own_info[i];
  const int blocks = info & 0xFFFF, np = info >> 16;
  aligned[tg] = (blocks == 1 && np == kOwnerSlots) ? 1 : 0;
  for (int j = np; j < kOwnerSlots; ++j) {
    owners[tg * kOwnerSlots + j] = -1;
    kmask[tg * kOwnerSlots + j] = 0u;
  }
}

// per (slot, block): the block's pages and row masks in its owner
__global__ void k_owner_pages(DevProblem p, const int32_t *owner_of, const int32_t *pos_of, const int64_t *owner_ptr,
                              int32_t *owners, uint32_t *kmask) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(p.slots) * p.n_kv) return;
  const int t = owner_of[i];
  if (t < 0) return;
  const int g = int(i / p.n_kv), k = int(i % p.n_kv);
  const int c = p.kv_valid[i];
  const int64_t at = (owner_ptr[g] + t) * kOwnerSlots + pos_of[i];
  const int32_t pg0 = int32_t(kv_off(p, g, k) / kPageRows);
  for (int j = 0; j < pages_of(c); ++j) {
    owners[at + j] = pg0 + j;
    kmask[at + j] = page_mask(c, j);
  }
}

// revq_ptr and qwalk_ptr over all (owner, group) pairs
__global__ __launch_bounds__(kScanThreads) void k_owner_scans(const BwdSummary *s, int ng, const int64_t *rcount,
                                                              const int64_t *qlen, int64_t *revq_ptr,
                                                              int64_t *qwalk_ptr, BwdSummary *out) {
  __shared__ int64_t lds[kScanThreads];
  const int64_t n = s->n_own * ng;
  int64_t c1 = 0, c2 = 0;
  for (int64_t base = 0; base < n; base += kScanThreads) {
    const int64_t t = base + threadIdx.x;
    int64_t t1, t2;
    const int64_t p1 = c1 + block_scan(t < n ? rcount[t] : 0, lds, &t1);
    const int64_t p2 = c2 + block_scan(t < n ? qlen[t] : 0, lds, &t2);
    if (t < n) {
      revq_ptr[t] = p1;
      qwalk_ptr[t] = p2;
    }
    c1 += t1;
    c2 += t2;
  }
  if (threadIdx.x == 0) {
    revq_ptr[n] = c1;
    qwalk_ptr[n] = c2;
    out->revq_total = c1;
    out->qwalk_total = c2;
  }
}

// per (owner, group): reverse-Q list (ascending q) and Q-page walk
__global__ void k_owner_fill(DevProblem p, int64_t n_own, int gsz, int ng, const int64_t *owner_ptr,
                             const int32_t *owner_slot, const uint8_t *split_of, const uint32_t *own_q,
                             const uint32_t *fullq, int nqw, const int64_t *revq_ptr, const int64_t *qwalk_ptr,
                             int32_t *revq, int32_t *qwalk, int32_t *qpages) {
  const int64_t wi = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (wi >= n_own * ng) return;
  const int64_t tg = wi / ng;
  const int grp = int(wi % ng);
  const int g = owner_slot[tg];
  const int64_t t = tg - owner_ptr[g];
  int lo, hi;
  group_range(split_of[tg] != 0, grp, gsz, p.n_q, &lo, &hi);
  const uint32_t *bm = own_q + (int64_t(g) * p.n_kv + t) * nqw;
  const uint32_t *fm = fullq + int64_t(g) * nqw;
  const int w0 = lo >> 5, w1 = min(nqw, (hi + 31) >> 5);
  int64_t r = revq_ptr[wi];
  for (int w = w0; w < w1; ++w)
    for (uint32_t bits = bm[w] & range_word(w, lo, hi); bits; bits &= bits - 1) revq[r++] = 32 * w + __ffs(bits) - 1;
  int64_t pos = qwalk_ptr[wi];
  const int64_t end = qwalk_ptr[wi + 1];
  int32_t first = -1;
  auto emit = [&](int32_t qp) {
    if (first < 0) first = qp;
    qwalk[pos] = qp;
    qpages[pos] = qp >= 0 ? qp : first;
    ++pos;
  };
  for (int w = w0; w < w1; ++w)  // full query blocks: all 8 pages
    for (uint32_t bits = bm[w] & fm[w] & range_word(w, lo, hi); bits; bits &= bits - 1) {
      const int q = 32 * w + __ffs(bits) - 1;
      for (int j = 0; j < kOwnerSlots; ++j) emit(kOwnerSlots * q + j);
    }
  for (int w = w0; w < w1; ++w)  // partial query blocks: their valid pages
    for (uint32_t bits = bm[w] & ~fm[w] & range_word(w, lo, hi); bits; bits &= bits - 1) {
      const int q = 32 * w + __ffs(bits) - 1;
      const int np = pages_of(p.q_valid[int64_t(g) * p.n_q + q]);
      for (int j = 0; j < np; ++j) emit(kOwnerSlots * q + j);
    }
  while (pos < end) emit(-1);
}

// largest i in [0, n) with ptr[i] <= x (ptr non-decreasing, ptr[0] <= x)
__device__ __forceinline__ int64_t upper_index(const int64_t *ptr, int64_t n, int64_t x) {
  int64_t lo = 0, hi = n - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (ptr[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// per 8-page step: adjacency word, bit 8 j + i = (Q page j of the step, owner page i)
// belong to a selected block pair; pair count of the step for the visited-pair check
__global__ void k_adj(DevProblem p, const int32_t *page_block, int64_t n_own, int ng, int64_t n_steps,
                      unsigned long long mult, const int32_t *owner_slot, const int64_t *qwalk_ptr,
                      const int32_t *owners, const int32_t *qwalk, const uint32_t *edge, int nkw, uint64_t *adj,
                      BwdSummary *s) {
  __shared__ unsigned long long acc;
  if (threadIdx.x == 0) acc = 0;
  __syncthreads();
  const int64_t st = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (st < n_steps) {
    const int64_t pos = int64_t(kOwnerSlots) * st;
    const int64_t tg = upper_index(qwalk_ptr, n_own * ng, pos) / ng;
    const int g = owner_slot[tg];
    const int64_t n_pages = p.seq_kv / kPageRows;
    int kb[kOwnerSlots];
    int kcount[kOwnerSlots];
    for (int i = 0; i < kOwnerSlots; ++i) {
      const int32_t kp = owners[tg * kOwnerSlots + i];
      kb[i] = -1;
      kcount[i] = 0;
      if (kp < 0) continue;
      const int k = page_block[int64_t(g) * n_pages + kp];
      kb[i] = k;
      kcount[i] = __popc(page_mask(p.kv_valid[int64_t(g) * p.n_kv + k], int(kp - kv_off(p, g, k) / kPageRows)));
    }
    uint64_t word = 0;
    unsigned long long pairs = 0;
    for (int j = 0; j < kOwnerSlots; ++j) {
      const int32_t qp = qwalk[pos + j];
      if (qp < 0) continue;
      const int qb = qp / kOwnerSlots;
      const int qcount = __popc(page_mask(p.q_valid[int64_t(g) * p.n_q + qb], qp % kOwnerSlots));
      const uint32_t *row = edge + (int64_t(g) * p.n_q + qb) * nkw;
      for (int i = 0; i < kOwnerSlots; ++i) {
        if (kb[i] < 0 || !((row[kb[i] >> 5] >> (kb[i] & 31)) & 1u)) continue;
        word |= uint64_t(1) << (kOwnerSlots * j + i);
        pairs += (unsigned long long)qcount * (unsigned long long)kcount[i];
      }
    }
    adj[st] = word;
    if (pairs) atomicAdd(&acc, mult * pairs);
  }
  __syncthreads();
  if (threadIdx.x == 0 && acc) atomicAdd(&s->useful_check, acc);
}

// Work items (section 3.3.2): every (owner, group) with a non-empty Q walk, plus group 0
// of an owner with none (it still writes its zero gradients), in (owner, group) order.
// One workgroup scans the n_own * ng pairs: item_pos[w] = index of pair w among the
// items (item_pos[n] = their number), item_w[index] = w.  Then per owner with more than
// one item: consecutive fp32 partial slots in group order (part_base) and one reduce
// entry (red_pos), in owner order.  Counts per graph slot for a shared graph (each
// (b, h) repeats them), over all slots otherwise.
__global__ __launch_bounds__(kScanThreads) void k_item_scan(const BwdSummary *s, int ng, const int64_t *qwalk_ptr,
                                                            int64_t *item_pos, int64_t *item_w, int64_t *part_base,
                                                            int64_t *red_pos, BwdSummary *out) {
  __shared__ int64_t lds[kScanThreads];
  const int64_t n_own = s->n_own, n = n_own * ng;
  int64_t c = 0;
  for (int64_t base = 0; base < n; base += kScanThreads) {
    const int64_t w = base + threadIdx.x;
    bool flag = false;
    if (w < n) {
      const int64_t tg = w / ng;
      const bool empty_owner = qwalk_ptr[(tg + 1) * ng] == qwalk_ptr[tg * ng];
      flag = qwalk_ptr[w + 1] > qwalk_ptr[w] || (w % ng == 0 && empty_owner);
    }
    int64_t tot;
    const int64_t pos = c + block_scan(flag ? 1 : 0, lds, &tot);
    if (w < n) {
      item_pos[w] = pos;
      if (flag) item_w[pos] = w;
    }
    c += tot;
  }
  if (threadIdx.x == 0) item_pos[n] = c;
  __syncthreads();
  int64_t cp = 0, cr = 0;
  for (int64_t base = 0; base < n_own; base += kScanThreads) {
    const int64_t tg = base + threadIdx.x;
    const int64_t cnt = tg < n_own ? item_pos[(tg + 1) * ng] - item_pos[tg * ng] : 0;
    int64_t tp, tr;
    const int64_t pp = cp + block_scan(cnt > 1 ? cnt : 0, lds, &tp);
    const int64_t pr = cr + block_scan(cnt > 1 ? 1 : 0, lds, &tr);
    if (tg < n_own) {
      part_base[tg] = pp;
      red_pos[tg] = pr;
    }
    cp += tp;
    cr += tr;
  }
  if (threadIdx.x == 0) {
    out->n_witems = c;
    out->n_part = cp;
    out->n_red = cr;
  }
}

// per work item f: queue sort key (steps descending, then f) and the launch item at its
// XCD position, with its fp32 partial slot when its owner has more than one item
__global__ void k_bwd_items(DevProblem p, int ng, int64_t n_w, int64_t n_items, int64_t n_part_slot,
                            const int64_t *qwalk_ptr, const int32_t *owner_slot, const int64_t *item_pos,
                            const int64_t *item_w, const int64_t *part_base, unsigned long long *keys,
                            BwdItem *items) {
  const int64_t f = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (f >= n_items) return;
  const int64_t w = item_w[p.per_head ? f : f % n_w];
  const int64_t tg = w / ng;
  const int bh = p.per_head ? owner_slot[tg] : int(f / n_w);
  const int32_t steps = int32_t((qwalk_ptr[w + 1] - qwalk_ptr[w]) / kOwnerSlots);
  keys[f] = ((unsigned long long)(0x7FFFFFFF - steps) << 32) | (unsigned long long)(uint32_t)f;
  const int64_t first = item_pos[tg * ng], cnt = item_pos[(tg + 1) * ng] - first;
  BwdItem x{};
  x.qwalk_off = qwalk_ptr[w];
  x.bh = bh;
  x.owner = int32_t(tg);
  x.n_steps = steps;
  x.partial = cnt > 1 ? int32_t((p.per_head ? 0 : int64_t(bh) * n_part_slot) + part_base[tg] + (item_pos[w] - first))
                      : -1;
  items[launch_position(f, n_items, p.xcd_chunk)] = x;
}

// reduce entries of the owners split over several items, in (bh, owner) order
__global__ void k_bwd_reduce_list(DevProblem p, int64_t n_own, int ng, int64_t n_part_slot, int64_t n_red_slot,
                                  const int32_t *owner_slot, const int64_t *item_pos, const int64_t *part_base,
                                  const int64_t *red_pos, int64_t n, BwdReduce *reduce) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t tg = p.per_head ? i : i % n_own;
  const int bh = p.per_head ? owner_slot[tg] : int(i / n_own);
  const int64_t cnt = item_pos[(tg + 1) * ng] - item_pos[tg * ng];
  if (cnt < 2) return;
  const int64_t at = (p.per_head ? 0 : int64_t(bh) * n_red_slot) + red_pos[tg];
  reduce[at] = BwdReduce{bh, int32_t(tg), int32_t((p.per_head ? 0 : int64_t(bh) * n_part_slot) + part_base[tg]),
                         int32_t(cnt)};
}

// The last bwd_tail_len(count) items of each XCD's launch sequence (positions 8 j + x)
// in descending step count, ties in their order: one workgroup per XCD sorts its tail
// in LDS (bitonic, over kMaxBwdTail keys), the same order as the host planner's.
__global__ __launch_bounds__(1024) void k_bwd_tails(BwdItem *items, int64_t n) {
  __shared__ unsigned long long key[kMaxBwdTail];
  __shared__ BwdItem buf[kMaxBwdTail];
  const int x = int(blockIdx.x);
  const int64_t cnt = n > x ? (n - x + kXcds - 1) / kXcds : 0;
  const int64_t t = bwd_tail_len(cnt);
  const int64_t j0 = cnt - t;
  for (int i = int(threadIdx.x); i < kMaxBwdTail; i += int(blockDim.x)) {
    if (i < t) {
      const BwdItem it = items[(j0 + i) * kXcds + x];
      buf[i] = it;
      key[i] = ((unsigned long long)(uint32_t)(0x7FFFFFFF - it.n_steps) << 32) | (unsigned long long)(uint32_t)i;
    } else {
      key[i] = ~0ull;
    }
  }
  __syncthreads();
  for (int k = 2; k <= kMaxBwdTail; k <<= 1)
    for (int h = k >> 1; h > 0; h >>= 1) {
      for (int i = int(threadIdx.x); i < kMaxBwdTail; i += int(blockDim.x)) {
        const int l = i ^ h;
        if (l > i) {
          const unsigned long long a = key[i], b = key[l];
          if ((a > b) == ((i & k) == 0)) {
            key[i] = b;
            key[l] = a;
          }
        }
      }
      __syncthreads();
    }
  for (int i = int(threadIdx.x); i < t; i += int(blockDim.x)) items[(j0 + i) * kXcds + x] = buf[uint32_t(key[i])];
}

__global__ void k_bwd_queue_out(DevProblem p, int ng, int64_t n_w, int64_t n_items, const int64_t *owner_ptr,
                                const int32_t *owner_slot, const int64_t *item_w, const unsigned long long *keys,
                                int32_t *queue) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n_items) return;
  const int64_t f = int64_t(keys[i] & 0xFFFFFFFFull);
  const int64_t w = item_w[p.per_head ? f : f % n_w];
  const int64_t tg = w / ng;
  const int g = owner_slot[tg];
  queue[2 * i] = p.per_head ? g : int(f / n_w);
  queue[2 * i + 1] = int32_t((tg - owner_ptr[g]) * ng + w % ng);
}

}  // namespace

kpage_status build_backward_device(const DevProblem &p, const int32_t *page_block, int q_group, hipStream_t st,
                                   const DevAlloc &alloc, DevBwdTables *t, std::string *err) {
  const int G = p.slots;
  const int gsz = q_group > 0 ? std::min(q_group, p.n_q) : p.n_q;
  const int ng = (p.n_q + gsz - 1) / gsz;
  t->n_groups = ng;
  const int64_t GK = int64_t(G) * p.n_kv, GQ = int64_t(G) * p.n_q;
  const int64_t n_pages = p.seq_kv / kPageRows;
  const int nkw = (p.n_kv + 31) / 32, nqw = (p.n_q + 31) / 32;
  const unsigned long long mult = p.per_head ? 1ull : (unsigned long long)p.batch * p.heads;
  // owner packing keeps the covered query blocks and one placed bit per block in LDS
  const size_t owners_lds = size_t(nqw + nkw) * 4;
  if (owners_lds > size_t(kOwnersLdsMax)) {
    *err = "too many query and key blocks for the GPU planner's owner packing";
    return KPAGE_ERR_UNSUPPORTED;
  }
  bool oom = false;
  auto A = [&](int64_t n, size_t elem) -> void * {
    void *q = alloc(size_t(std::max<int64_t>(n, 1)) * elem);
    if (!q) oom = true;
    return q;
  };
  BwdSummary *d_sum = static_cast<BwdSummary *>(A(1, sizeof(BwdSummary)));
  int32_t *owner_of = static_cast<int32_t *>(A(GK, 4));
  int32_t *pos_of = static_cast<int32_t *>(A(GK, 4));
  int32_t *own_info = static_cast<int32_t *>(A(GK, 4));
  int32_t *n_own = static_cast<int32_t *>(A(G, 4));
  int32_t *n_unc = static_cast<int32_t *>(A(G, 4));
  uint32_t *edge = static_cast<uint32_t *>(A(GQ * nkw, 4));
  uint32_t *own_q = static_cast<uint32_t *>(A(GK * nqw, 4));
  uint32_t *rev_k = static_cast<uint32_t *>(A(GK * nqw, 4));
  uint32_t *fullq = static_cast<uint32_t *>(A(int64_t(G) * nqw, 4));
  int64_t *rcount = static_cast<int64_t *>(A(GK * ng, 8));
  int64_t *qlen = static_cast<int64_t *>(A(GK * ng, 8));
  int32_t *owner_slot = static_cast<int32_t *>(A(GK, 4));
  uint8_t *split_of = static_cast<uint8_t *>(A(GK, 1));
  int64_t *item_pos = static_cast<int64_t *>(A(GK * ng + 1, 8));
  int64_t *item_w = static_cast<int64_t *>(A(GK * ng, 8));
  int64_t *part_base = static_cast<int64_t *>(A(GK, 8));
  int64_t *red_pos = static_cast<int64_t *>(A(GK, 8));
  // owner-indexed tables at their upper bound (at most one owner per block)
  t->owner_ptr = static_cast<int64_t *>(A(G + 1, 8));
  t->owners = static_cast<int32_t *>(A(GK * kOwnerSlots, 4));
  t->kmask = static_cast<uint32_t *>(A(GK * kOwnerSlots, 4));
  t->aligned = static_cast<uint8_t *>(A(GK, 1));
  t->revq_ptr = static_cast<int64_t *>(A(GK * ng + 1, 8));
  t->qwalk_ptr = static_cast<int64_t *>(A(GK * ng + 1, 8));
  t->uncovered_ptr = static_cast<int64_t *>(A(G + 1, 8));
  t->uncovered = static_cast<int32_t *>(A(int64_t(G) * n_pages, 4));
  if (oom) {
    *err = "device allocation failed while planning the backward";
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
  KP_CHECK(hipMemsetAsync(d_sum, 0, sizeof(BwdSummary), st));
  KP_CHECK(hipMemsetAsync(edge, 0, size_t(std::max<int64_t>(GQ * nkw, 1)) * 4, st));
  KP_CHECK(hipMemsetAsync(own_q, 0, size_t(std::max<int64_t>(GK * nqw, 1)) * 4, st));
  KP_CHECK(hipMemsetAsync(rev_k, 0, size_t(std::max<int64_t>(GK * nqw, 1)) * 4, st));
  KP_CHECK(hipMemsetAsync(fullq, 0, size_t(std::max<int64_t>(int64_t(G) * nqw, 1)) * 4, st));
  hipLaunchKernelGGL(k_block_revq, dim3(blocks_for(GQ, TB)), dim3(TB), 0, st, p, nqw, rev_k);
  hipLaunchKernelGGL(k_owners, dim3(G), dim3(kScanThreads), owners_lds, st, p, rev_k, nqw, nkw, owner_of, pos_of,
                     own_info, n_own);
  hipLaunchKernelGGL(k_uncovered, dim3(G), dim3(kScanThreads), 0, st, p, page_block, n_unc, nullptr, nullptr);
  hipLaunchKernelGGL(k_slot_scans, dim3(1), dim3(kScanThreads), 0, st, G, n_own, n_unc, t->owner_ptr,
                     t->uncovered_ptr, d_sum);
  hipLaunchKernelGGL(k_uncovered, dim3(G), dim3(kScanThreads), 0, st, p, page_block, n_unc, t->uncovered_ptr,
                     t->uncovered);
  hipLaunchKernelGGL(k_edges, dim3(blocks_for(GQ, TB)), dim3(TB), 0, st, p, owner_of, nkw, nqw, edge, own_q, fullq);
  hipLaunchKernelGGL(k_owner_counts, dim3(blocks_for(GK, TB)), dim3(TB), 0, st, p, t->owner_ptr, n_own, own_info,
                     own_q, fullq, nqw, gsz, ng, rcount, qlen, owner_slot, split_of, t->aligned, t->owners,
                     t->kmask);
  hipLaunchKernelGGL(k_owner_pages, dim3(blocks_for(GK, TB)), dim3(TB), 0, st, p, owner_of, pos_of, t->owner_ptr,
                     t->owners, t->kmask);
  hipLaunchKernelGGL(k_owner_scans, dim3(1), dim3(kScanThreads), 0, st, d_sum, ng, rcount, qlen, t->revq_ptr,
                     t->qwalk_ptr, d_sum);
  hipLaunchKernelGGL(k_item_scan, dim3(1), dim3(kScanThreads), 0, st, d_sum, ng, t->qwalk_ptr, item_pos, item_w,
                     part_base, red_pos, d_sum);
  KP_CHECK(hipGetLastError());
  BwdSummary h{};
  KP_CHECK(hipMemcpyAsync(&h, d_sum, sizeof(BwdSummary), hipMemcpyDeviceToHost, st));
  KP_CHECK(hipStreamSynchronize(st));
  t->n_own = h.n_own;
  t->revq_total = h.revq_total;
  t->qwalk_total = h.qwalk_total;
  t->uncovered_total = h.uncovered_total;
  t->max_uncovered = h.max_uncovered;
  const int64_t n_w = h.n_witems;  // work items per graph slot (shared graph) or in all
  t->n_items = int64_t(mult) * n_w;
  t->n_partials = int64_t(mult) * h.n_part;
  t->n_reduce = int64_t(mult) * h.n_red;
  if (t->n_items >= (int64_t(1) << 31) || t->n_partials >= (int64_t(1) << 31)) {
    *err = "more than 2^31 backward work items";
    return KPAGE_ERR_UNSUPPORTED;
  }
  const int64_t n_steps = h.qwalk_total / kOwnerSlots;
  t->revq = static_cast<int32_t *>(A(h.revq_total, 4));
  t->qwalk = static_cast<int32_t *>(A(h.qwalk_total, 4));
  t->qpages = static_cast<int32_t *>(A(h.qwalk_total, 4));
  t->adj = static_cast<uint64_t *>(A(n_steps, 8));
  t->items = static_cast<BwdItem *>(A(t->n_items, sizeof(BwdItem)));
  t->bwd_queue = static_cast<int32_t *>(A(2 * t->n_items, 4));
  unsigned long long *keys = static_cast<unsigned long long *>(A(2 * t->n_items, 8));
  t->reduce = static_cast<BwdReduce *>(A(t->n_reduce, sizeof(BwdReduce)));
  if (oom) {
    *err = "device allocation failed while planning the backward";
    return KPAGE_ERR_OOM;
  }
  if (h.n_own > 0) {
    hipLaunchKernelGGL(k_owner_fill, dim3(blocks_for(h.n_own * ng, TB)), dim3(TB), 0, st, p, h.n_own, gsz, ng,
                       t->owner_ptr, owner_slot, split_of, own_q, fullq, nqw, t->revq_ptr, t->qwalk_ptr, t->revq,
                       t->qwalk, t->qpages);
    if (n_steps > 0)
      hipLaunchKernelGGL(k_adj, dim3(blocks_for(n_steps, TB)), dim3(TB), 0, st, p, page_block, h.n_own, ng, n_steps,
                         mult, owner_slot, t->qwalk_ptr, t->owners, t->qwalk, edge, nkw, t->adj, d_sum);
    hipLaunchKernelGGL(k_bwd_items, dim3(blocks_for(t->n_items, TB)), dim3(TB), 0, st, p, ng, n_w, t->n_items,
                       h.n_part, t->qwalk_ptr, owner_slot, item_pos, item_w, part_base, keys, t->items);
    if (t->n_reduce > 0) {
      const int64_t n_red_threads = p.per_head ? h.n_own : int64_t(mult) * h.n_own;
      hipLaunchKernelGGL(k_bwd_reduce_list, dim3(blocks_for(n_red_threads, TB)), dim3(TB), 0, st, p, h.n_own, ng,
                         h.n_part, h.n_red, owner_slot, item_pos, part_base, red_pos, n_red_threads, t->reduce);
    }
    hipLaunchKernelGGL(k_bwd_tails, dim3(kXcds), dim3(1024), 0, st, t->items, t->n_items);
    size_t tmp_bytes = 0;
    KP_CHECK(hipcub::DeviceRadixSort::SortKeys(nullptr, tmp_bytes, keys, keys + t->n_items, int(t->n_items), 0, 64,
                                               st));
    void *tmp = A(int64_t(std::max<size_t>(tmp_bytes, 16)), 1);
    if (oom) {
      *err = "device allocation failed while planning the backward";
      return KPAGE_ERR_OOM;
    }
    KP_CHECK(hipcub::DeviceRadixSort::SortKeys(tmp, tmp_bytes, keys, keys + t->n_items, int(t->n_items), 0, 64, st));
    hipLaunchKernelGGL(k_bwd_queue_out, dim3(blocks_for(t->n_items, TB)), dim3(TB), 0, st, p, ng, n_w, t->n_items,
                       t->owner_ptr, owner_slot, item_w, keys + t->n_items, t->bwd_queue);
  }
  KP_CHECK(hipGetLastError());
  KP_CHECK(hipMemcpyAsync(&h, d_sum, sizeof(BwdSummary), hipMemcpyDeviceToHost, st));
  KP_CHECK(hipStreamSynchronize(st));
#undef KP_CHECK
  t->bwd_physical = mult * (unsigned long long)kBlockRows * kBlockRows * (unsigned long long)n_steps;
  t->bwd_useful_check = h.useful_check;
  return KPAGE_OK;
}

}  // namespace kpage
