// Host planner: Page16 walks, Q64/Q128 routes and queues, validity words,
// K/V owners, reverse-Q lists, Q-page walks and page-pair adjacency words.
//
// KPage paper: section 3.2.1 (Page16 count p = ceil(c / 16), full pages of the
// selected blocks first, then one partial tail per partial block, then dummy
// pages), 3.2.2 (routes by c_q with 64 rows as the threshold; one queue per
// route, longer walks first; walks padded to whole iterations of 16 or 8 pages),
// 3.2.4 (two 16-bit page masks per 32-bit word), 3.3.1 (owners of eight page
// slots, full blocks aligned to their own owner, partial blocks packed without
// crossing an owner, by least growth of the owner's reverse neighbourhood), 3.3.2 (reverse-Q lists from an owner x Q bitmap; full Q
// blocks first, then pages of partial Q blocks), 3.3.3 (one 64-bit adjacency
// word per 8 x 8 page step), 3.4 (metadata depends only on the graph and the
// valid-row counts) and 4.4 (pair-capacity accounting).
#include "plan.hpp"

#include <algorithm>
#include <sstream>
#include <tuple>

namespace kpage {

namespace {

inline int pages_of(int c) { return (c + kPageRows - 1) / kPageRows; }
inline uint32_t tail_mask(int c) { return (1u << (c % kPageRows)) - 1u; }
inline uint32_t page_mask(int c, int j) {  // mask of page j of a block with c valid rows
  return (j + 1) * kPageRows <= c ? kFullMask : tail_mask(c);
}

template <class T>
std::string str(const T &v) {
  std::ostringstream os;
  os << v;
  return os.str();
}

}  // namespace

kpage_status load_scalars(const kpage_problem *p, const kpage_plan_opts *o, Problem *out, int *align64,
                          int *align128, std::string *err) {
  if (!p) { *err = "problem is NULL"; return KPAGE_ERR_INVALID; }
  if (p->batch < 1 || p->heads < 1) { *err = "batch and heads must be >= 1"; return KPAGE_ERR_INVALID; }
  if (p->head_dim != 64 && p->head_dim != 128) {
    *err = "head_dim " + str(p->head_dim) + " not supported (64 or 128)";
    return KPAGE_ERR_UNSUPPORTED;
  }
  if (p->n_q_blocks < 1 || p->n_kv_blocks < 1) { *err = "n_q_blocks and n_kv_blocks must be >= 1"; return KPAGE_ERR_INVALID; }
  if (p->seq_q != int64_t(kBlockRows) * p->n_q_blocks) { *err = "seq_q must equal 128 * n_q_blocks"; return KPAGE_ERR_INVALID; }
  if (p->seq_kv < kPageRows || p->seq_kv % kPageRows) { *err = "seq_kv must be a positive multiple of 16"; return KPAGE_ERR_INVALID; }
  if (p->per_head != 0 && p->per_head != 1) { *err = "per_head must be 0 or 1"; return KPAGE_ERR_INVALID; }
  if (!p->q_valid || !p->kv_valid || !p->q2k_ptr || (!p->q2k_idx)) {
    *err = "q_valid, kv_valid, q2k_ptr and q2k_idx are required";
    return KPAGE_ERR_INVALID;
  }
  int a64 = 16, a128 = 8;
  if (o) {
    if (o->q_group < 0) { *err = "q_group must be >= 0"; return KPAGE_ERR_INVALID; }
    if (o->align_q64) a64 = o->align_q64;
    if (o->align_q128) a128 = o->align_q128;
    if (a64 < 16 || a64 % 16 || a128 < 8 || a128 % 8) {
      *err = "align_q64 must be a multiple of 16 and align_q128 a multiple of 8";
      return KPAGE_ERR_INVALID;
    }
  }
  *align64 = a64;
  *align128 = a128;
  Problem &P = *out;
  P.batch = p->batch; P.heads = p->heads; P.head_dim = p->head_dim;
  P.n_q = p->n_q_blocks; P.n_kv = p->n_kv_blocks;
  P.seq_q = p->seq_q; P.seq_kv = p->seq_kv;
  P.per_head = p->per_head == 1;
  P.slots = P.per_head ? P.batch * P.heads : 1;
  P.q_group = o ? o->q_group : 0;
  P.grouped = !(o && o->ungrouped);
  return KPAGE_OK;
}

kpage_status load_problem(const kpage_problem *p, const kpage_plan_opts *o, Problem *out, int *align64,
                          int *align128, std::string *err) {
  kpage_status s = load_scalars(p, o, out, align64, align128, err);
  if (s != KPAGE_OK) return s;
  Problem &P = *out;
  const size_t G = P.slots, nq = P.n_q, nk = P.n_kv;
  P.q_valid.assign(p->q_valid, p->q_valid + G * nq);
  P.kv_valid.assign(p->kv_valid, p->kv_valid + G * nk);
  P.q2k_ptr.assign(p->q2k_ptr, p->q2k_ptr + G * (nq + 1));
  P.kv_offset.resize(G * nk);
  for (size_t g = 0; g < G; ++g)
    for (size_t k = 0; k < nk; ++k)
      P.kv_offset[g * nk + k] = p->kv_offset ? p->kv_offset[g * nk + k] : int64_t(kBlockRows) * int64_t(k);
  for (int32_t c : P.q_valid)
    if (c < 0 || c > kBlockRows) { *err = "q_valid outside [0,128]"; return KPAGE_ERR_INVALID; }
  for (int32_t c : P.kv_valid)
    if (c < 0 || c > kBlockRows) { *err = "kv_valid outside [0,128]"; return KPAGE_ERR_INVALID; }
  int64_t nnz = 0;
  for (size_t g = 0; g < G; ++g)
    for (size_t q = 0; q < nq; ++q) {
      int64_t a = P.q2k_ptr[g * (nq + 1) + q], b = P.q2k_ptr[g * (nq + 1) + q + 1];
      if (a < 0 || b < a) { *err = "q2k_ptr must be non-negative and non-decreasing within a row"; return KPAGE_ERR_INVALID; }
      nnz = std::max(nnz, b);
    }
  P.q2k_idx.assign(p->q2k_idx, p->q2k_idx + nnz);
  // footprints: page aligned, inside seq_kv, pairwise disjoint
  const int64_t n_pages = P.seq_kv / kPageRows;
  std::vector<int32_t> owner_block(n_pages);
  for (size_t g = 0; g < G; ++g) {
    std::fill(owner_block.begin(), owner_block.end(), -1);
    for (size_t k = 0; k < nk; ++k) {
      int64_t off = P.kv_offset[g * nk + k];
      int c = P.kv_valid[g * nk + k];
      if (off < 0 || off % kPageRows) { *err = "kv_offset must be a non-negative multiple of 16"; return KPAGE_ERR_INVALID; }
      if (off + int64_t(kPageRows) * pages_of(c) > P.seq_kv) { *err = "a K/V block footprint exceeds seq_kv"; return KPAGE_ERR_INVALID; }
      for (int j = 0; j < pages_of(c); ++j) {
        int64_t pg = off / kPageRows + j;
        if (owner_block[pg] >= 0) { *err = "K/V block page footprints overlap"; return KPAGE_ERR_INVALID; }
        owner_block[pg] = int32_t(k);
      }
    }
    std::vector<int32_t> seen(nk, -1);
    for (size_t q = 0; q < nq; ++q) {
      int64_t a = P.q2k_ptr[g * (nq + 1) + q], b = P.q2k_ptr[g * (nq + 1) + q + 1];
      for (int64_t e = a; e < b; ++e) {
        int32_t k = P.q2k_idx[e];
        if (k < 0 || k >= P.n_kv) { *err = "q2k_idx entry outside [0, n_kv)"; return KPAGE_ERR_INVALID; }
        if (seen[k] == int32_t(q)) { *err = "duplicate K/V block in a selection list"; return KPAGE_ERR_INVALID; }
        seen[k] = int32_t(q);
      }
    }
  }
  return KPAGE_OK;
}

void build_forward(const Problem &P, FwdTables *T, PairStats *S) {
  const int G = P.slots, nq = P.n_q, nk = P.n_kv;
  const int BH = P.batch * P.heads;
  std::vector<int> bh_per_slot(G, 0);
  for (int bh = 0; bh < BH; ++bh) bh_per_slot[P.slot_of(bh)]++;
  T->route.assign(size_t(G) * nq, 0);
  T->nfull.assign(size_t(G) * nq, 0);
  T->unpadded.assign(size_t(G) * nq, 0);
  T->walk_ptr.assign(size_t(G) * (nq + 1), 0);
  T->walk.clear();
  T->valid.clear();
  std::vector<uint32_t> masks;
  for (int g = 0; g < G; ++g) {
    const int32_t *cq = &P.q_valid[size_t(g) * nq];
    const int32_t *ck = &P.kv_valid[size_t(g) * nk];
    const int64_t *ok = &P.kv_offset[size_t(g) * nk];
    const uint64_t mult = uint64_t(bh_per_slot[g]);
    for (int q = 0; q < nq; ++q) {
      T->walk_ptr[size_t(g) * (nq + 1) + q] = int64_t(T->walk.size());
      if (cq[q] == 0) continue;
      const int route = cq[q] <= 64 ? 64 : 128;
      const int per_step = route == 64 ? T->align64 : T->align128;
      const int64_t a = P.q2k_ptr[size_t(g) * (nq + 1) + q], b = P.q2k_ptr[size_t(g) * (nq + 1) + q + 1];
      const size_t start = T->walk.size();
      masks.clear();
      uint64_t useful = 0, psum = 0;
      // full pages of every selected block, in selection order
      for (int64_t e = a; e < b; ++e) {
        const int k = P.q2k_idx[e];
        const int32_t base = int32_t(ok[k] / kPageRows);
        for (int j = 0; j < ck[k] / kPageRows; ++j) {
          T->walk.push_back(base + j);
          masks.push_back(kFullMask);
        }
        useful += uint64_t(cq[q]) * uint64_t(ck[k]);
        psum += uint64_t(pages_of(ck[k]));
      }
      const int n_full = int(T->walk.size() - start);
      // then the partial tail of every partial block, in selection order
      for (int64_t e = a; e < b; ++e) {
        const int k = P.q2k_idx[e];
        if (ck[k] % kPageRows) {
          T->walk.push_back(int32_t(ok[k] / kPageRows) + ck[k] / kPageRows);
          masks.push_back(tail_mask(ck[k]));
        }
      }
      const int unpadded = int(T->walk.size() - start);
      while ((T->walk.size() - start) % per_step) {
        T->walk.push_back(-1);
        masks.push_back(0);
      }
      for (size_t i = 0; i + 1 < masks.size(); i += 2) T->valid.push_back(masks[i] | (masks[i + 1] << 16));
      T->route[size_t(g) * nq + q] = route;
      T->nfull[size_t(g) * nq + q] = n_full;
      T->unpadded[size_t(g) * nq + q] = unpadded;
      const uint64_t M = uint64_t(route == 64 ? 64 : 128);
      const uint64_t len = uint64_t(T->walk.size() - start);
      S->useful += mult * useful;
      S->whole_block += mult * uint64_t(kBlockRows) * kBlockRows * uint64_t(b - a);
      S->paged_m128 += mult * uint64_t(kBlockRows) * kPageRows * psum;
      S->nominal += mult * M * kPageRows * psum;
      S->scheduled += mult * M * kPageRows * len;
    }
    T->walk_ptr[size_t(g) * (nq + 1) + nq] = int64_t(T->walk.size());
  }
  // per-route queues: longest unpadded walk first, then (bh, q) ascending
  for (int route : {64, 128}) {
    std::vector<std::tuple<int, int, int>> ent;
    for (int bh = 0; bh < BH; ++bh) {
      const int g = P.slot_of(bh);
      for (int q = 0; q < nq; ++q)
        if (T->route[size_t(g) * nq + q] == route) ent.emplace_back(-T->unpadded[size_t(g) * nq + q], bh, q);
    }
    std::sort(ent.begin(), ent.end());
    auto &out = route == 64 ? T->q64_queue : T->q128_queue;
    out.clear();
    for (auto &x : ent) {
      out.push_back(std::get<1>(x));
      out.push_back(std::get<2>(x));
    }
  }
}

// Group items.  A query block of the M64 x N256 route with at most 32 valid rows leaves
// three of its item's four waves' worth of MFMA work unused for every page it gathers:
// its 4-page stages are bound by the gathers, not by the matrix cores.  Blocks whose
// selections overlap share most pages, so up to four of them run as one M128 x N128 item
// over the union of their walks (wave w computes member w's rows and masks the pages its
// block did not select): the union is gathered once.  Greedy, per slot, in block order:
// the first free block opens a group, which then takes, among the free blocks that share
// a page with every member, the one with the largest share of its pages already in the
// group's union (ties: lower block), while that share is at least one half.  A group of
// one stays a plain item.  Union walk: the pages that
// are full and selected by every member (in the first member's walk order; no masking
// in their stages), then the other pages every member selected (same order), then each
// member's remaining pages in its walk order, padded with dummies to whole 4-page stages.
void build_groups(const Problem &P, const FwdTables &F, GroupTables *T) {
  const int G = P.slots, nq = P.n_q;
  T->group_ptr.assign(size_t(G) + 1, 0);
  T->members.clear();
  T->walk_ptr.assign(1, 0);
  T->walk.clear();
  T->nfull.clear();
  T->npages.clear();
  T->valid.clear();
  T->in_group.assign(size_t(G) * nq, 0);
  const int64_t n_pg = P.seq_kv / kPageRows;
  const size_t W = size_t((n_pg + 63) / 64);
  std::vector<uint64_t> bits, uni(W), inter(W);
  std::vector<uint32_t> pmask(size_t(n_pg), 0);
  auto candidates = [&](int g) {  // eligible blocks of slot g, ascending; none past the limits
    std::vector<int> cand;
    for (int q = 0; q < nq; ++q) {
      const int cq = P.q_valid[size_t(g) * nq + q];
      if (F.route[size_t(g) * nq + q] == 64 && cq > 0 && cq <= kGroupMaxRows && F.unpadded[size_t(g) * nq + q] > 0)
        cand.push_back(q);
    }
    if (cand.size() < 2 || cand.size() > size_t(kGroupMaxCands)) cand.clear();
    return cand;
  };
  bool grouped = P.grouped && W <= size_t(kGroupMaxWords);
  if (grouped) {
    int64_t words = 0;
    for (int g = 0; g < G; ++g) words += int64_t(candidates(g).size()) * int64_t(W);
    grouped = words <= kGroupMaxBitsetWords;
  }
  for (int g = 0; g < G; ++g) {
    T->group_ptr[size_t(g) + 1] = T->group_ptr[size_t(g)];
    if (!grouped) continue;
    const std::vector<int> cand = candidates(g);
    if (cand.empty()) continue;
    // page sets as bitsets, and every page's row mask
    bits.assign(cand.size() * W, 0);
    std::vector<int> n_of(cand.size(), 0);
    for (size_t c = 0; c < cand.size(); ++c) {
      const int64_t a = F.walk_ptr[size_t(g) * (nq + 1) + cand[c]];
      const int n = F.unpadded[size_t(g) * nq + cand[c]];
      for (int i = 0; i < n; ++i) {
        const int32_t pg = F.walk[size_t(a + i)];
        bits[c * W + size_t(pg >> 6)] |= uint64_t(1) << (pg & 63);
        pmask[size_t(pg)] = (F.valid[size_t((a + i) >> 1)] >> (16 * ((a + i) & 1))) & kFullMask;
      }
      n_of[c] = n;
    }
    std::vector<uint8_t> free_(cand.size(), 1);
    for (size_t c0 = 0; c0 < cand.size(); ++c0) {
      if (!free_[c0]) continue;
      free_[c0] = 0;
      std::vector<size_t> grp{c0};
      std::copy(bits.begin() + c0 * W, bits.begin() + (c0 + 1) * W, uni.begin());
      std::copy(bits.begin() + c0 * W, bits.begin() + (c0 + 1) * W, inter.begin());
      while (grp.size() < size_t(kGroupMembers)) {
        size_t best = cand.size();
        int64_t best_in = 0, best_n = 1;
        for (size_t c = c0 + 1; c < cand.size(); ++c) {
          if (!free_[c]) continue;
          // one pass: pages shared with every member, and pages already in the union
          const uint64_t *bc = &bits[c * W];
          uint64_t sh = 0;
          int64_t in = 0;
          for (size_t w = 0; w < W; ++w) {
            sh |= inter[w] & bc[w];
            in += __builtin_popcountll(uni[w] & bc[w]);
          }
          if (sh == 0) continue;  // no page selected by every member and by the candidate
          if (best == cand.size() || in * best_n > best_in * n_of[c]) {
            best = c;
            best_in = in;
            best_n = n_of[c];
          }
        }
        if (best == cand.size() || 2 * best_in < best_n) break;
        free_[best] = 0;
        grp.push_back(best);
        for (size_t w = 0; w < W; ++w) {
          uni[w] |= bits[best * W + w];
          inter[w] &= bits[best * W + w];
        }
      }
      if (grp.size() < 2) continue;
      // union walk
      auto in_member = [&](size_t c, int32_t pg) { return (bits[c * W + size_t(pg >> 6)] >> (pg & 63)) & 1u; };
      std::vector<int32_t> order;
      auto walk_of = [&](size_t c, int i) {
        return F.walk[size_t(F.walk_ptr[size_t(g) * (nq + 1) + cand[c]] + i)];
      };
      std::vector<uint8_t> used(size_t(n_pg), 0);
      for (int i = 0; i < n_of[grp[0]]; ++i) {
        const int32_t pg = walk_of(grp[0], i);
        if (pmask[size_t(pg)] != kFullMask) continue;
        bool all = true;
        for (size_t m = 1; m < grp.size(); ++m) all = all && in_member(grp[m], pg);
        if (all) {
          order.push_back(pg);
          used[size_t(pg)] = 1;
        }
      }
      const int n_full = int(order.size());
      // then the other pages every member selected, so that the first sub-tile holds a
      // valid key for every member whenever they share a page
      for (int i = 0; i < n_of[grp[0]]; ++i) {
        const int32_t pg = walk_of(grp[0], i);
        if (used[size_t(pg)]) continue;
        bool all = true;
        for (size_t m = 1; m < grp.size(); ++m) all = all && in_member(grp[m], pg);
        if (all) {
          order.push_back(pg);
          used[size_t(pg)] = 1;
        }
      }
      for (size_t m = 0; m < grp.size(); ++m)
        for (int i = 0; i < n_of[grp[m]]; ++i) {
          const int32_t pg = walk_of(grp[m], i);
          if (!used[size_t(pg)]) {
            order.push_back(pg);
            used[size_t(pg)] = 1;
          }
        }
      const int n_real = int(order.size());
      while (order.size() % 4) order.push_back(-1);
      T->walk.insert(T->walk.end(), order.begin(), order.end());
      T->walk_ptr.push_back(int64_t(T->walk.size()));
      T->nfull.push_back(n_full);
      T->npages.push_back(n_real);
      for (int w = 0; w < kGroupMembers; ++w) {
        for (size_t i = 0; i < order.size(); i += 2) {
          uint32_t word = 0;
          for (int h = 0; h < 2; ++h) {
            const int32_t pg = order[i + size_t(h)];
            if (pg >= 0 && size_t(w) < grp.size() && in_member(grp[size_t(w)], pg))
              word |= pmask[size_t(pg)] << (16 * h);
          }
          T->valid.push_back(word);
        }
      }
      for (int w = 0; w < kGroupMembers; ++w) {
        const int32_t q = size_t(w) < grp.size() ? cand[grp[size_t(w)]] : -1;
        T->members.push_back(q);
        if (q >= 0) T->in_group[size_t(g) * nq + q] = 1;
      }
      T->group_ptr[size_t(g) + 1]++;
    }
  }
}

void build_backward(const Problem &P, BwdTables *T, PairStats *S) {
  const int G = P.slots, nq = P.n_q, nk = P.n_kv;
  const int BH = P.batch * P.heads;
  std::vector<int> bh_per_slot(G, 0);
  for (int bh = 0; bh < BH; ++bh) bh_per_slot[P.slot_of(bh)]++;
  *T = BwdTables();
  T->owner_ptr.push_back(0);
  T->revq_ptr.push_back(0);
  T->qwalk_ptr.push_back(0);
  T->uncovered_ptr.push_back(0);
  S->bwd_physical = 0;
  S->bwd_useful_check = 0;
  const int gsz = P.q_group > 0 ? std::min(P.q_group, nq) : nq;
  const int n_groups = (nq + gsz - 1) / gsz;
  T->n_groups = n_groups;
  std::vector<std::vector<std::vector<int>>> steps_of(G);  // [slot][owner][group]
  const int64_t n_pages = P.seq_kv / kPageRows;
  for (int g = 0; g < G; ++g) {
    const int32_t *cq = &P.q_valid[size_t(g) * nq];
    const int32_t *ck = &P.kv_valid[size_t(g) * nk];
    const int64_t *ok = &P.kv_offset[size_t(g) * nk];
    const uint64_t mult = uint64_t(bh_per_slot[g]);
    // owners (reading of section 3.3.1's packing): every full block is an owner of its
    // own, in block order; the partial blocks then fill owners one at a time: the
    // smallest unplaced one opens an owner, and while one fits, the fitting block that
    // adds the fewest query blocks to the owner's reverse neighbourhood joins (ties to
    // the smaller index).  Reverse neighbourhoods as bitsets over query blocks.
    std::vector<std::vector<int32_t>> own;
    std::vector<std::vector<int32_t>> own_blocks;
    std::vector<int32_t> owner_of(nk, -1);
    for (int k = 0; k < nk; ++k) {
      if (ck[k] != kBlockRows) continue;
      owner_of[k] = int32_t(own.size());
      own.emplace_back();
      own_blocks.push_back({k});
      for (int j = 0; j < kOwnerSlots; ++j) own.back().push_back(int32_t(ok[k] / kPageRows) + j);
    }
    {
      const int qw = (nq + 63) / 64;
      std::vector<int32_t> partial;
      for (int k = 0; k < nk; ++k)
        if (ck[k] > 0 && ck[k] < kBlockRows) partial.push_back(k);
      std::vector<uint64_t> rq(size_t(nk) * qw, 0);  // reverse neighbourhood of each block
      for (int q = 0; q < nq; ++q) {
        if (cq[q] == 0) continue;
        const int64_t a = P.q2k_ptr[size_t(g) * (nq + 1) + q], b = P.q2k_ptr[size_t(g) * (nq + 1) + q + 1];
        for (int64_t e = a; e < b; ++e) {
          const int k = P.q2k_idx[e];
          if (ck[k] > 0) rq[size_t(k) * qw + q / 64] |= uint64_t(1) << (q % 64);
        }
      }
      std::vector<uint8_t> placed(nk, 0);
      std::vector<uint64_t> covered(qw);
      for (size_t s0 = 0; s0 < partial.size(); ++s0) {
        const int seed = partial[s0];
        if (placed[seed]) continue;
        const int cur = int(own.size());
        own.emplace_back();
        own_blocks.emplace_back();
        std::fill(covered.begin(), covered.end(), 0);
        auto place = [&](int k) {
          placed[k] = 1;
          owner_of[k] = cur;
          own_blocks[cur].push_back(k);
          for (int j = 0; j < pages_of(ck[k]); ++j) own[cur].push_back(int32_t(ok[k] / kPageRows) + j);
          for (int w = 0; w < qw; ++w) covered[w] |= rq[size_t(k) * qw + w];
        };
        place(seed);
        for (;;) {
          const int free_slots = kOwnerSlots - int(own[cur].size());
          int best = -1, best_new = 0;
          for (size_t i = s0 + 1; i < partial.size() && free_slots > 0; ++i) {
            const int k = partial[i];
            if (placed[k] || pages_of(ck[k]) > free_slots) continue;
            int new_q = 0;
            for (int w = 0; w < qw; ++w) new_q += __builtin_popcountll(rq[size_t(k) * qw + w] & ~covered[w]);
            if (best < 0 || new_q < best_new) {
              best = k;
              best_new = new_q;
              if (new_q == 0) break;  // the smallest index adding nothing
            }
          }
          if (best < 0) break;
          place(best);
        }
      }
    }
    const int n_own = int(own.size());
    // per-page block and row mask, for adjacency and the visited-pair check
    std::vector<int32_t> page_block(n_pages, -1);
    for (int k = 0; k < nk; ++k)
      for (int j = 0; j < pages_of(ck[k]); ++j) page_block[ok[k] / kPageRows + j] = k;
    for (int64_t pg = 0; pg < n_pages; ++pg)
      if (page_block[pg] < 0) T->uncovered.push_back(int32_t(pg));
    T->uncovered_ptr.push_back(int64_t(T->uncovered.size()));
    // graph edges (c_q > 0, c_k > 0) as a dense bit matrix and the owner x Q bitmap
    std::vector<uint8_t> edge(size_t(nq) * nk, 0);
    std::vector<uint8_t> bitmap(size_t(n_own) * nq, 0);
    for (int q = 0; q < nq; ++q) {
      if (cq[q] == 0) continue;
      const int64_t a = P.q2k_ptr[size_t(g) * (nq + 1) + q], b = P.q2k_ptr[size_t(g) * (nq + 1) + q + 1];
      for (int64_t e = a; e < b; ++e) {
        const int k = P.q2k_idx[e];
        if (ck[k] == 0) continue;
        edge[size_t(q) * nk + k] = 1;
        bitmap[size_t(owner_of[k]) * nq + q] = 1;
      }
    }
    for (int t = 0; t < n_own; ++t) {
      auto &pages = own[t];
      const uint8_t al = (own_blocks[t].size() == 1 && pages.size() == size_t(kOwnerSlots)) ? 1 : 0;
      while (pages.size() < size_t(kOwnerSlots)) pages.push_back(-1);
      std::vector<int> owner_steps;
      // an owner whose reverse neighbourhood holds at most gsz Q blocks is within the
      // bound the groups serve: its whole list is group 0, the other groups are empty
      int n_revq = 0;
      for (int q = 0; q < nq; ++q) n_revq += bitmap[size_t(t) * nq + q];
      const bool split = n_revq > gsz;
      for (int grp = 0; grp < n_groups; ++grp) {
        // reverse neighbourhood of owner t inside Q group grp, ascending q
        std::vector<int32_t> R;
        const int q_lo = split ? grp * gsz : (grp == 0 ? 0 : nq);
        const int q_hi = split ? std::min(nq, (grp + 1) * gsz) : (grp == 0 ? nq : nq);
        for (int q = q_lo; q < q_hi; ++q)
          if (bitmap[size_t(t) * nq + q]) R.push_back(q);
        T->revq.insert(T->revq.end(), R.begin(), R.end());
        T->revq_ptr.push_back(int64_t(T->revq.size()));
        const size_t w0 = T->qwalk.size();
        for (int q : R)
          if (cq[q] == kBlockRows)
            for (int j = 0; j < 8; ++j) T->qwalk.push_back(8 * q + j);
        for (int q : R)
          if (cq[q] > 0 && cq[q] < kBlockRows)
            for (int j = 0; j < pages_of(cq[q]); ++j) T->qwalk.push_back(8 * q + j);
        while ((T->qwalk.size() - w0) % 8) T->qwalk.push_back(-1);
        T->qwalk_ptr.push_back(int64_t(T->qwalk.size()));
        const int n_steps = int((T->qwalk.size() - w0) / 8);
        for (int s = 0; s < n_steps; ++s) {
          uint64_t word = 0;
          for (int j = 0; j < 8; ++j) {
            const int32_t qp = T->qwalk[w0 + 8 * s + j];
            if (qp < 0) continue;
            const int qb = qp / 8;
            const uint32_t qm = page_mask(cq[qb], qp % 8);
            for (int i = 0; i < 8; ++i) {
              const int32_t kp = pages[i];
              if (kp < 0) continue;
              const int kb = page_block[kp];
              if (!edge[size_t(qb) * nk + kb]) continue;
              word |= uint64_t(1) << (8 * j + i);
              const uint32_t km = page_mask(ck[kb], int(kp - ok[kb] / kPageRows));
              S->bwd_useful_check += mult * uint64_t(__builtin_popcount(qm)) * uint64_t(__builtin_popcount(km));
            }
          }
          T->adj.push_back(word);
        }
        S->bwd_physical += mult * uint64_t(kBlockRows) * kBlockRows * uint64_t(n_steps);
        owner_steps.push_back(n_steps);
      }
      T->owners.insert(T->owners.end(), pages.begin(), pages.end());
      T->aligned.push_back(al);
      steps_of[g].push_back(owner_steps);
    }
    T->owner_ptr.push_back(T->owner_ptr.back() + n_own);
  }
  // work items: every (owner, group) with a non-empty neighbourhood (n_steps > 0); an owner
  // without any keeps one item for group 0, which writes its zero gradients
  std::vector<std::tuple<int, int, int, int>> ent;
  for (int bh = 0; bh < BH; ++bh) {
    const int g = P.slot_of(bh);
    for (size_t t = 0; t < steps_of[g].size(); ++t) {
      const auto &st = steps_of[g][t];
      bool any = false;
      for (int grp = 0; grp < n_groups; ++grp)
        if (st[grp] > 0) {
          ent.emplace_back(-st[grp], bh, int(t), grp);
          any = true;
        }
      if (!any) ent.emplace_back(0, bh, int(t), 0);
    }
  }
  std::sort(ent.begin(), ent.end());
  for (auto &x : ent) {
    T->bwd_queue.push_back(std::get<1>(x));
    T->bwd_queue.push_back(std::get<2>(x) * n_groups + std::get<3>(x));
  }
  T->built = true;
}

}  // namespace kpage
