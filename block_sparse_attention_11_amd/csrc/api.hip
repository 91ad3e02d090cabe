// C ABI: plan handle, descriptor validation, device uploads and kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "device.hpp"
#include "kpage.h"
#include "plan.hpp"
#include "plan_dev.hpp"
#include "select.hpp"

using namespace kpage;

namespace {

// HIP event pairs around every launch, pooled and kept per kernel id until read.
class EventTimer final : public LaunchTimer {
 public:
  explicit EventTimer(bool split) : split_(split) {}
  bool split_routes() const override { return split_; }
  ~EventTimer() override {
    for (auto &k : pending_)
      for (auto &p : k) {
        (void)hipEventDestroy(p.first);
        (void)hipEventDestroy(p.second);
      }
    for (hipEvent_t e : pool_) (void)hipEventDestroy(e);
  }
  void before(int kid, hipStream_t s) override {
    hipEvent_t e = take();
    (void)hipEventRecord(e, s);
    open_[kid] = e;
  }
  void after(int kid, hipStream_t s) override {
    hipEvent_t e = take();
    (void)hipEventRecord(e, s);
    pending_[kid].emplace_back(open_[kid], e);
  }
  // sum of elapsed milliseconds and launch count of one kernel; returns false on a HIP error
  bool read(int kid, double *ms, int64_t *n) {
    double total = 0;
    for (auto &p : pending_[kid]) {
      float t = 0;
      if (hipEventSynchronize(p.second) != hipSuccess || hipEventElapsedTime(&t, p.first, p.second) != hipSuccess)
        return false;
      total += t;
      pool_.push_back(p.first);
      pool_.push_back(p.second);
    }
    *ms = total;
    *n = int64_t(pending_[kid].size());
    pending_[kid].clear();
    return true;
  }

 private:
  hipEvent_t take() {
    if (pool_.empty()) {
      hipEvent_t e = nullptr;
      (void)hipEventCreate(&e);
      return e;
    }
    hipEvent_t e = pool_.back();
    pool_.pop_back();
    return e;
  }
  bool split_;
  std::vector<hipEvent_t> pool_;
  hipEvent_t open_[KPAGE_K_COUNT] = {};
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending_[KPAGE_K_COUNT];
};

}  // namespace

struct kpage_plan {
  Problem P;
  FwdTables F;
  BwdTables B;
  GroupTables GT;  // group items (device-planned plans: host copies for export)
  PairStats S;
  bool fwd_on_device = false;
  // built by kpage_plan_device: the descriptor and every table live on the device
  // (the host Problem holds the scalars only); host copies of the tables are made
  // for export
  bool device_planned = false;
  bool fwd_on_host = true;
  DevProblem DP;
  DevFwdTables DF;
  DevBwdTables DB;  // backward tables of a device-planned plan
  bool bwd_on_device = false;
  // forward device tables
  FwdItem *d_items128 = nullptr, *d_items64 = nullptr;
  int32_t *d_order = nullptr;  // launch position -> item of either route (NULL: M128 then M64)
  FwdGroup *d_groups = nullptr;  // member tables of the group items (NULL: none)
  int n_items128 = 0, n_items64 = 0;
  int32_t *d_pages = nullptr;
  uint32_t *d_valid = nullptr;
  // backward device tables
  BwdItem *d_bitems = nullptr;
  int n_bitems = 0;
  int32_t *d_owners = nullptr, *d_qpages = nullptr, *d_uncovered = nullptr;
  uint32_t *d_kmask = nullptr;
  uint64_t *d_adj = nullptr;
  int64_t *d_uncovered_ptr = nullptr;
  int max_uncovered = 0;
  // owners split over several Q groups: fp32 partial slots in the workspace, reduce list
  BwdReduce *d_reduce = nullptr;
  const int32_t *d_qvalid = nullptr;  // [slots][n_q] query sizes for the backward's row masks
  int n_reduce = 0;
  int64_t n_partials = -1;  // -1: not counted yet
  std::vector<void *> allocations;
  EventTimer *timer = nullptr;
};
typedef struct kpage_plan PlanT;

namespace {

thread_local std::string g_last_error;

kpage_status fail(kpage_status s, const std::string &msg) {
  g_last_error = msg;
  return s;
}

kpage_status hip_fail(hipError_t e, const char *what) {
  return fail(KPAGE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Runs an entry point's body; a failed host allocation inside it (lazy table builds)
// becomes KPAGE_ERR_OOM instead of an exception crossing the C ABI.
template <class F>
kpage_status guarded(F &&body) {
  try {
    return body();
  } catch (const std::bad_alloc &) {
    return fail(KPAGE_ERR_OOM, "host allocation failed");
  }
}

template <class T>
kpage_status upload(PlanT *pl, const std::vector<T> &host, T **dev, hipStream_t stream) {
  const size_t bytes = std::max<size_t>(host.size() * sizeof(T), sizeof(T));
  void *p = nullptr;
  hipError_t e = hipMalloc(&p, bytes);
  if (e != hipSuccess) return fail(KPAGE_ERR_OOM, std::string("hipMalloc: ") + hipGetErrorString(e));
  pl->allocations.push_back(p);
  if (!host.empty()) {
    e = hipMemcpyAsync(p, host.data(), host.size() * sizeof(T), hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
  }
  *dev = static_cast<T *>(p);
  return KPAGE_OK;
}

// Copy a walk table with every dummy slot (-1) pointed at the first page of its
// own walk, so the kernels always load finite data; the row masks keep those
// slots out of the result.  `ptr` lists walk boundaries.
std::vector<int32_t> redirect_dummies(const std::vector<int32_t> &walk, const std::vector<int64_t> &ptr) {
  std::vector<int32_t> out(walk);
  for (size_t i = 0; i + 1 < ptr.size(); ++i) {
    const int64_t a = ptr[i], b = ptr[i + 1];
    if (b <= a) continue;
    const int32_t first = walk[a];
    for (int64_t j = a; j < b; ++j)
      if (out[j] < 0) out[j] = first;
  }
  return out;
}

// Launch order (launch_position): the plan's queues (longest walk first) keep their
// order for export; this permutation only decides which workgroup runs which item.
template <class T>
std::vector<T> xcd_interleave(const std::vector<T> &seq, int64_t chunk) {
  const int64_t n = int64_t(seq.size());
  std::vector<T> out(seq.size());
  for (int64_t p = 0; p < n; ++p) out[size_t(launch_position(p, n, chunk))] = seq[size_t(p)];
  return out;
}

// The last tail_len(count) items of each XCD's launch sequence (positions 8 j + x) in
// descending step count (ties keep their order), so that an XCD ends on its shortest
// owners instead of whichever came last in spatial order.
void sort_xcd_tails(std::vector<BwdItem> &items) {
  const int64_t n = int64_t(items.size());
  for (int x = 0; x < kXcds; ++x) {
    const int64_t cnt = n > x ? (n - x + kXcds - 1) / kXcds : 0;
    const int64_t t = bwd_tail_len(cnt);
    std::vector<BwdItem> tail;
    for (int64_t j = cnt - t; j < cnt; ++j) tail.push_back(items[size_t(j * kXcds + x)]);
    std::stable_sort(tail.begin(), tail.end(), [](const BwdItem &a, const BwdItem &b) { return a.n_steps > b.n_steps; });
    for (int64_t j = cnt - t; j < cnt; ++j) items[size_t(j * kXcds + x)] = tail[size_t(j - (cnt - t))];
  }
}

kpage_status ensure_forward_on_device(PlanT *pl, hipStream_t stream) {
  if (pl->fwd_on_device) return KPAGE_OK;
  const Problem &P = pl->P;
  const FwdTables &F = pl->F;
  const int nq = P.n_q;
  std::vector<int32_t> pages = redirect_dummies(F.walk, F.walk_ptr);
  const GroupTables &GT = pl->GT;
  const bool has_groups = !GT.members.empty();
  std::vector<FwdItem> it128, it64;
  auto make = [&](int bh, int q) {
    const int g = P.slot_of(bh);
    FwdItem x{};
    x.walk_off = F.walk_ptr[size_t(g) * (nq + 1) + q];
    x.walk_len = int32_t(F.walk_ptr[size_t(g) * (nq + 1) + q + 1] - x.walk_off);
    x.bh = bh;
    x.q = q;
    x.n_full = F.nfull[size_t(g) * nq + q];
    x.n_pages = F.unpadded[size_t(g) * nq + q];
    x.c_q = P.q_valid[size_t(g) * nq + q];
    return x;
  };
  for (size_t i = 0; i < F.q128_queue.size(); i += 2) it128.push_back(make(F.q128_queue[i], F.q128_queue[i + 1]));
  for (size_t i = 0; i < F.q64_queue.size(); i += 2) {
    const int bh = F.q64_queue[i], q = F.q64_queue[i + 1];
    if (has_groups && GT.in_group[size_t(P.slot_of(bh)) * nq + q]) continue;  // runs inside its group item
    it64.push_back(make(bh, q));
  }
  // group items: union walks after the plan's walks, member validity words after its
  // words; one FwdGroup per group of a slot, shared by the (batch, head)s of the slot
  std::vector<FwdGroup> groups;
  std::vector<uint32_t> valid_all;
  if (has_groups) {
    const std::vector<int32_t> gpages = redirect_dummies(GT.walk, GT.walk_ptr);
    const int64_t walk_base = int64_t(pages.size());
    const int64_t valid_base = int64_t(F.valid.size());
    pages.insert(pages.end(), gpages.begin(), gpages.end());
    valid_all = F.valid;
    valid_all.insert(valid_all.end(), GT.valid.begin(), GT.valid.end());
    const size_t ng = GT.nfull.size();
    groups.resize(ng);
    for (size_t i = 0; i < ng; ++i) {
      FwdGroup &gr = groups[i];
      for (int w = 0; w < kGroupMembers; ++w) {
        gr.q[w] = GT.members[i * kGroupMembers + size_t(w)];
        gr.c_q[w] = 0;
      }
      gr.valid_off = valid_base + 2 * GT.walk_ptr[i];
      gr.pad = 0;
    }
    for (int g = 0; g < P.slots; ++g)
      for (int64_t i = GT.group_ptr[size_t(g)]; i < GT.group_ptr[size_t(g) + 1]; ++i)
        for (int w = 0; w < kGroupMembers; ++w)
          if (groups[size_t(i)].q[w] >= 0) groups[size_t(i)].c_q[w] = P.q_valid[size_t(g) * nq + groups[size_t(i)].q[w]];
    for (int bh = 0; bh < P.batch * P.heads; ++bh) {
      const int g = P.slot_of(bh);
      for (int64_t i = GT.group_ptr[size_t(g)]; i < GT.group_ptr[size_t(g) + 1]; ++i) {
        FwdItem x{};
        x.walk_off = walk_base + GT.walk_ptr[size_t(i)];
        x.walk_len = int32_t(GT.walk_ptr[size_t(i) + 1] - GT.walk_ptr[size_t(i)]);
        x.bh = bh;
        x.q = ~int32_t(i);
        x.n_full = GT.nfull[size_t(i)];
        x.n_pages = GT.npages[size_t(i)];
        x.c_q = kBlockRows;
        it128.push_back(x);
      }
    }
  }
  // head-major, spatial order inside a head; a head's group items after its other M128 items
  auto head_major = [nq](const FwdItem &a, const FwdItem &b) {
    const int64_t ka = a.q >= 0 ? a.q : int64_t(nq) + ~a.q, kb = b.q >= 0 ? b.q : int64_t(nq) + ~b.q;
    return a.bh != b.bh ? a.bh < b.bh : ka < kb;
  };
  std::stable_sort(it128.begin(), it128.end(), head_major);
  std::stable_sort(it64.begin(), it64.end(), head_major);
  // blocks without valid rows still own their output rows: cleanup items (empty walk)
  // after the M64 items
  const size_t n64 = it64.size();
  for (int bh = 0; bh < P.batch * P.heads; ++bh)
    for (int q = 0; q < nq; ++q)
      if (P.q_valid[size_t(P.slot_of(bh)) * nq + q] == 0) it64.push_back(make(bh, q));
  // Launch order: one list of both routes, head-major, each head's M128 items before its
  // M64 items (so that they gather pages the M128 items have just brought into the
  // caches), cleanup items last; the list position of M128 item i of head bh is i + (M64
  // items of heads < bh), of M64 item j, j + (M128 items of heads <= bh).  The list is
  // dealt to the XCDs by launch_position; order[b] names workgroup b's item (i, or ~j).
  const int BH = P.batch * P.heads;
  std::vector<int64_t> pre128(BH + 1, 0), pre64(BH + 1, 0);
  for (const FwdItem &x : it128) ++pre128[x.bh + 1];
  for (size_t j = 0; j < n64; ++j) ++pre64[it64[j].bh + 1];
  for (int bh = 0; bh < BH; ++bh) {
    pre128[bh + 1] += pre128[bh];
    pre64[bh + 1] += pre64[bh];
  }
  const int64_t chunk = xcd_chunk_for(P.seq_q, P.seq_kv, P.head_dim);
  const int64_t n_all = int64_t(it128.size() + it64.size());
  std::vector<int32_t> order(static_cast<size_t>(n_all));
  for (size_t i = 0; i < it128.size(); ++i)
    order[size_t(launch_position(int64_t(i) + pre64[it128[i].bh], n_all, chunk))] = int32_t(i);
  for (size_t j = 0; j < it64.size(); ++j) {
    const int64_t L = j < n64 ? int64_t(j) + pre128[it64[j].bh + 1] : int64_t(it128.size() + j);
    order[size_t(launch_position(L, n_all, chunk))] = ~int32_t(j);
  }
  // each XCD's last kFwdTail entries longest-first (fwd_tail_cost, ties in launch order)
  for (int x = 0; x < kXcds; ++x) {
    const int64_t cnt = n_all > x ? (n_all - x + kXcds - 1) / kXcds : 0;
    const int64_t t = std::min<int64_t>(kFwdTail, cnt);
    std::vector<int32_t> tail;
    for (int64_t j = cnt - t; j < cnt; ++j) tail.push_back(order[size_t(j * kXcds + x)]);
    auto cost = [&](int32_t tag) {
      return tag >= 0 ? fwd_tail_cost(128, it128[size_t(tag)].n_pages) : fwd_tail_cost(64, it64[size_t(~tag)].n_pages);
    };
    std::stable_sort(tail.begin(), tail.end(), [&](int32_t a, int32_t b) { return cost(a) > cost(b); });
    for (int64_t j = cnt - t; j < cnt; ++j) order[size_t(j * kXcds + x)] = tail[size_t(j - (cnt - t))];
  }
  kpage_status s;
  if ((s = upload(pl, order, &pl->d_order, stream)) != KPAGE_OK) return s;
  if ((s = upload(pl, pages, &pl->d_pages, stream)) != KPAGE_OK) return s;
  if ((s = upload(pl, has_groups ? valid_all : F.valid, &pl->d_valid, stream)) != KPAGE_OK) return s;
  if (has_groups && (s = upload(pl, groups, &pl->d_groups, stream)) != KPAGE_OK) return s;
  if ((s = upload(pl, it128, &pl->d_items128, stream)) != KPAGE_OK) return s;
  if ((s = upload(pl, it64, &pl->d_items64, stream)) != KPAGE_OK) return s;
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  pl->n_items128 = int(it128.size());
  pl->n_items64 = int(it64.size());
  pl->fwd_on_device = true;
  return KPAGE_OK;
}

// device table -> host vector; false when the copy fails
template <class T>
bool copy_down(std::vector<T> &dst, const T *src, int64_t n) {
  dst.resize(size_t(std::max<int64_t>(n, 0)));
  return n <= 0 || hipMemcpy(dst.data(), src, size_t(n) * sizeof(T), hipMemcpyDeviceToHost) == hipSuccess;
}

// device-planned plans: the forward tables, copied for export
kpage_status ensure_forward_on_host(PlanT *pl) {
  if (pl->fwd_on_host) return KPAGE_OK;
  const DevFwdTables &T = pl->DF;
  FwdTables &F = pl->F;
  const int64_t GQ = int64_t(pl->P.slots) * pl->P.n_q;
  const bool ok = copy_down(F.route, T.route, GQ) &&
                  copy_down(F.walk_ptr, T.walk_ptr, int64_t(pl->P.slots) * (pl->P.n_q + 1)) &&
                  copy_down(F.walk, T.walk, T.walk_total) && copy_down(F.nfull, T.nfull, GQ) &&
                  copy_down(F.valid, T.valid, T.walk_total / 2) &&
                  copy_down(F.q64_queue, T.q64_queue, 2 * int64_t(T.n_q64)) &&
                  copy_down(F.q128_queue, T.q128_queue, 2 * int64_t(T.n_q128)) &&
                  copy_down(F.unpadded, T.unpadded, GQ);
  GroupTables &GT = pl->GT;
  GT.group_ptr = T.g_group_ptr;
  GT.walk_ptr = T.g_walk_ptr;
  const int64_t gw = T.g_walk_ptr.empty() ? 0 : T.g_walk_ptr.back();
  const bool gok = copy_down(GT.members, T.g_members, T.n_groups * kGroupMembers) &&
                   copy_down(GT.nfull, T.g_nfull, T.n_groups) && copy_down(GT.npages, T.g_npages, T.n_groups) &&
                   copy_down(GT.walk, T.g_walk, gw) && copy_down(GT.valid, T.g_valid, 2 * gw);
  if (!ok || !gok) return fail(KPAGE_ERR_HIP, "copying the forward tables to the host failed");
  pl->fwd_on_host = true;
  return KPAGE_OK;
}

void *plan_alloc(PlanT *pl, size_t bytes) {
  void *p = nullptr;
  if (hipMalloc(&p, std::max<size_t>(bytes, 16)) != hipSuccess) return nullptr;
  pl->allocations.push_back(p);
  return p;
}

// device-planned plans: the backward tables are built by kernels from the device
// descriptor and the forward planner's page table
kpage_status build_backward_on_device(PlanT *pl, hipStream_t stream) {
  std::string err;
  DevBwdTables &T = pl->DB;
  kpage_status s = build_backward_device(
      pl->DP, pl->DF.page_block, pl->P.q_group, stream, [pl](size_t b) { return plan_alloc(pl, b); }, &T, &err);
  if (s != KPAGE_OK) return fail(s, err);
  pl->d_bitems = T.items;
  pl->n_bitems = int(T.n_items);
  pl->d_reduce = T.reduce;
  pl->n_reduce = int(T.n_reduce);
  pl->n_partials = T.n_partials;
  pl->d_owners = T.owners;
  pl->d_kmask = T.kmask;
  pl->d_qpages = T.qpages;
  pl->d_adj = T.adj;
  pl->d_uncovered = T.uncovered;
  pl->d_uncovered_ptr = T.uncovered_ptr;
  pl->max_uncovered = T.max_uncovered;
  pl->d_qvalid = pl->DP.q_valid;
  pl->S.bwd_physical = T.bwd_physical;
  pl->S.bwd_useful_check = T.bwd_useful_check;
  pl->bwd_on_device = true;
  return KPAGE_OK;
}

kpage_status ensure_backward_on_host(PlanT *pl) {
  if (pl->B.built) return KPAGE_OK;
  if (!pl->device_planned) {
    build_backward(pl->P, &pl->B, &pl->S);
    return KPAGE_OK;
  }
  if (!pl->bwd_on_device) {  // export before the first backward call
    const kpage_status s = build_backward_on_device(pl, nullptr);
    if (s != KPAGE_OK) return s;
  }
  const DevBwdTables &T = pl->DB;
  BwdTables &B = pl->B;
  const int64_t G = pl->P.slots;
  const int64_t n_pairs = T.n_own * T.n_groups;  // (owner, group) pairs
  B.n_groups = T.n_groups;
  const bool ok = copy_down(B.owner_ptr, T.owner_ptr, G + 1) &&
                  copy_down(B.owners, T.owners, T.n_own * kOwnerSlots) && copy_down(B.aligned, T.aligned, T.n_own) &&
                  copy_down(B.revq_ptr, T.revq_ptr, n_pairs + 1) && copy_down(B.revq, T.revq, T.revq_total) &&
                  copy_down(B.qwalk_ptr, T.qwalk_ptr, n_pairs + 1) && copy_down(B.qwalk, T.qwalk, T.qwalk_total) &&
                  copy_down(B.adj, T.adj, T.qwalk_total / kOwnerSlots) &&
                  copy_down(B.bwd_queue, T.bwd_queue, 2 * T.n_items) &&
                  copy_down(B.uncovered_ptr, T.uncovered_ptr, G + 1) &&
                  copy_down(B.uncovered, T.uncovered, T.uncovered_total);
  if (!ok) return fail(KPAGE_ERR_HIP, "copying the backward tables to the host failed");
  B.built = true;
  return KPAGE_OK;
}

// Backward launch items from the exported work order: one per (owner, Q group) entry,
// launched in (bh, owner, group) order.  Owners with more than one item accumulate
// fp32 partials (one slot per item, consecutive in group order) that the reduce pass
// sums; an owner with a single item writes bf16 directly.
void make_bwd_items(const Problem &P, const BwdTables &B, std::vector<BwdItem> *items, std::vector<BwdReduce> *reduce,
                    int64_t *n_partials) {
  const int ng = B.n_groups;
  items->clear();
  reduce->clear();
  for (size_t i = 0; i < B.bwd_queue.size(); i += 2) {
    const int bh = B.bwd_queue[i], tg_local = B.bwd_queue[i + 1];
    const int64_t t = B.owner_ptr[P.slot_of(bh)] + tg_local / ng;
    const int64_t w = t * ng + tg_local % ng;
    BwdItem x{};
    x.qwalk_off = B.qwalk_ptr[w];
    x.n_steps = int32_t((B.qwalk_ptr[w + 1] - B.qwalk_ptr[w]) / 8);
    x.bh = bh;
    x.owner = int32_t(t);
    x.partial = tg_local % ng;  // group, until the slots are assigned below
    items->push_back(x);
  }
  std::stable_sort(items->begin(), items->end(), [](const BwdItem &a, const BwdItem &b) {
    if (a.bh != b.bh) return a.bh < b.bh;
    if (a.owner != b.owner) return a.owner < b.owner;
    return a.partial < b.partial;
  });
  int64_t n_part = 0;
  for (size_t i = 0; i < items->size();) {
    size_t j = i;
    while (j < items->size() && (*items)[j].bh == (*items)[i].bh && (*items)[j].owner == (*items)[i].owner) ++j;
    if (j - i > 1) {
      reduce->push_back(BwdReduce{(*items)[i].bh, (*items)[i].owner, int32_t(n_part), int32_t(j - i)});
      for (size_t k = i; k < j; ++k) (*items)[k].partial = int32_t(n_part++);
    } else {
      (*items)[i].partial = -1;
    }
    i = j;
  }
  *n_partials = n_part;
}

kpage_status ensure_backward_on_device(PlanT *pl, hipStream_t stream) {
  if (pl->bwd_on_device) return KPAGE_OK;
  if (pl->device_planned) return build_backward_on_device(pl, stream);
  ensure_backward_on_host(pl);
  const Problem &P = pl->P;
  const BwdTables &B = pl->B;
  const int nk = P.n_kv;
  const size_t n_own = B.aligned.size();
  // row masks of owner pages (K/V sizes); query-row validity reaches the kernels
  // through LSE = -inf of invalid rows
  std::vector<uint32_t> kmask(n_own * kOwnerSlots, 0);
  for (int g = 0; g < P.slots; ++g) {
    const int32_t *ck = &P.kv_valid[size_t(g) * nk];
    const int64_t *ok = &P.kv_offset[size_t(g) * nk];
    std::vector<std::pair<int64_t, int>> starts;  // (first page, block)
    for (int k = 0; k < nk; ++k)
      if (ck[k] > 0) starts.emplace_back(ok[k] / kPageRows, k);
    std::sort(starts.begin(), starts.end());
    for (int64_t t = B.owner_ptr[g]; t < B.owner_ptr[g + 1]; ++t) {
      for (int i = 0; i < kOwnerSlots; ++i) {
        const int32_t pg = B.owners[size_t(t) * kOwnerSlots + i];
        if (pg < 0) continue;
        auto itb = std::upper_bound(starts.begin(), starts.end(), std::make_pair(int64_t(pg), 1 << 30));
        const int k = std::prev(itb)->second;
        const int j = int(pg - ok[k] / kPageRows);
        const int c = ck[k];
        kmask[size_t(t) * kOwnerSlots + i] = (j + 1) * kPageRows <= c ? kFullMask : ((1u << (c % kPageRows)) - 1u);
      }
    }
  }
  std::vector<int32_t> qpages = redirect_dummies(B.qwalk, B.qwalk_ptr);
  std::vector<int32_t> owners(B.owners);
  std::vector<BwdItem> items;
  std::vector<BwdReduce> reduce;
  make_bwd_items(P, B, &items, &reduce, &pl->n_partials);
  items = xcd_interleave(items, xcd_chunk_for(P.seq_q, P.seq_kv, P.head_dim));
  sort_xcd_tails(items);
  kpage_status s;
  if ((s = upload(pl, items, &pl->d_bitems, stream)) != KPAGE_OK) return s;
  if ((s = upload(pl, owners, &pl->d_owners, stream)) != KPAGE_OK) return s;
  if ((s = upload(pl, kmask, &pl->d_kmask, stream)) != KPAGE_OK) return s;
  if ((s = upload(pl, qpages, &pl->d_qpages, stream)) != KPAGE_OK) return s;
  if ((s = upload(pl, B.adj, &pl->d_adj, stream)) != KPAGE_OK) return s;
  if ((s = upload(pl, B.uncovered, &pl->d_uncovered, stream)) != KPAGE_OK) return s;
  if ((s = upload(pl, B.uncovered_ptr, &pl->d_uncovered_ptr, stream)) != KPAGE_OK) return s;
  if ((s = upload(pl, reduce, &pl->d_reduce, stream)) != KPAGE_OK) return s;
  int32_t *qv = nullptr;
  if ((s = upload(pl, P.q_valid, &qv, stream)) != KPAGE_OK) return s;
  pl->d_qvalid = qv;
  pl->n_reduce = int(reduce.size());
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  pl->n_bitems = int(items.size());
  for (int g = 0; g < P.slots; ++g)
    pl->max_uncovered = std::max(pl->max_uncovered, int(B.uncovered_ptr[g + 1] - B.uncovered_ptr[g]));
  pl->bwd_on_device = true;
  return KPAGE_OK;
}

bool bad_scale(float s) { return !(s > 0.f) || !std::isfinite(s); }

// byte offset of the partial slots in the backward workspace
size_t partials_offset(size_t rows) { return (2 * rows * 4 + 255) / 256 * 256; }

kpage_status count_partials(PlanT *pl) {
  if (pl->n_partials >= 0) return KPAGE_OK;
  if (pl->device_planned) return build_backward_on_device(pl, nullptr);  // sets n_partials
  const kpage_status s = ensure_backward_on_host(pl);
  if (s != KPAGE_OK) return s;
  std::vector<BwdItem> items;
  std::vector<BwdReduce> reduce;
  make_bwd_items(pl->P, pl->B, &items, &reduce, &pl->n_partials);
  return KPAGE_OK;
}

}  // namespace

extern "C" {

const char *kpage_last_error(void) { return g_last_error.c_str(); }

static kpage_status select_args(const kpage_select_layout *l, SelectArgs *a) {
  if (!l) return fail(KPAGE_ERR_INVALID, "layout is NULL");
  if (l->head_dim != 64 && l->head_dim != 128) return fail(KPAGE_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (l->batch < 1 || l->heads < 1) return fail(KPAGE_ERR_INVALID, "batch and heads must be >= 1");
  if (int64_t(l->batch) * l->heads > 65535) return fail(KPAGE_ERR_UNSUPPORTED, "batch * heads above 65535");
  if (l->n_q_blocks < 1 || l->n_kv_blocks < 1) return fail(KPAGE_ERR_INVALID, "n_q_blocks and n_kv_blocks must be >= 1");
  if (l->n_kv_blocks > kSelectMaxKv) return fail(KPAGE_ERR_UNSUPPORTED, "more than 4096 key blocks");
  if (l->seq_q != int64_t(128) * l->n_q_blocks) return fail(KPAGE_ERR_INVALID, "seq_q must equal 128 * n_q_blocks");
  if (l->seq_kv < 1) return fail(KPAGE_ERR_INVALID, "seq_kv must be >= 1");
  if (!l->q_valid || !l->kv_valid) return fail(KPAGE_ERR_INVALID, "q_valid and kv_valid are required");
  a->q_valid = l->q_valid;
  a->kv_valid = l->kv_valid;
  a->kv_offset = l->kv_offset;
  a->seq_q = l->seq_q;
  a->seq_kv = l->seq_kv;
  a->n_q = l->n_q_blocks;
  a->n_kv = l->n_kv_blocks;
  a->bh_count = l->batch * l->heads;
  return KPAGE_OK;
}

kpage_status kpage_select_workspace_size(const kpage_select_layout *layout, size_t *bytes) {
  if (!bytes) return fail(KPAGE_ERR_INVALID, "bytes is NULL");
  SelectArgs a{};
  const kpage_status s = select_args(layout, &a);
  if (s != KPAGE_OK) return s;
  *bytes = select_workspace(a, layout->head_dim).total;
  return KPAGE_OK;
}

kpage_status kpage_select_topk(const kpage_select_layout *layout, const void *q, const void *k, int32_t top_k,
                               int64_t *q2k_ptr, int32_t *q2k_idx, void *workspace, size_t workspace_bytes,
                               void *stream) {
  SelectArgs a{};
  kpage_status s = select_args(layout, &a);
  if (s != KPAGE_OK) return s;
  if (!q || !k || !q2k_ptr || !q2k_idx || !workspace) return fail(KPAGE_ERR_INVALID, "tensor or output pointer is NULL");
  if (top_k < 1) return fail(KPAGE_ERR_INVALID, "top_k must be >= 1");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k)) % 16)
    return fail(KPAGE_ERR_INVALID, "q and k must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(KPAGE_ERR_INVALID, "workspace must be 256-byte aligned");
  if (workspace_bytes < select_workspace(a, layout->head_dim).total)
    return fail(KPAGE_ERR_INVALID, "workspace smaller than kpage_select_workspace_size()");
  const hipError_t e = launch_select(a, layout->head_dim, top_k, q, k, workspace, q2k_ptr, q2k_idx,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "selection launch");
  return KPAGE_OK;
}

static kpage_status cluster_args(const kpage_select_clusters *c, ClusterArgs *a) {
  if (!c) return fail(KPAGE_ERR_INVALID, "clusters descriptor is NULL");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(KPAGE_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c->batch < 1 || c->heads < 1) return fail(KPAGE_ERR_INVALID, "batch and heads must be >= 1");
  if (int64_t(c->batch) * c->heads > 65535) return fail(KPAGE_ERR_UNSUPPORTED, "batch * heads above 65535");
  if (c->n_q_clusters < 1 || c->n_kv_clusters < 1 || c->n_q_blocks < 1 || c->n_kv_blocks < 1)
    return fail(KPAGE_ERR_INVALID, "cluster and block counts must be >= 1");
  if (c->n_kv_clusters > kSelectMaxKv) return fail(KPAGE_ERR_UNSUPPORTED, "more than 4096 K clusters");
  if (!c->q_centroids || !c->kv_centroids || !c->q_cluster_size || !c->kv_cluster_size || !c->q_block_cluster ||
      !c->kv_block_cluster)
    return fail(KPAGE_ERR_INVALID, "a clusters array is NULL");
  a->q_cent = c->q_centroids;
  a->k_cent = c->kv_centroids;
  a->q_size = c->q_cluster_size;
  a->k_size = c->kv_cluster_size;
  a->q_block_cluster = c->q_block_cluster;
  a->k_block_cluster = c->kv_block_cluster;
  a->n_qc = c->n_q_clusters;
  a->n_kc = c->n_kv_clusters;
  a->n_q = c->n_q_blocks;
  a->n_kv = c->n_kv_blocks;
  a->bh_count = c->batch * c->heads;
  return KPAGE_OK;
}

kpage_status kpage_select_top_p_workspace_size(const kpage_select_clusters *c, size_t *bytes) {
  if (!bytes) return fail(KPAGE_ERR_INVALID, "bytes is NULL");
  ClusterArgs a{};
  const kpage_status s = cluster_args(c, &a);
  if (s != KPAGE_OK) return s;
  *bytes = cluster_workspace(a, c->head_dim).total;
  return KPAGE_OK;
}

kpage_status kpage_select_top_p(const kpage_select_clusters *c, double top_p, double scale, int64_t *q2k_ptr,
                                int32_t *q2k_idx, void *workspace, size_t workspace_bytes, void *stream) {
  ClusterArgs a{};
  kpage_status s = cluster_args(c, &a);
  if (s != KPAGE_OK) return s;
  if (!(top_p > 0.0 && top_p <= 1.0)) return fail(KPAGE_ERR_INVALID, "top_p must lie in (0, 1]");
  if (!(scale > 0.0) || !std::isfinite(scale)) return fail(KPAGE_ERR_INVALID, "scale must be positive and finite");
  if (!q2k_ptr || !q2k_idx || !workspace) return fail(KPAGE_ERR_INVALID, "output or workspace pointer is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(KPAGE_ERR_INVALID, "workspace must be 256-byte aligned");
  if (workspace_bytes < cluster_workspace(a, c->head_dim).total)
    return fail(KPAGE_ERR_INVALID, "workspace smaller than kpage_select_top_p_workspace_size()");
  a.top_p = top_p;
  a.scale = scale;
  const hipError_t e = launch_select_top_p(a, c->head_dim, workspace, q2k_ptr, q2k_idx, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cluster selection launch");
  return KPAGE_OK;
}

kpage_status kpage_plan(const kpage_problem *problem, const kpage_plan_opts *opts, kpage_plan_t **out) {
  if (!out) return fail(KPAGE_ERR_INVALID, "out is NULL");
  *out = nullptr;
  PlanT *pl = new (std::nothrow) PlanT();
  if (!pl) return fail(KPAGE_ERR_OOM, "host allocation failed");
  std::string err;
  int a64 = 16, a128 = 8;
  kpage_status s = load_problem(problem, opts, &pl->P, &a64, &a128, &err);
  if (s != KPAGE_OK) {
    delete pl;
    return fail(s, err);
  }
  pl->F.align64 = a64;
  pl->F.align128 = a128;
  try {
    build_forward(pl->P, &pl->F, &pl->S);
    build_groups(pl->P, pl->F, &pl->GT);
  } catch (const std::bad_alloc &) {
    delete pl;
    return fail(KPAGE_ERR_OOM, "host allocation failed while planning");
  }
  *out = pl;
  g_last_error.clear();
  return KPAGE_OK;
}

static kpage_status plan_device_body(const kpage_problem *problem, int64_t q2k_nnz, const kpage_plan_opts *opts,
                                     void *stream, kpage_plan_t **out);

kpage_status kpage_plan_device(const kpage_problem *problem, int64_t q2k_nnz, const kpage_plan_opts *opts,
                               void *stream, kpage_plan_t **out) {
  return guarded([&] { return plan_device_body(problem, q2k_nnz, opts, stream, out); });
}

static kpage_status plan_device_body(const kpage_problem *problem, int64_t q2k_nnz, const kpage_plan_opts *opts,
                                     void *stream, kpage_plan_t **out) {
  if (!out) return fail(KPAGE_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (!problem) return fail(KPAGE_ERR_INVALID, "problem is NULL");
  // scalar checks of the host loader on a descriptor without arrays
  kpage_problem shell = *problem;
  if (!shell.q_valid || !shell.kv_valid || !shell.q2k_ptr || !shell.q2k_idx)
    return fail(KPAGE_ERR_INVALID, "q_valid, kv_valid, q2k_ptr and q2k_idx are required");
  if (q2k_nnz < 0) return fail(KPAGE_ERR_INVALID, "q2k_nnz must be >= 0");
  PlanT *pl = new (std::nothrow) PlanT();
  if (!pl) return fail(KPAGE_ERR_OOM, "host allocation failed");
  std::string err;
  int a64 = 16, a128 = 8;
  kpage_status s = load_scalars(&shell, opts, &pl->P, &a64, &a128, &err);
  if (s != KPAGE_OK) {
    delete pl;
    return fail(s, err);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Problem &P = pl->P;
  const int64_t G = P.slots, nq = P.n_q, nk = P.n_kv;
  auto alloc = [pl](size_t bytes) { return plan_alloc(pl, bytes); };
  auto own = [&](const void *src, size_t bytes) -> void * {  // plan-owned copy of a descriptor array
    void *d = alloc(bytes);
    if (d && bytes && hipMemcpyAsync(d, src, bytes, hipMemcpyDeviceToDevice, st) != hipSuccess) return nullptr;
    return d;
  };
  DevProblem &D = pl->DP;
  D.batch = P.batch; D.heads = P.heads; D.n_q = P.n_q; D.n_kv = P.n_kv; D.slots = P.slots;
  D.seq_q = P.seq_q; D.seq_kv = P.seq_kv; D.per_head = P.per_head; D.nnz = q2k_nnz;
  D.xcd_chunk = xcd_chunk_for(P.seq_q, P.seq_kv, P.head_dim);
  D.q_valid = static_cast<const int32_t *>(own(shell.q_valid, size_t(G * nq) * 4));
  D.kv_valid = static_cast<const int32_t *>(own(shell.kv_valid, size_t(G * nk) * 4));
  D.q2k_ptr = static_cast<const int64_t *>(own(shell.q2k_ptr, size_t(G * (nq + 1)) * 8));
  D.q2k_idx = static_cast<const int32_t *>(own(shell.q2k_idx, size_t(q2k_nnz) * 4));
  if (shell.kv_offset) {
    D.kv_offset = static_cast<const int64_t *>(own(shell.kv_offset, size_t(G * nk) * 8));
  } else {  // the plan keeps explicit offsets (host copies expect them)
    std::vector<int64_t> off(size_t(G * nk));
    for (int64_t i = 0; i < G * nk; ++i) off[size_t(i)] = int64_t(kBlockRows) * (i % nk);
    int64_t *d = static_cast<int64_t *>(alloc(off.size() * 8));
    if (d && hipMemcpy(d, off.data(), off.size() * 8, hipMemcpyHostToDevice) != hipSuccess) d = nullptr;
    D.kv_offset = d;
  }
  if (!D.q_valid || !D.kv_valid || !D.q2k_ptr || !D.q2k_idx || !D.kv_offset) {
    kpage_plan_destroy(pl);
    return fail(KPAGE_ERR_OOM, "device allocation or copy failed while planning");
  }
  pl->F.align64 = a64;
  pl->F.align128 = a128;
  s = build_forward_device(D, a64, a128, P.grouped, st, alloc, &pl->DF, &err);
  if (s != KPAGE_OK) {
    kpage_plan_destroy(pl);
    return fail(s, err);
  }
  pl->device_planned = true;
  pl->fwd_on_host = false;
  pl->S = pl->DF.stats;
  pl->d_pages = pl->DF.pages;
  pl->d_valid = pl->DF.valid;
  pl->d_items128 = pl->DF.items128;
  pl->d_items64 = pl->DF.items64;
  pl->d_order = pl->DF.order;
  pl->d_groups = pl->DF.groups;
  pl->n_items128 = int(pl->DF.n_q128 + pl->DF.n_gitems);
  pl->n_items64 = int(pl->DF.n_q64 - pl->DF.n_members + pl->DF.n_zero);
  pl->fwd_on_device = true;
  *out = pl;
  g_last_error.clear();
  return KPAGE_OK;
}

kpage_status kpage_plan_upload(kpage_plan_t *plan, void *stream) {
  if (!plan) return fail(KPAGE_ERR_INVALID, "plan is NULL");
  return guarded([&] { return ensure_forward_on_device(plan, static_cast<hipStream_t>(stream)); });
}

kpage_status kpage_attn_fwd(kpage_plan_t *plan, const void *q, const void *k, const void *v, void *o, float *lse,
                            float softmax_scale, void *stream) {
  if (!plan) return fail(KPAGE_ERR_INVALID, "plan is NULL");
  if (!q || !k || !v || !o || !lse) return fail(KPAGE_ERR_INVALID, "tensor pointer is NULL");
  if (bad_scale(softmax_scale)) return fail(KPAGE_ERR_INVALID, "softmax_scale must be positive and finite");
  hipStream_t st = static_cast<hipStream_t>(stream);
  kpage_status s = guarded([&] { return ensure_forward_on_device(plan, st); });
  if (s != KPAGE_OK) return s;
  FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.pages = plan->d_pages;
  a.valid = plan->d_valid;
  a.seq_q = plan->P.seq_q;
  a.seq_kv = plan->P.seq_kv;
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.groups = plan->d_groups;
  FwdArgs a64 = a;
  a.items = plan->d_items128;
  a.order = plan->d_order;
  a.n_items = plan->n_items128;
  a64.items = plan->d_items64;
  a64.n_items = plan->n_items64;
  const hipError_t e = launch_fwd(a, a64, plan->P.head_dim, st, plan->timer);
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return KPAGE_OK;
}

kpage_status kpage_bwd_workspace_size(kpage_plan_t *plan, size_t *bytes) {
  if (!plan || !bytes) return fail(KPAGE_ERR_INVALID, "plan or bytes is NULL");
  const size_t rows = size_t(plan->P.batch) * plan->P.heads * size_t(plan->P.seq_q);
  // fp32 LSE * log2(e), then fp32 D = rowsum(dO * O), each [BH, seq_q]; with Q groups,
  // then the fp32 dK/dV partials of owners split over several groups
  *bytes = 2 * rows * 4;
  if (plan->P.q_group > 0) {
    const kpage_status s = guarded([&] { return count_partials(plan); });
    if (s != KPAGE_OK) return s;
    *bytes = partials_offset(rows) + size_t(plan->n_partials) * 2 * 128 * size_t(plan->P.head_dim) * 4;
  }
  return KPAGE_OK;
}

// Backward launches on device tables that already exist, with `workspace` (device
// memory of at least the workspace size) holding lse2, D and the Q-group partials.
static kpage_status launch_backward(kpage_plan_t *plan, const void *q, const void *k, const void *v, const void *o,
                                    const float *lse, const void *dO, void *dq, void *dk, void *dv, void *workspace,
                                    float softmax_scale, hipStream_t st) {
  const Problem &P = plan->P;
  const size_t rows = size_t(P.batch) * P.heads * size_t(P.seq_q);
  // the K/V pass addresses delta as lse2 plus a 32-bit byte offset
  if (rows * 4 >= (size_t(1) << 31)) return fail(KPAGE_ERR_UNSUPPORTED, "more than 2^29 query rows in one call");
  BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dO; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.q_valid = plan->d_qvalid;
  a.lse2 = static_cast<float *>(workspace);
  a.delta = static_cast<float *>(workspace) + rows;
  a.items = plan->d_bitems;
  a.n_items = plan->n_bitems;
  a.owners = plan->d_owners;
  a.owner_kmask = plan->d_kmask;
  a.qpages = plan->d_qpages;
  a.adj = plan->d_adj;
  a.uncovered = plan->d_uncovered;
  a.uncovered_ptr = plan->d_uncovered_ptr;
  if (plan->n_reduce > 0 && reinterpret_cast<uintptr_t>(workspace) % 16)
    return fail(KPAGE_ERR_INVALID, "workspace must be 16-byte aligned when q_group > 0");
  a.reduce = plan->d_reduce;
  a.n_reduce = plan->n_reduce;
  a.part = plan->n_reduce > 0 ? reinterpret_cast<float *>(static_cast<char *>(workspace) + partials_offset(rows))
                              : nullptr;
  a.fitems128 = plan->d_items128;
  a.fitems64 = plan->d_items64;
  a.fgroups = plan->d_groups;
  a.forder = plan->d_order;
  a.n_fitems128 = plan->n_items128;
  a.n_fitems64 = plan->n_items64;
  a.pages = plan->d_pages;
  a.valid = plan->d_valid;
  a.seq_q = P.seq_q;
  a.seq_kv = P.seq_kv;
  a.heads = P.heads;
  a.n_q = P.n_q;
  a.per_head = P.per_head ? 1 : 0;
  a.bh_count = P.batch * P.heads;
  a.max_uncovered = plan->max_uncovered;
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  hipError_t e = launch_bwd(a, P.head_dim, st, plan->timer);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return KPAGE_OK;
}

kpage_status kpage_attn_bwd(kpage_plan_t *plan, const void *q, const void *k, const void *v, const void *o,
                            const float *lse, const void *dO, void *dq, void *dk, void *dv, void *workspace,
                            size_t workspace_bytes, float softmax_scale, void *stream) {
  if (!plan) return fail(KPAGE_ERR_INVALID, "plan is NULL");
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || !workspace)
    return fail(KPAGE_ERR_INVALID, "tensor or workspace pointer is NULL");
  if (bad_scale(softmax_scale)) return fail(KPAGE_ERR_INVALID, "softmax_scale must be positive and finite");
  size_t need = 0;
  kpage_status s = kpage_bwd_workspace_size(plan, &need);
  if (s != KPAGE_OK) return s;
  if (workspace_bytes < need) return fail(KPAGE_ERR_INVALID, "workspace smaller than kpage_bwd_workspace_size()");
  hipStream_t st = static_cast<hipStream_t>(stream);
  s = guarded([&] { return ensure_forward_on_device(plan, st); });  // the dQ pass walks the forward tables
  if (s != KPAGE_OK) return s;
  s = guarded([&] { return ensure_backward_on_device(plan, st); });
  if (s != KPAGE_OK) return s;
  return launch_backward(plan, q, k, v, o, lse, dO, dq, dk, dv, workspace, softmax_scale, st);
}

// ---- backward without allocation: the workspace is a static device array ----
//
// `scratch` is a file-scope device array; host code never passes its name to a kernel
// (on the host the name is only a stand-in for the symbol).  Its device address is
// looked up once per device with that device current and kept in g_scratch_ptr.
static __device__ __align__(256) char scratch[KPAGE_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices];

static kpage_status scratch_on_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(KPAGE_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KPAGE_OK;
}

kpage_status kpage_attn_bwd_noalloc(kpage_plan_t *plan, const void *q, const void *k, const void *v, const void *o,
                                    const float *lse, const void *dO, void *dq, void *dk, void *dv,
                                    float softmax_scale, void *stream) {
  if (!plan) return fail(KPAGE_ERR_INVALID, "plan is NULL");
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return fail(KPAGE_ERR_INVALID, "tensor pointer is NULL");
  if (bad_scale(softmax_scale)) return fail(KPAGE_ERR_INVALID, "softmax_scale must be positive and finite");
  const Problem &P = plan->P;
  const size_t rows = size_t(P.batch) * P.heads * size_t(P.seq_q);
  size_t need = 2 * rows * 4;
  if (need > KPAGE_NOALLOC_SCRATCH_BYTES)
    return fail(KPAGE_ERR_INVALID, "the backward needs " + std::to_string(need) + " bytes of workspace, more than the " +
                                       std::to_string(KPAGE_NOALLOC_SCRATCH_BYTES) + "-byte static scratch");
  if (!plan->fwd_on_device || !plan->bwd_on_device)
    return fail(KPAGE_ERR_INVALID, "the plan's device tables are not built yet: run kpage_attn_bwd once on this plan");
  if (plan->n_reduce > 0)
    need = partials_offset(rows) + size_t(plan->n_partials) * 2 * 128 * size_t(P.head_dim) * 4;
  if (need > KPAGE_NOALLOC_SCRATCH_BYTES)
    return fail(KPAGE_ERR_INVALID, "the backward needs " + std::to_string(need) + " bytes of workspace, more than the " +
                                       std::to_string(KPAGE_NOALLOC_SCRATCH_BYTES) + "-byte static scratch");
  void *ws = nullptr;
  const kpage_status s = scratch_on_current_device(&ws);
  if (s != KPAGE_OK) return s;
  return launch_backward(plan, q, k, v, o, lse, dO, dq, dk, dv, ws, softmax_scale, static_cast<hipStream_t>(stream));
}

kpage_status kpage_plan_stats(const kpage_plan_t *plan, kpage_pair_stats *out) {
  if (!plan || !out) return fail(KPAGE_ERR_INVALID, "plan or out is NULL");
  out->useful = plan->S.useful;
  out->whole_block = plan->S.whole_block;
  out->paged_m128 = plan->S.paged_m128;
  out->nominal = plan->S.nominal;
  out->scheduled = plan->S.scheduled;
  out->bwd_physical = plan->S.bwd_physical;
  out->bwd_useful_check = plan->S.bwd_useful_check;
  return KPAGE_OK;
}

kpage_status kpage_plan_export(kpage_plan_t *plan, int table_id, void *host_buf, size_t *bytes) {
  if (!plan || !bytes) return fail(KPAGE_ERR_INVALID, "plan or bytes is NULL");
  if (table_id < 0 || table_id >= KPAGE_T_COUNT) return fail(KPAGE_ERR_INVALID, "unknown table id");
  if (table_id >= KPAGE_T_OWNER_PTR && table_id <= KPAGE_T_UNCOVERED) {
    const kpage_status s = guarded([&] { return ensure_backward_on_host(plan); });
    if (s != KPAGE_OK) return s;
  } else {
    const kpage_status s = guarded([&] { return ensure_forward_on_host(plan); });
    if (s != KPAGE_OK) return s;
  }
  const void *src = nullptr;
  size_t n = 0;
  switch (table_id) {
#define KPAGE_TABLE(id, vec) \
  case id:                   \
    src = vec.data();        \
    n = vec.size() * sizeof(vec[0]); \
    break;
    KPAGE_TABLE(KPAGE_T_FWD_ROUTE, plan->F.route)
    KPAGE_TABLE(KPAGE_T_FWD_WALK_PTR, plan->F.walk_ptr)
    KPAGE_TABLE(KPAGE_T_FWD_WALK, plan->F.walk)
    KPAGE_TABLE(KPAGE_T_FWD_NFULL, plan->F.nfull)
    KPAGE_TABLE(KPAGE_T_FWD_VALID, plan->F.valid)
    KPAGE_TABLE(KPAGE_T_Q64_QUEUE, plan->F.q64_queue)
    KPAGE_TABLE(KPAGE_T_Q128_QUEUE, plan->F.q128_queue)
    KPAGE_TABLE(KPAGE_T_OWNER_PTR, plan->B.owner_ptr)
    KPAGE_TABLE(KPAGE_T_OWNERS, plan->B.owners)
    KPAGE_TABLE(KPAGE_T_OWNER_ALIGNED, plan->B.aligned)
    KPAGE_TABLE(KPAGE_T_REVQ_PTR, plan->B.revq_ptr)
    KPAGE_TABLE(KPAGE_T_REVQ, plan->B.revq)
    KPAGE_TABLE(KPAGE_T_QWALK_PTR, plan->B.qwalk_ptr)
    KPAGE_TABLE(KPAGE_T_QWALK, plan->B.qwalk)
    KPAGE_TABLE(KPAGE_T_ADJ, plan->B.adj)
    KPAGE_TABLE(KPAGE_T_BWD_QUEUE, plan->B.bwd_queue)
    KPAGE_TABLE(KPAGE_T_UNCOVERED_PTR, plan->B.uncovered_ptr)
    KPAGE_TABLE(KPAGE_T_UNCOVERED, plan->B.uncovered)
    KPAGE_TABLE(KPAGE_T_GROUP_PTR, plan->GT.group_ptr)
    KPAGE_TABLE(KPAGE_T_GROUP_MEMBERS, plan->GT.members)
    KPAGE_TABLE(KPAGE_T_GROUP_WALK_PTR, plan->GT.walk_ptr)
    KPAGE_TABLE(KPAGE_T_GROUP_WALK, plan->GT.walk)
    KPAGE_TABLE(KPAGE_T_GROUP_NFULL, plan->GT.nfull)
    KPAGE_TABLE(KPAGE_T_GROUP_VALID, plan->GT.valid)
#undef KPAGE_TABLE
  }
  if (!host_buf) {
    *bytes = n;
    return KPAGE_OK;
  }
  if (*bytes < n) return fail(KPAGE_ERR_INVALID, "host buffer too small for the table");
  if (n) std::memcpy(host_buf, src, n);
  *bytes = n;
  return KPAGE_OK;
}

kpage_status kpage_timing_enable(kpage_plan_t *plan, int enable) {
  if (!plan) return fail(KPAGE_ERR_INVALID, "plan is NULL");
  if (enable < 0 || enable > 2) return fail(KPAGE_ERR_INVALID, "enable must be 0, 1 or 2");
  if (plan->timer && plan->timer->split_routes() != (enable == 2)) {  // switching modes drops the record
    delete plan->timer;
    plan->timer = nullptr;
  }
  if (enable && !plan->timer) plan->timer = new (std::nothrow) EventTimer(enable == 2);
  if (enable && !plan->timer) return fail(KPAGE_ERR_OOM, "host allocation failed");
  if (!enable && plan->timer) {
    delete plan->timer;
    plan->timer = nullptr;
  }
  return KPAGE_OK;
}

kpage_status kpage_timing_read(kpage_plan_t *plan, int kernel_id, double *total_ms, int64_t *launches) {
  if (!plan || !total_ms || !launches) return fail(KPAGE_ERR_INVALID, "plan, total_ms or launches is NULL");
  if (kernel_id < 0 || kernel_id >= KPAGE_K_COUNT) return fail(KPAGE_ERR_INVALID, "unknown kernel id");
  *total_ms = 0;
  *launches = 0;
  if (!plan->timer) return KPAGE_OK;
  if (!plan->timer->read(kernel_id, total_ms, launches)) return fail(KPAGE_ERR_HIP, "reading HIP events failed");
  return KPAGE_OK;
}

void kpage_plan_destroy(kpage_plan_t *plan) {
  if (!plan) return;
  delete plan->timer;
  if (!plan->allocations.empty()) {
    (void)hipDeviceSynchronize();
    for (void *p : plan->allocations) (void)hipFree(p);
  }
  delete plan;
}

}  // extern "C"
