// Host-side planner of the KPage page tables (KPage paper, sections 3.2-3.4).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "kpage.h"

namespace kpage {

constexpr int kPageRows = 16;
constexpr int kBlockRows = 128;
constexpr int kOwnerSlots = 8;
constexpr uint32_t kFullMask = 0xFFFFu;

struct Problem {
  int batch = 0, heads = 0, head_dim = 0, n_q = 0, n_kv = 0, slots = 0;
  int64_t seq_q = 0, seq_kv = 0;
  bool per_head = false;
  int q_group = 0;  // Q blocks per backward Q group; 0 = one group
  bool grouped = true;  // run small query blocks in group items (build_groups)
  std::vector<int32_t> q_valid, kv_valid;   // [slots][n]
  std::vector<int64_t> kv_offset;           // [slots][n_kv]
  std::vector<int64_t> q2k_ptr;             // [slots][n_q + 1]
  std::vector<int32_t> q2k_idx;
  int slot_of(int bh) const { return per_head ? bh : 0; }
};

struct PairStats {
  uint64_t useful = 0, whole_block = 0, paged_m128 = 0, nominal = 0, scheduled = 0;
  uint64_t bwd_physical = 0, bwd_useful_check = 0;
};

// Forward tables, concatenated over graph slots.
struct FwdTables {
  int align64 = 16, align128 = 8;
  std::vector<int32_t> route;       // [slots][n_q]
  std::vector<int64_t> walk_ptr;    // [slots][n_q + 1]
  std::vector<int32_t> walk;        // page ids, -1 dummy
  std::vector<int32_t> nfull;       // [slots][n_q]
  std::vector<uint32_t> valid;      // 2 page masks per word
  std::vector<int32_t> q64_queue;   // pairs (bh, q)
  std::vector<int32_t> q128_queue;  // pairs (bh, q)
  std::vector<int32_t> unpadded;    // [slots][n_q] real pages per walk
};

// Group items (launch-level, not part of the paper's tables): per graph slot, query
// blocks of the M64 x N256 route with at most 32 valid rows whose walks overlap are run
// four at a time as one M128 x N128 item over the union of their walks, one member per
// wave.  The GPU planner builds the same tables (plan_dev.hip).
constexpr int kGroupMembers = 4;
constexpr int kGroupMaxRows = 32;
// Grouping runs where its working sets fit the GPU planner's LDS (both planners apply
// the same limits): page bitsets of at most 2048 words (seq_kv up to 2^21 rows) and at
// most 16384 candidate blocks per graph slot.
constexpr int kGroupMaxWords = 2048;
constexpr int kGroupMaxCands = 16384;
// and the page bitsets of all slots' candidates together at most 2^25 words (256 MiB of
// device memory while the GPU planner groups); beyond that no slot groups
constexpr int64_t kGroupMaxBitsetWords = int64_t(1) << 25;
struct GroupTables {
  std::vector<int64_t> group_ptr;   // [slots + 1] offsets into the group list
  std::vector<int32_t> members;     // [n_groups][4] query blocks, -1 = none (at least 2 members)
  std::vector<int64_t> walk_ptr;    // [n_groups + 1] union walks, multiples of 4 entries
  std::vector<int32_t> walk;        // page ids, -1 dummy (only at the end)
  std::vector<int32_t> nfull;       // [n_groups] leading pages that are full and in every member's walk
  std::vector<int32_t> npages;      // [n_groups] real pages of the union walk
  std::vector<uint32_t> valid;      // member w of group i: words [2 walk_ptr[i] + w len / 2, + len / 2)
  std::vector<uint8_t> in_group;    // [slots][n_q] 1 when the block is a group member
};

// Backward tables, concatenated over graph slots.
struct BwdTables {
  bool built = false;
  int n_groups = 1;                 // Q groups (section 3.3.2)
  std::vector<int64_t> owner_ptr;   // [slots + 1]
  std::vector<int32_t> owners;      // [n_own][8]
  std::vector<uint8_t> aligned;     // [n_own]
  std::vector<int64_t> revq_ptr;    // [n_own * n_groups + 1], per (owner, group), owner-major
  std::vector<int32_t> revq;
  std::vector<int64_t> qwalk_ptr;   // [n_own * n_groups + 1]
  std::vector<int32_t> qwalk;
  std::vector<uint64_t> adj;        // one word per step
  std::vector<int32_t> bwd_queue;   // pairs (bh, owner within slot * n_groups + group)
  std::vector<int64_t> uncovered_ptr;  // [slots + 1] K/V pages outside every block footprint
  std::vector<int32_t> uncovered;
};

// Validates the scalar fields of the C descriptor and copies them (no array access).
kpage_status load_scalars(const kpage_problem *p, const kpage_plan_opts *o, Problem *out, int *align64,
                          int *align128, std::string *err);
// Validates the C descriptor and copies it.  Returns KPAGE_OK or an error with `err` set.
kpage_status load_problem(const kpage_problem *p, const kpage_plan_opts *o, Problem *out, int *align64,
                          int *align128, std::string *err);
void build_forward(const Problem &p, FwdTables *t, PairStats *s);
void build_backward(const Problem &p, BwdTables *t, PairStats *s);
// Group items of the forward and dQ launches (empty tables when p.grouped is false).
void build_groups(const Problem &p, const FwdTables &f, GroupTables *t);

}  // namespace kpage
