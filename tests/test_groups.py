"""Group items of the host planner (CPU only: planning touches no device memory).

Query blocks of the M64 x N256 route with at most 32 valid rows whose walks overlap run
up to four at a time as one M128 x N128 item over the union of their walks.  These
tests check the exported group tables against the rule stated in kpage.h and
plan.cpp, re-derived here from the plan's own forward tables: membership (eligible
blocks, each in at most one group, the greedy choice by covered share), the union
walk (every member page once, the common full pages first, dummies only at the end),
the common full prefix (then the other pages every member selected) and every
member's validity words.
"""
import numpy as np
import pytest

import block_sparse_attention_11_amd as K
from tests.problems import make_problem
from workloads import make_workload

FULL = 0xFFFF


def _tables(plan):
    names = ("fwd_route", "fwd_walk_ptr", "fwd_walk", "fwd_valid", "group_ptr", "group_members",
             "group_walk_ptr", "group_walk", "group_nfull", "group_valid")
    return {n: K.kpage_plan_export(plan, n) for n in names}


def _walk(T, nq, g, q):
    """Real pages of block q's walk in slot g and the row mask of each."""
    ptr = T["fwd_walk_ptr"].reshape(-1, nq + 1)
    a, b = int(ptr[g, q]), int(ptr[g, q + 1])
    pages, masks = [], []
    for i in range(a, b):
        pg = int(T["fwd_walk"][i])
        if pg < 0:
            continue
        pages.append(pg)
        masks.append((int(T["fwd_valid"][i >> 1]) >> (16 * (i & 1))) & FULL)
    return pages, masks


def _greedy(cands, sets):
    """The grouping rule: in block order, a free block opens a group, which takes, among
    the free blocks that share a page with every member, the one with the largest share
    of its pages inside the group's union (ties: lower block) while that share is at
    least one half, up to four members."""
    free = {q: True for q in cands}
    groups = []
    for i, a in enumerate(cands):
        if not free[a]:
            continue
        free[a] = False
        grp, uni, inter = [a], set(sets[a]), set(sets[a])
        while len(grp) < 4:
            best, best_in, best_n = None, 0, 1
            for b in cands[i + 1:]:
                if not free[b] or not (inter & sets[b]):
                    continue
                inn = len(uni & sets[b])
                if best is None or inn * best_n > best_in * len(sets[b]):
                    best, best_in, best_n = b, inn, len(sets[b])
            if best is None or 2 * best_in < best_n:
                break
            free[best] = False
            grp.append(best)
            uni |= sets[best]
            inter &= sets[best]
        if len(grp) >= 2:
            groups.append(grp)
    return groups


def check_groups(problem, plan=None):
    plan = plan or K.kpage_plan(problem)
    T = _tables(plan)
    nq = problem.n_q
    G = problem.q_valid.shape[0]
    route = T["fwd_route"].reshape(G, nq)
    gptr = T["group_ptr"]
    assert gptr.shape == (G + 1,) and gptr[0] == 0 and np.all(np.diff(gptr) >= 0)
    members = T["group_members"].reshape(-1, 4)
    wptr = T["group_walk_ptr"]
    n_groups = members.shape[0]
    assert gptr[-1] == n_groups and wptr.shape == (n_groups + 1,) and T["group_nfull"].shape == (n_groups,)
    assert T["group_valid"].size == 2 * wptr[-1]
    total = 0
    for g in range(G):
        cands = [q for q in range(nq) if route[g, q] == 64 and 0 < problem.q_valid[g, q] <= 32
                 and _walk(T, nq, g, q)[0]]
        walks = {q: _walk(T, nq, g, q) for q in cands}
        sets = {q: set(walks[q][0]) for q in cands}
        want = _greedy(cands, sets)
        got = []
        for i in range(int(gptr[g]), int(gptr[g + 1])):
            mem = [int(x) for x in members[i]]
            k = sum(x >= 0 for x in mem)
            assert k >= 2 and all(x >= 0 for x in mem[:k]) and all(x < 0 for x in mem[k:]), mem
            got.append(mem[:k])
            a, b = int(wptr[i]), int(wptr[i + 1])
            walk = [int(x) for x in T["group_walk"][a:b]]
            assert (b - a) % 4 == 0
            n_real = sum(x >= 0 for x in walk)
            assert all(x >= 0 for x in walk[:n_real]) and all(x < 0 for x in walk[n_real:]), "dummies at the end"
            assert b - a - n_real < 4
            real = walk[:n_real]
            assert len(set(real)) == len(real), "a page appears once"
            assert set(real) == set().union(*(sets[q] for q in mem[:k]))
            pmask = {}
            for q in mem[:k]:
                pmask.update(zip(*walks[q]))
            # the common full prefix: full pages selected by every member, in the first
            # member's walk order; no further page is full in every member
            shared = [p for p in walks[mem[0]][0] if all(p in sets[q] for q in mem[:k])]
            common = [p for p in shared if pmask[p] == FULL]
            nf = int(T["group_nfull"][i])
            assert real[:nf] == common
            # then the other pages every member selected, then the rest member by member
            assert real[nf:len(shared)] == [p for p in shared if pmask[p] != FULL]
            rest = []
            for q in mem[:k]:
                rest += [p for p in walks[q][0] if p not in shared and p not in rest]
            assert real[len(shared):] == rest
            # validity words of each wave (member w, or none)
            words = T["group_valid"][2 * a:2 * b].reshape(4, (b - a) // 2)
            for w in range(4):
                q = mem[w]
                for j in range(b - a):
                    p = walk[j]
                    want_m = pmask[p] if (q >= 0 and p >= 0 and p in sets[q]) else 0
                    assert (int(words[w, j >> 1]) >> (16 * (j & 1))) & FULL == want_m, (i, w, j)
        assert got == want, (g, got, want)
        total += len(got)
    return total


@pytest.mark.parametrize("cfg,heads", [(3, [0]), (4, [0, 5]), (5, [3])])
def test_workload_groups_follow_the_rule(cfg, heads):
    w = make_workload(cfg, heads=heads)
    n = check_groups(w)
    if cfg in (3, 4):
        assert n > 0  # both layouts have blocks of at most 32 rows with overlapping walks


def test_hand_worked_groups():
    """Blocks 1-4 hold 20, 32, 8 and 32 rows (block 0, 128 rows, takes the other route).
    K blocks 0, 1, 3 are full (pages 0-7, 8-15, 24-31), K block 2 holds 10 rows (one
    tail page, 16).  Walks: blocks 1 and 2 [0..7, 16], block 3 [24..31], block 4
    [0..15].  Block 1 opens a group with union {0..7, 16}: block 2 has 9 of its 9 pages
    in it, block 4 8 of 16, block 3 none, so block 2 joins; then block 4 (share exactly
    one half) joins; block 3 (share 0) does not, and alone it forms no group.  Union
    walk: the pages that are full and selected by every member, in block 1's walk order
    (0..7), then block 1's remaining page 16, then block 4's pages 8..15, then 3
    dummies to the next multiple of 4."""
    cq = [128, 20, 32, 8, 32]
    ck = [128, 128, 10, 128]
    rows = [[0, 1, 2, 3], [0, 2], [0, 2], [3], [0, 1]]
    p = make_problem(cq, ck, rows, heads=1, head_dim=64)
    plan = K.kpage_plan(p)
    assert check_groups(p, plan) == 1
    T = _tables(plan)
    assert T["group_members"].tolist() == [1, 2, 4, -1]
    walk = T["group_walk"].tolist()
    assert walk[:8] == list(range(8)) and T["group_nfull"].tolist() == [8]
    assert sorted(walk[8:17]) == [8, 9, 10, 11, 12, 13, 14, 15, 16]
    assert walk[8] == 16  # block 1's tail page before block 4's pages
    assert len(walk) == 20 and walk[17:] == [-1, -1, -1]


def test_ungrouped_plan_has_no_groups():
    w = make_workload(3, heads=[0])
    plan = K.kpage_plan(w, grouped=False)
    T = _tables(plan)
    assert T["group_members"].size == 0 and T["group_walk"].size == 0
    assert T["group_ptr"].tolist() == [0, 0]


def test_random_layouts_follow_the_rule():
    rng = np.random.default_rng(41)
    sizes = [1, 7, 8, 15, 16, 17, 31, 32, 33, 64, 100, 128]
    for _ in range(40):
        n_q, n_kv = int(rng.integers(2, 14)), int(rng.integers(1, 10))
        cq = rng.choice(sizes, size=n_q)
        ck = rng.choice([0, 5, 16, 17, 64, 127, 128], size=n_kv)
        base = rng.permutation(n_kv)[:max(1, n_kv // 2)].tolist()
        rows = []
        for _q in range(n_q):
            extra = rng.permutation(n_kv)[:int(rng.integers(0, 3))].tolist()
            rows.append(sorted(set(base[:int(rng.integers(1, len(base) + 1))] + extra)))
        p = make_problem(cq, ck, rows, heads=2, head_dim=64)
        check_groups(p)


@pytest.mark.parametrize("rows_past,grouped", [(0, True), (16, False)])
def test_grouping_stops_past_the_page_bitset_limit(rows_past, grouped):
    """Both planners group only while a page bitset fits 2048 words (seq_kv up to 2^21
    rows); one page more and every block runs alone."""
    limit = 2048 * 64 * 16
    seq_kv = limit + rows_past
    # K blocks 0 and 1 at the start, block 2 ending at seq_kv
    p = make_problem([20, 32, 8], [128, 128, 128], [[0, 1], [0, 1], [0, 2]], heads=1, head_dim=64,
                     kv_offset=[0, 128, seq_kv - 128], seq_kv=seq_kv)
    plan = K.kpage_plan(p)
    members = K.kpage_plan_export(plan, "group_members")
    if grouped:
        assert members.tolist() == [0, 1, 2, -1]
        check_groups(p, plan)
    else:
        assert members.size == 0


def many_small_blocks_problem(per_slot):
    """Two graph slots of `per_slot` 8-row query blocks that all select K block 0, over a
    K/V sequence of 2^21 rows (page bitsets of 2048 words each)."""
    from tests.problems import Problem
    seq_kv = 2048 * 64 * 16
    G, n_kv = 2, 2
    qv = np.full((G, per_slot), 8, dtype=np.int32)
    kv = np.full((G, n_kv), 128, dtype=np.int32)
    off = np.tile(np.array([0, seq_kv - 128], dtype=np.int64), (G, 1))
    ptr = np.tile(np.arange(per_slot + 1, dtype=np.int64), (G, 1))
    ptr[1] += per_slot
    idx = np.zeros(G * per_slot, dtype=np.int32)
    return Problem(batch=1, heads=G, head_dim=64, n_q=per_slot, n_kv=n_kv, seq_q=128 * per_slot, seq_kv=seq_kv,
                   per_head=True, q_valid=qv, kv_valid=kv, kv_offset=off, q2k_ptr=ptr, q2k_idx=idx)


def test_grouping_stops_past_the_total_bitset_limit():
    """2 x 8193 candidates of 2048-word bitsets pass the 2^25-word limit of all slots'
    bitsets together: no slot groups."""
    plan = K.kpage_plan(many_small_blocks_problem(8193))
    assert K.kpage_plan_export(plan, "group_members").size == 0
    assert K.kpage_plan_export(plan, "group_ptr").tolist() == [0, 0, 0]
