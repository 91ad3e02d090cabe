"""Pins for the integer planner oracle (CPU only).

Checks the oracle planner against values the paper prints (tests/golden/paper_facts.json),
a hand-worked tiny layout (tests/golden/tiny_layout.json), closed forms for 3D window
masks (tests/golden/window_counts.json) and invariants stated in sections 3.2-3.4 of the
KPage paper.
"""
import json
import os
from collections import Counter

import numpy as np
import pytest

from oracle import oracle_plan
from tests.problems import make_problem
from workloads import make_workload, tile_layout
from workloads.configs import _window_rows

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_paper_worked_example_tile_waste():
    """A 128 x 32 useful region in a whole 128 x 128 tile wastes 3/4 of it (sections 1 and 2)."""
    facts = _gold("paper_facts.json")
    p = make_problem([128], [32], [[0]])
    s = oracle_plan(p).stats
    assert 1 - s["useful"] / s["whole_block"] == facts["waste_useful_128x32_in_128x128_tile"]["value"]


def test_both_routes_present_the_same_tile_area():
    facts = _gold("paper_facts.json")
    area = facts["positions_per_physical_tile"]["value"]
    steps = facts["pages_per_step"]["value"]
    # one Q64 step and one Q128 step, each over exactly one step of full pages
    p = make_problem([64, 128], [128, 128], [[0, 1], [0]])
    t = oracle_plan(p)
    assert t.stats["scheduled"] == 2 * area
    assert t.fwd_walk_ptr[0, 1] - t.fwd_walk_ptr[0, 0] == steps["q64"]
    assert t.fwd_walk_ptr[0, 2] - t.fwd_walk_ptr[0, 1] == steps["q128"]


def test_tiny_layout_worked_by_hand():
    g = _gold("tiny_layout.json")
    w = make_workload(1)
    assert list(w.q_valid[0]) == g["valid"]
    t = oracle_plan(w)
    assert t.owners.tolist() == g["owners"]
    assert t.owner_aligned.tolist() == g["owner_aligned"]
    assert sorted(set(t.q64_queue[:, 1].tolist())) == g["q64_blocks"]
    assert sorted(set(t.q128_queue[:, 1].tolist())) == g["q128_blocks"]
    pages = sorted(p for o in g["owners"] for p in o if p >= 0)
    assert len(pages) == g["total_pages"]
    # tail masks appear in the validity words exactly where the tail pages sit
    for q in range(w.n_q):
        a, b = t.fwd_walk_ptr[0, q], t.fwd_walk_ptr[0, q + 1]
        walk = t.fwd_walk[a:b]
        words = t.fwd_valid[a // 2:b // 2]
        masks = [(int(wd) >> (16 * h)) & 0xFFFF for wd in words for h in (0, 1)]
        for pos, page in enumerate(walk):
            if page >= 0 and str(page // 8) in g["tail_masks"] and page % 8 == g["pages"][page // 8] - 1:
                assert masks[pos] == g["tail_masks"][str(page // 8)]


def _axis_sum(extents, r):
    return sum(extents[i] * extents[j] for i in range(len(extents)) for j in range(len(extents)) if abs(i - j) <= r)


def _axis_count(n, r):
    return sum(1 for i in range(n) for j in range(n) if abs(i - j) <= r)


def _extents(n, t):
    return [min(t, n - t * i) for i in range(-(-n // t))]


@pytest.mark.parametrize("case", _gold("window_counts.json")["cases"], ids=lambda c: f"{c['T']}x{c['H']}x{c['W']}")
def test_window_mask_counts_closed_form(case):
    T, H, W, r = case["T"], case["H"], case["W"], case["radius"]
    ext = [_extents(T, 4), _extents(H, 4), _extents(W, 8)]
    useful = np.prod([_axis_sum(e, rr) for e, rr in zip(ext, r)])
    edges = np.prod([_axis_count(len(e), rr) for e, rr in zip(ext, r)])
    assert useful == case["useful"] and edges == case["edges"]
    _, c, coords = tile_layout(T, H, W)
    rows, _ = _window_rows(coords, r)
    p = make_problem(c, c, rows)
    s = oracle_plan(p).stats
    assert s["useful"] == useful
    assert s["whole_block"] == 128 * 128 * edges
    for key in ("paged_m128", "nominal", "scheduled"):
        assert s[key] == case[key], key


def _check_invariants(p, t, align64=16, align128=8):
    facts = _gold("paper_facts.json")
    G = p.q_valid.shape[0]
    for g in range(G):
        ck, ok = p.kv_valid[g], p.kv_offset[g]
        pages_of = {k: [int(ok[k]) // 16 + j for j in range(-(-int(ck[k]) // 16))] for k in range(p.n_kv)}
        for k in range(p.n_kv):
            assert 16 * len(pages_of[k]) - int(ck[k]) <= facts["max_padding_rows_per_block"]["value"]
        for q in range(p.n_q):
            a, b = t.fwd_walk_ptr[g, q], t.fwd_walk_ptr[g, q + 1]
            walk = t.fwd_walk[a:b]
            cq = int(p.q_valid[g, q])
            if cq == 0:
                assert len(walk) == 0 and t.fwd_route[g, q] == 0
                continue
            G_ = align64 if cq <= 64 else align128
            assert t.fwd_route[g, q] == (64 if cq <= 64 else 128)
            assert len(walk) % G_ == 0 and np.sum(walk < 0) < G_
            # graph unchanged: the walk's real pages are exactly the pages of the selected blocks
            expect = Counter(pg for k in p.q2k_idx[p.q2k_ptr[g, q]:p.q2k_ptr[g, q + 1]] for pg in pages_of[int(k)])
            assert Counter(int(x) for x in walk if x >= 0) == expect
            masks = [(int(wd) >> (16 * h)) & 0xFFFF for wd in t.fwd_valid[a // 2:b // 2] for h in (0, 1)]
            nf = int(t.fwd_nfull[g, q])
            assert all((m == 0xFFFF) == (i < nf) for i, m in enumerate(masks))
            assert all(m == 0 for m, x in zip(masks, walk) if x < 0)
        # owners: each page in exactly one owner, no block crosses an owner
        owners = t.owners[t.owner_ptr[g]:t.owner_ptr[g + 1]]
        seen = Counter(int(x) for o in owners for x in o if x >= 0)
        assert all(v == 1 for v in seen.values())
        assert set(seen) == {pg for k in range(p.n_kv) for pg in pages_of[k]}
        where = {int(x): i for i, o in enumerate(owners) for x in o if x >= 0}
        for k in range(p.n_kv):
            assert len({where[pg] for pg in pages_of[k]}) <= 1
        # reverse-Q lists equal the brute-force reverse neighbourhoods
        for ti, o in enumerate(owners):
            ot = int(t.owner_ptr[g]) + ti
            R = t.revq[t.revq_ptr[ot]:t.revq_ptr[ot + 1]].tolist()
            blocks = {k for k in range(p.n_kv) if pages_of[k] and where[pages_of[k][0]] == ti}
            brute = sorted({q for q in range(p.n_q) if int(p.q_valid[g, q]) > 0 and
                            any(int(k) in blocks for k in p.q2k_idx[p.q2k_ptr[g, q]:p.q2k_ptr[g, q + 1]])})
            assert R == brute
        # Q-page walks: full Q blocks first, then the pages of partial ones; adjacency from the graph
        edges = {(q, int(k)) for q in range(p.n_q) for k in p.q2k_idx[p.q2k_ptr[g, q]:p.q2k_ptr[g, q + 1]]}
        block_of_page = {pg: k for k in range(p.n_kv) for pg in pages_of[k]}
        for ti, o in enumerate(owners):
            ot = int(t.owner_ptr[g]) + ti
            R = t.revq[t.revq_ptr[ot]:t.revq_ptr[ot + 1]].tolist()
            qw = t.qwalk[t.qwalk_ptr[ot]:t.qwalk_ptr[ot + 1]]
            assert len(qw) % 8 == 0 and np.sum(qw < 0) < 8
            real = [int(x) for x in qw if x >= 0]
            assert Counter(real) == Counter(8 * q + j for q in R for j in range(-(-int(p.q_valid[g, q]) // 16)))
            fullness = [int(p.q_valid[g, x // 8]) == 128 for x in real]
            assert fullness == sorted(fullness, reverse=True)
            for s_ in range(len(qw) // 8):
                word = int(t.adj[int(t.qwalk_ptr[ot]) // 8 + s_])
                for j in range(8):
                    for i in range(8):
                        qp, kp = int(qw[8 * s_ + j]), int(o[i])
                        want = qp >= 0 and kp >= 0 and (qp // 8, block_of_page[kp]) in edges
                        assert bool(word >> (8 * j + i) & 1) == want
    # queues: longest unpadded walk first
    for queue in (t.q64_queue, t.q128_queue):
        lens = []
        for bh, q in queue:
            g = bh if p.per_head else 0
            a, b = t.fwd_walk_ptr[g, q], t.fwd_walk_ptr[g, q + 1]
            lens.append(int(np.sum(t.fwd_walk[a:b] >= 0)))
        assert lens == sorted(lens, reverse=True)
    s = t.stats
    assert s["bwd_useful_check"] == s["useful"]
    assert s["useful"] <= s["nominal"] <= s["paged_m128"] <= s["whole_block"]
    assert s["nominal"] <= s["scheduled"]


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_invariants_on_shared_layout_workloads(cfg):
    w = make_workload(cfg, heads=[0])
    _check_invariants(w, oracle_plan(w))


def test_invariants_on_independent_partitions():
    w = make_workload(5, heads=[0, 1])
    _check_invariants(w, oracle_plan(w))


def test_invariants_on_random_small_layouts():
    rng = np.random.default_rng(42)
    for trial in range(30):
        n_q, n_kv = int(rng.integers(1, 12)), int(rng.integers(1, 12))
        cq = rng.choice([0, 1, 15, 16, 17, 63, 64, 65, 100, 127, 128], size=n_q)
        ck = rng.choice([0, 1, 15, 16, 17, 63, 64, 65, 100, 127, 128], size=n_kv)
        rows = [sorted(rng.choice(n_kv, size=int(rng.integers(0, n_kv + 1)), replace=False).tolist())
                for _ in range(n_q)]
        p = make_problem(cq, ck, rows)
        _check_invariants(p, oracle_plan(p))


def test_shared_layout_is_the_special_case_of_independent_partitions():
    """Section 3.4.1: n_Q = n_KV, c^Q = c^K and o_k = 128 k give the same tables as the shared layout."""
    import copy
    w = make_workload(3, heads=[0, 1])
    t1 = oracle_plan(w)
    w2 = copy.copy(w)
    w2.per_head = True
    nnz = len(w.q2k_idx)
    w2.q_valid = np.tile(w.q_valid, (2, 1))
    w2.kv_valid = np.tile(w.kv_valid, (2, 1))
    w2.kv_offset = np.tile(w.kv_offset, (2, 1))
    w2.q2k_ptr = np.concatenate([w.q2k_ptr, w.q2k_ptr + nnz])
    w2.q2k_idx = np.concatenate([w.q2k_idx, w.q2k_idx])
    t2 = oracle_plan(w2)
    for f in ("fwd_route", "fwd_nfull"):
        assert np.array_equal(np.tile(getattr(t1, f), (2, 1)), getattr(t2, f)), f
    n_walk = len(t1.fwd_walk)
    assert np.array_equal(np.concatenate([t1.fwd_walk_ptr, t1.fwd_walk_ptr + n_walk]), t2.fwd_walk_ptr)
    for f in ("fwd_walk", "fwd_valid", "owners", "owner_aligned", "revq", "qwalk", "adj"):
        assert np.array_equal(np.concatenate([getattr(t1, f)] * 2), getattr(t2, f)), f
    for f in ("q64_queue", "q128_queue", "bwd_queue"):
        assert np.array_equal(getattr(t1, f), getattr(t2, f)), f
    assert t1.stats == t2.stats


def test_adjacency_marks_only_graph_edges():
    """A Q block connected to one of two blocks sharing an owner gets page pairs for that block only (3.3.3)."""
    p = make_problem([128, 128], [32, 32], [[0], [1]])
    t = oracle_plan(p)
    assert t.owners.tolist() == [[0, 1, 8, 9, -1, -1, -1, -1]]
    assert t.revq.tolist() == [0, 1]
    assert len(t.adj) == 2
    for s, qb in enumerate((0, 1)):
        word = int(t.adj[s])
        for j in range(8):
            for i in range(8):
                want = i < 4 and ((qb == 0 and i < 2) or (qb == 1 and 2 <= i < 4))
                assert bool(word >> (8 * j + i) & 1) == want


def test_uncovered_pages_worked_by_hand():
    """Pages outside every footprint of a layout with gaps, worked by hand: footprints are
    pages 28-31 (c=50 at row 448), 0-7 (c=128 at 0), 10 (c=3 at 160), 12-18 (c=97 at 192),
    8 (c=16 at 128), none (c=0), 20-22 (c=33 at 320) of 32 pages."""
    ck = [50, 128, 3, 97, 16, 0, 33]
    off = [448, 0, 160, 192, 128, 0, 320]
    p = make_problem([128, 64], ck, [[0, 1], [2, 3]], heads=2, kv_offset=off, seq_kv=512, sort_rows=False)
    t = oracle_plan(p)
    assert t.uncovered.tolist() == [9, 11, 19, 23, 24, 25, 26, 27]
    assert t.uncovered_ptr.tolist() == [0, 8]


@pytest.mark.parametrize("cfg,heads", [(1, None), (2, None), (5, [3, 7])])
def test_uncovered_pages_complement_the_footprints(cfg, heads):
    """Per slot: uncovered count = seq_kv / 16 - sum of ceil(c_k / 16) (footprints are disjoint)."""
    w = make_workload(cfg, heads=heads)
    t = oracle_plan(w)
    for g in range(w.kv_valid.shape[0]):
        n = int(t.uncovered_ptr[g + 1] - t.uncovered_ptr[g])
        assert n == w.seq_kv // 16 - sum(-(-int(c) // 16) for c in w.kv_valid[g])


def _group_lists(t, n_groups):
    """revq lists per (owner, group), owner-major."""
    return [t.revq[t.revq_ptr[i]:t.revq_ptr[i + 1]].tolist() for i in range(len(t.revq_ptr) - 1)]


@pytest.mark.parametrize("q_group", [1, 3, 8])
def test_q_groups_partition_each_reverse_neighbourhood(q_group):
    """Section 3.3.2: the group lists of an owner are its one-group list cut at multiples of
    q_group, unless that list holds at most q_group Q blocks, which then stays whole in
    group 0; no group list exceeds q_group blocks (the bound the grouping serves); every
    edge's token pairs are still visited once (bwd_useful_check == useful); the work items
    are the non-empty (owner, group) pairs, and an owner without any keeps one item for
    group 0."""
    for w in (make_workload(1), make_workload(3, heads=[0]), make_workload(5, heads=[1])):
        one = oracle_plan(w)
        t = oracle_plan(w, q_group=q_group)
        n_groups = -(-w.n_q // q_group)
        R1 = _group_lists(one, 1)
        Rg = _group_lists(t, n_groups)
        assert len(Rg) == len(R1) * n_groups
        for o, r in enumerate(R1):
            parts = Rg[o * n_groups:(o + 1) * n_groups]
            assert sum(parts, []) == r
            assert max(len(part) for part in parts) <= q_group
            if len(r) <= q_group:
                assert parts[0] == r
            else:
                for grp, part in enumerate(parts):
                    assert all(grp * q_group <= q < (grp + 1) * q_group for q in part)
        assert t.stats["bwd_useful_check"] == t.stats["useful"] == one.stats["useful"]
        assert np.array_equal(t.owners, one.owners)
        # work items
        BH = w.batch * w.heads
        want = set()
        for bh in range(BH):
            g = bh if w.per_head else 0
            for o in range(int(t.owner_ptr[g + 1] - t.owner_ptr[g])):
                oo = int(t.owner_ptr[g]) + o
                grps = [grp for grp in range(n_groups) if Rg[oo * n_groups + grp]] or [0]
                want |= {(bh, o * n_groups + grp) for grp in grps}
        got = [tuple(x) for x in t.bwd_queue.tolist()]
        assert len(got) == len(set(got)) and set(got) == want


def test_q_group_not_below_n_q_is_one_group():
    w = make_workload(3, heads=[0])
    a, b = oracle_plan(w), oracle_plan(w, q_group=w.n_q)
    for f in ("revq_ptr", "revq", "qwalk_ptr", "qwalk", "adj", "bwd_queue"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert a.stats == b.stats


def test_q_groups_worked_by_hand():
    """Two K blocks in one owner (c = 32 each), Q blocks 0..3 full: q0 -> k0, q1 -> k1, q3 -> k0.
    With q_group = 2 the owner's list [0, 1, 3] splits into [0, 1] and [3]."""
    p = make_problem([128, 128, 128, 128], [32, 32], [[0], [1], [], [0]])
    t = oracle_plan(p, q_group=2)
    assert t.owners.tolist() == [[0, 1, 8, 9, -1, -1, -1, -1]]
    assert t.revq_ptr.tolist() == [0, 2, 3]
    assert t.revq.tolist() == [0, 1, 3]
    assert t.qwalk_ptr.tolist() == [0, 16, 24]
    assert t.qwalk.tolist() == list(range(0, 16)) + list(range(24, 32))
    # group 0 (2 steps) before group 1 (1 step)
    assert t.bwd_queue.tolist() == [[0, 0], [0, 1]]
    full = (1 << 64) - 1
    k0 = sum(1 << (8 * j + i) for j in range(8) for i in (0, 1))
    k1 = sum(1 << (8 * j + i) for j in range(8) for i in (2, 3))
    assert t.adj.tolist() == [k0, k1, k0]
    assert t.stats["bwd_physical"] == 3 * 128 * 128
    assert full != k0


def test_q_groups_keep_short_lists_whole_worked_by_hand():
    """Q blocks 0..3 full, K blocks 0 and 1 full (owners 0 and 1, pages 0..7 and 8..15);
    q1 -> k0, q2 -> k0 (owner 0: [1, 2]) and q0, q1, q3 -> k1 (owner 1: [0, 1, 3]).  With
    q_group = 2 the ranges are {0, 1} and {2, 3}: owner 0's two blocks are within the
    bound and stay in group 0 although they straddle the ranges; owner 1's three are cut
    into [0, 1] and [3].  Steps: (0, 0) 2, (0, 1) 0, (1, 0) 2, (1, 1) 1; work items by
    descending steps then owner, group: (0, 0), (0, 2), (0, 3)."""
    p = make_problem([128] * 4, [128, 128], [[1], [0, 1], [0], [1]])
    t = oracle_plan(p, q_group=2)
    assert t.owners.tolist() == [list(range(8)), list(range(8, 16))]
    assert t.revq_ptr.tolist() == [0, 2, 2, 4, 5]
    assert t.revq.tolist() == [1, 2, 0, 1, 3]
    assert t.qwalk_ptr.tolist() == [0, 16, 16, 32, 40]
    assert t.qwalk.tolist() == list(range(8, 24)) + list(range(0, 16)) + list(range(24, 32))
    assert t.bwd_queue.tolist() == [[0, 0], [0, 2], [0, 3]]
    assert t.adj.tolist() == [(1 << 64) - 1] * 5
    assert t.stats["bwd_physical"] == t.stats["useful"] == 5 * 128 * 128


def _order_case(key):
    g = _gold("order_conventions.json")[key]
    return g


def test_walk_section_order_worked_by_hand():
    """Reading R12/R13: full pages in K_q order (not page order), then each partial block's
    tail page in K_q order, then dummies; masks two per word, even position low."""
    g = _order_case("walk_order")
    p = make_problem(g["q_valid"], g["kv_valid"], g["rows"], sort_rows=False)
    t = oracle_plan(p)
    for q, (walk, nf, words) in enumerate(zip(g["walks"], g["n_full"], g["valid_words"])):
        a, b = int(t.fwd_walk_ptr[0, q]), int(t.fwd_walk_ptr[0, q + 1])
        assert t.fwd_walk[a:b].tolist() == walk, q
        assert int(t.fwd_nfull[0, q]) == nf
        assert t.fwd_valid[a // 2:b // 2].tolist() == words, q


def test_queue_and_backward_order_ties_worked_by_hand():
    """Reading R14 (queue ties: unpadded pages, then b*H + h, then q) and R26 (backward
    work order: steps, then b*H + h, then owner) on a layout with ties in both."""
    g = _order_case("queue_ties")
    p = make_problem(g["q_valid"], g["kv_valid"], g["rows"], heads=g["heads"], sort_rows=False)
    t = oracle_plan(p)
    assert t.q128_queue.tolist() == g["q128_queue"]
    assert t.q64_queue.tolist() == g["q64_queue"]
    assert t.owners.tolist() == g["owners"]
    assert t.revq.tolist() == g["revq"]
    assert t.qwalk.tolist() == g["qwalk"]
    assert [int(x) for x in t.adj] == [int(x, 16) for x in g["adj"]]
    assert t.bwd_queue.tolist() == g["bwd_queue"]
    assert t.stats["useful"] == g["useful"] and t.stats["bwd_physical"] == g["bwd_physical"]


def test_q_group_work_order_worked_by_hand():
    """Reading R30: (owner, group) lists owner-major, items by steps, then b*H + h, owner,
    group, exported as (b*H + h, owner * n_groups + group)."""
    g0 = _order_case("queue_ties")
    g = _order_case("q_group_order")
    p = make_problem(g0["q_valid"], g0["kv_valid"], g0["rows"], heads=g0["heads"], sort_rows=False)
    t = oracle_plan(p, q_group=g["q_group"])
    assert t.revq_ptr.tolist() == g["revq_ptr"]
    assert t.bwd_queue.tolist() == g["bwd_queue"]
