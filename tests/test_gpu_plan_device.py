"""GPU-built plans (kpage_plan_device) against host-built plans (kpage_plan).

The host planner is pinned bit for bit to the oracle planner by the CPU tests, so
equality of every exported table (forward walks, routes, masks, queues; backward
owners, reverse-Q lists, Q-page walks, adjacency words, work order, uncovered pages)
and pair count with the host plan is equality with the oracle.  Attention through
both plans must then be bitwise equal (same kernels, same launch order), forward and
backward; the device plan builds both table sets with kernels, without copying its
descriptor to the host.
"""
import copy
import sys
import time

import numpy as np
import pytest
import torch

import block_sparse_attention_11_amd as K
from tests.problems import make_problem, random_tensors
from tests.test_gpu_fwd import EDGE_CASES
from workloads import make_workload

pytestmark = pytest.mark.gpu

FWD_TABLES = ("fwd_route", "fwd_walk_ptr", "fwd_walk", "fwd_nfull", "fwd_valid", "q64_queue", "q128_queue",
              "group_ptr", "group_members", "group_walk_ptr", "group_walk", "group_nfull", "group_valid")
BWD_TABLES = ("owner_ptr", "owners", "owner_aligned", "revq_ptr", "revq", "qwalk_ptr", "qwalk", "adj", "bwd_queue",
              "uncovered_ptr", "uncovered")
FWD_STATS = ("useful", "whole_block", "paged_m128", "nominal", "scheduled")
BWD_STATS = ("bwd_physical", "bwd_useful_check")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def same_plans(p, label, bwd=True, **opts):
    h = K.kpage_plan(p, **opts)
    d = K.kpage_plan_device(p, **opts)
    for t in FWD_TABLES:
        a, b = K.kpage_plan_export(h, t), K.kpage_plan_export(d, t)
        assert a.dtype == b.dtype and np.array_equal(a, b), (label, t, a.shape, b.shape)
    sh, sd = K.kpage_plan_stats(h), K.kpage_plan_stats(d)
    for n in FWD_STATS:
        assert sh[n] == sd[n], (label, n, sh[n], sd[n])
    if bwd:  # exporting a backward table builds the backward tables of both plans
        for t in BWD_TABLES:
            a, b = K.kpage_plan_export(h, t), K.kpage_plan_export(d, t)
            assert a.dtype == b.dtype and np.array_equal(a, b), (label, t, a.shape, b.shape)
        sh, sd = K.kpage_plan_stats(h), K.kpage_plan_stats(d)
        for n in BWD_STATS:
            assert sh[n] == sd[n], (label, n, sh[n], sd[n])
    _say(f"  {label}: tables equal (walk {K.kpage_plan_export(d, 'fwd_walk').size} pages, useful {sd['useful']}"
         + (f", {K.kpage_plan_export(d, 'adj').size} backward steps)" if bwd else ")"))
    return h, d


CASES = {
    "tiny 5x6x10 d=64": lambda: make_workload(1),
    "16x32x32 two heads": lambda: make_workload(2, heads=[0, 1]),
    "21x30x52 two heads": lambda: make_workload(3, heads=[0, 1]),
    "21x45x80 top-87 two heads (per-head graphs)": lambda: make_workload(4, heads=[0, 1]),
    "SVG2-like partitions two heads": lambda: make_workload(5, heads=[0, 1]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_device_plan_tables_equal_host_plan(name):
    _say(f"[plan] {name}")
    same_plans(CASES[name](), name)


@pytest.mark.parametrize("name", list(EDGE_CASES))
@pytest.mark.parametrize("align", [(0, 0), (32, 16)])
def test_device_plan_edge_cases(name, align):
    cq, ck, rows = EDGE_CASES[name]
    p = make_problem(cq, ck, rows, heads=3, head_dim=128, sort_rows=False)
    same_plans(p, f"{name} align {align}", align_q64=align[0], align_q128=align[1])


def test_device_plan_offsets_with_gaps_and_null_offsets():
    ck = [50, 128, 3, 97, 16, 0, 33]
    off = [448, 0, 160, 192, 128, 0, 320]
    rows = [[0, 1, 2], [3, 4, 6], [6, 0], [1, 3, 5], [2]]
    p = make_problem([128, 64, 90, 20, 128], ck, rows, heads=2, head_dim=128, kv_offset=off, seq_kv=512,
                     sort_rows=False)
    same_plans(p, "offsets with gaps")
    q = make_problem([128, 64, 90], [128, 40, 7], [[0, 1], [2], [2, 1, 0]], heads=2, head_dim=128)
    q.kv_offset = None  # NULL offsets: block k at row 128 k
    same_plans(q, "null offsets")


def test_device_plan_attention_is_bitwise_equal():
    w = make_workload(3, heads=[0, 1], with_do=True)
    h, d = same_plans(w, "21x30x52 two heads", bwd=False)  # backward tables built by the first backward call
    dev = torch.device("cuda", 0)
    q, k, v, do = (x.to(dev) for x in (w.q, w.k, w.v, w.do))
    outs = []
    for plan in (h, d):
        o, lse = K.attn_fwd(plan, q, k, v, w.scale)
        dq, dk, dv = K.attn_bwd(plan, q, k, v, o, lse, do, w.scale)
        torch.cuda.synchronize()
        outs.append([x.float().cpu().numpy() for x in (o, lse, dq, dk, dv)])
    for n, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), *outs):
        assert np.array_equal(a, b, equal_nan=True), n
    for t in BWD_TABLES:
        assert np.array_equal(K.kpage_plan_export(h, t), K.kpage_plan_export(d, t)), t
    sh, sd = K.kpage_plan_stats(h), K.kpage_plan_stats(d)
    assert sh["bwd_physical"] == sd["bwd_physical"] and sh["bwd_useful_check"] == sd["bwd_useful_check"]


@pytest.mark.parametrize("cfg,heads", [(3, [0, 1]), (4, [0, 1])])
def test_device_plan_groups_equal_host_groups(cfg, heads):
    """Group items built on the GPU: the same groups, union walks and member words as the
    host planner's, and none when both are planned ungrouped."""
    w = make_workload(cfg, heads=heads)
    h, d = K.kpage_plan(w), K.kpage_plan_device(w)
    assert K.kpage_plan_export(h, "group_members").size > 0
    for t in FWD_TABLES:
        a, b = K.kpage_plan_export(h, t), K.kpage_plan_export(d, t)
        assert a.dtype == b.dtype and np.array_equal(a, b), (cfg, t)
    h0, d0 = K.kpage_plan(w, grouped=False), K.kpage_plan_device(w, grouped=False)
    for x in (h0, d0):
        assert K.kpage_plan_export(x, "group_members").size == 0
        gp = K.kpage_plan_export(x, "group_ptr")
        assert gp.size == (len(heads) if w.per_head else 1) + 1 and not gp.any()
    _say(f"  workload {cfg}: {K.kpage_plan_export(d, 'group_members').size // 4} groups equal")


def test_device_plan_full_size_attention_is_bitwise_equal():
    """All 40 heads of the 21x30x52 workload (10,320 backward items, so every XCD's
    longest-first tail holds 64 owners): outputs of the GPU-built plan equal the host
    plan's bit for bit."""
    w = make_workload(3, with_do=True)
    _say(f"[device plan] full-size 21x30x52, {w.heads} heads")
    h, d = K.kpage_plan(w), K.kpage_plan_device(w)
    dev = torch.device("cuda", 0)
    q, k, v, do = (x.to(dev) for x in (w.q, w.k, w.v, w.do))
    outs = []
    for plan in (h, d):
        o, lse = K.attn_fwd(plan, q, k, v, w.scale)
        dq, dk, dv = K.attn_bwd(plan, q, k, v, o, lse, do, w.scale)
        torch.cuda.synchronize()
        outs.append([x.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
                     for x in (o, lse, dq, dk, dv)])
        del o, lse, dq, dk, dv
    for n, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), *outs):
        assert np.array_equal(a, b), n


def _bad(p, what):
    with pytest.raises(K.KpageError) as e:
        K.kpage_plan_device(p)
    assert e.value.status == K.KPAGE_ERR_INVALID, (what, e.value)
    # the host planner agrees
    with pytest.raises(K.KpageError) as e2:
        K.kpage_plan(p)
    assert e2.value.status == K.KPAGE_ERR_INVALID, what


GROUP_CASES = {
    "tiny 5x6x10 d=64, q_group 1": (lambda: make_workload(1), 1),
    "tiny 5x6x10 d=64, q_group 3": (lambda: make_workload(1), 3),
    "21x30x52 two heads, q_group 16": (lambda: make_workload(3, heads=[0, 1]), 16),
    "21x45x80 top-87 two heads (per-head graphs), q_group 64": (lambda: make_workload(4, heads=[0, 1]), 64),
    "SVG2-like partitions two heads, q_group 8": (lambda: make_workload(5, heads=[0, 1]), 8),
    # one owner of two Q blocks straddling the ranges (kept whole), one of three (split)
    "short lists kept whole, q_group 2": (
        lambda: make_problem([128] * 4, [128, 128], [[1], [0, 1], [0], [1]], heads=2, head_dim=128), 2),
}


@pytest.mark.parametrize("name", list(GROUP_CASES))
def test_device_plan_q_group_tables_equal_host_plan(name):
    make, q_group = GROUP_CASES[name]
    _say(f"[plan] {name}")
    h, d = same_plans(make(), name, q_group=q_group)
    assert K.kpage_bwd_workspace_size(h) == K.kpage_bwd_workspace_size(d)


@pytest.mark.parametrize("name,q_group", [("21x30x52 two heads", 16),
                                          ("21x45x80 top-87 two heads (per-head graphs)", 64)])
def test_device_plan_q_groups_attention_is_bitwise_equal(name, q_group):
    """Q groups planned on the GPU: the same work items, fp32 partial slots and reduce
    entries as the host plan, so the gradients are bitwise equal."""
    w = make_workload(3 if "21x30x52" in name else 4, heads=[0, 1], with_do=True)
    _say(f"[device plan] {name}, q_group {q_group}")
    h, d = K.kpage_plan(w, q_group=q_group), K.kpage_plan_device(w, q_group=q_group)
    assert K.kpage_bwd_workspace_size(h) == K.kpage_bwd_workspace_size(d)
    dev = torch.device("cuda", 0)
    q, k, v, do = (x.to(dev) for x in (w.q, w.k, w.v, w.do))
    outs = []
    for plan in (h, d):
        o, lse = K.attn_fwd(plan, q, k, v, w.scale)
        dq, dk, dv = K.attn_bwd(plan, q, k, v, o, lse, do, w.scale)
        torch.cuda.synchronize()
        outs.append([x.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
                     for x in (o, lse, dq, dk, dv)])
        del o, lse, dq, dk, dv
    for n, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), *outs):
        assert np.array_equal(a, b), n
    for t in BWD_TABLES:
        assert np.array_equal(K.kpage_plan_export(h, t), K.kpage_plan_export(d, t)), t


def test_device_plan_rejects_malformed_descriptors():
    base = make_problem([128, 64], [128, 40, 7], [[0, 1], [2]], heads=1, head_dim=128)
    p = copy.deepcopy(base)
    p.q2k_idx = np.array([0, 0, 2], dtype=np.int32)
    _bad(p, "duplicate block in a row")
    p = copy.deepcopy(base)
    p.q2k_idx = np.array([0, 5, 2], dtype=np.int32)
    _bad(p, "block id out of range")
    p = copy.deepcopy(base)
    p.q_valid = np.array([[129, 64]], dtype=np.int32)
    _bad(p, "q_valid out of range")
    p = copy.deepcopy(base)
    p.kv_valid = np.array([[128, -1, 7]], dtype=np.int32)
    _bad(p, "kv_valid out of range")
    p = copy.deepcopy(base)
    p.kv_offset = np.array([[0, 64, 256]], dtype=np.int64)
    _bad(p, "overlapping footprints")
    p = copy.deepcopy(base)
    p.kv_offset = np.array([[0, 136, 256]], dtype=np.int64)
    _bad(p, "offset not a multiple of 16")
    p = copy.deepcopy(base)
    p.q2k_ptr = np.array([[0, 2, 9]], dtype=np.int64)
    _bad(p, "row end past the index array")


def _plan_and_backward_tables(plan_fn, w):
    t0 = time.perf_counter()
    pl = plan_fn(w)
    t1 = time.perf_counter()
    K.kpage_plan_export(pl, "owner_ptr")  # builds the backward tables (device: kernels, then a copy down)
    t2 = time.perf_counter()
    return pl, t1 - t0, t2 - t1


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_device_plan_full_size(cfg):
    """Bit-exact on the full-size workloads (all heads); prints host and device planning time
    (not a speed assertion; the device's backward time includes copying its tables down)."""
    w = make_workload(cfg)
    K.kpage_plan_device(w)  # warm up kernels and allocator
    torch.cuda.synchronize()
    h, hf, hb = _plan_and_backward_tables(K.kpage_plan, w)
    d, df, db = _plan_and_backward_tables(K.kpage_plan_device, w)
    for t in FWD_TABLES + BWD_TABLES:
        assert np.array_equal(K.kpage_plan_export(h, t), K.kpage_plan_export(d, t)), (cfg, t)
    sh, sd = K.kpage_plan_stats(h), K.kpage_plan_stats(d)
    assert sh == sd, (cfg, sh, sd)
    _say(f"  workload {cfg}: forward plan host {hf * 1e3:.2f} ms, device {df * 1e3:.2f} ms; "
         f"backward tables host {hb * 1e3:.2f} ms, device {db * 1e3:.2f} ms")


def test_device_plan_random_layouts():
    """Random small layouts (sizes 0..128 with tails, shuffled offsets with gaps, empty rows,
    shared and per-head graphs, both alignments): every table equal to the host plan's."""
    from tests.problems import Problem
    rng = np.random.default_rng(23)
    sizes = [0, 1, 2, 15, 16, 17, 31, 48, 63, 64, 65, 100, 112, 113, 127, 128]
    for trial in range(30):
        G = int(rng.integers(1, 4))
        n_q, n_kv = int(rng.integers(1, 12)), int(rng.integers(1, 12))
        qv = rng.choice(sizes, size=(G, n_q)).astype(np.int32)
        kv = rng.choice(sizes, size=(G, n_kv)).astype(np.int32)
        off = np.zeros((G, n_kv), dtype=np.int64)
        seq_kv = 16
        for g in range(G):
            acc = 0
            for k in rng.permutation(n_kv):
                off[g, k] = acc
                acc += 16 * ((int(kv[g, k]) + 15) // 16) + 16 * int(rng.integers(0, 2))
            seq_kv = max(seq_kv, acc)
        ptr = np.zeros((G, n_q + 1), dtype=np.int64)
        idx = []
        for g in range(G):
            for q in range(n_q):
                row = rng.permutation(n_kv)[:int(rng.integers(0, n_kv + 1))].tolist()
                idx.extend(row)
                ptr[g, q + 1] = len(idx)
            if g + 1 < G:
                ptr[g + 1, 0] = len(idx)
        per_head = G > 1
        p = Problem(batch=1, heads=G if per_head else int(rng.integers(1, 3)), head_dim=64, n_q=n_q, n_kv=n_kv,
                    seq_q=128 * n_q, seq_kv=seq_kv, per_head=per_head, q_valid=qv, kv_valid=kv, kv_offset=off,
                    q2k_ptr=ptr, q2k_idx=np.asarray(idx, dtype=np.int32))
        align = [(0, 0), (32, 16)][trial % 2]
        same_plans(p, f"random layout {trial}", align_q64=align[0], align_q128=align[1])


@pytest.mark.parametrize("rows_past", [0, 16])
def test_device_plan_grouping_limit_equals_host(rows_past):
    """At and one page past the page-bitset limit of the grouping (2^21 K/V rows), the GPU
    planner groups exactly as the host planner does (a group, then none)."""
    seq_kv = 2048 * 64 * 16 + rows_past
    p = make_problem([20, 32, 8], [128, 128, 128], [[0, 1], [0, 1], [0, 2]], heads=1, head_dim=64,
                     kv_offset=[0, 128, seq_kv - 128], seq_kv=seq_kv)
    h, d = same_plans(p, f"seq_kv {seq_kv}", bwd=False)
    assert K.kpage_plan_export(d, "group_members").size == (4 if rows_past == 0 else 0)


def test_device_plan_total_bitset_limit_equals_host():
    """Past the limit on all slots' page bitsets together the GPU planner, like the host
    planner, builds no group items."""
    from tests.test_groups import many_small_blocks_problem
    h, d = same_plans(many_small_blocks_problem(8193), "2 x 8193 small blocks over 2^21 K/V rows", bwd=False)
    assert K.kpage_plan_export(d, "group_members").size == 0
