"""GPU block selection (kpage_select_topk, through the C ABI) against the selection oracle.

Both sides compute the block means and scores in fp64 in the same operation order, so the
selected lists must be identical, tie-breaking included.  Checked on the 21x45x80 layout
of the top-87 workload (sampled heads of the 40-head launch), on small layouts with empty
blocks, exact ties, shuffled offsets with gaps and top_k above the number of live blocks
(d = 64 and 128), and end to end: selection -> GPU planner -> attention gives the same
output as the host plan of the oracle's graph.
"""
import sys
import time

import numpy as np
import pytest
import torch

import block_sparse_attention_11_amd as K
from oracle.selection import select_topk as oracle_select
from tests.problems import make_problem
from workloads import make_workload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _gpu_rows(ptr, idx, B, H, n_q):
    ptr, idx = ptr.cpu().numpy(), idx.cpu().numpy()
    return {(b, h): [idx[ptr[b * H + h, q]:ptr[b * H + h, q + 1]].tolist() for q in range(n_q)]
            for b in range(B) for h in range(H)}


def _check(q, k, q_valid, kv_valid, kv_offset, top_k, label, heads=None):
    qd, kd = q.to(DEV).contiguous(), k.to(DEV).contiguous()
    qv = torch.as_tensor(np.asarray(q_valid, dtype=np.int32), device=DEV)
    kvv = torch.as_tensor(np.asarray(kv_valid, dtype=np.int32), device=DEV)
    ko = None if kv_offset is None else torch.as_tensor(np.asarray(kv_offset, dtype=np.int64), device=DEV)
    ptr, idx = K.select_topk(qd, kd, qv, kvv, ko, top_k)
    torch.cuda.synchronize()
    B, H = q.shape[:2]
    got = _gpu_rows(ptr, idx, B, H, len(q_valid))
    ref = oracle_select(q.float().numpy(), k.float().numpy(), q_valid, kv_valid, kv_offset, top_k, heads=heads)
    for key, rows in ref.items():
        assert got[key] == rows, (label, key)
    # CSR bookkeeping: contiguous rows, absolute offsets
    p = ptr.cpu().numpy()
    assert p[0, 0] == 0 and np.all(np.diff(p.reshape(-1)[:-1]) >= 0)
    _say(f"  {label}: {len(ref)} heads equal, {sum(len(r) for r in next(iter(ref.values())))} edges per head")


def test_select_top87_21x45x80_two_heads():
    w = make_workload(4, heads=[0, 1])
    _check(w.q, w.k, w.q_valid[0], w.kv_valid[0], w.kv_offset[0], 87, "21x45x80 top-87 two heads")


def test_select_top87_21x45x80_all_heads_two_checked():
    w = make_workload(4)
    _check(w.q, w.k, w.q_valid[0], w.kv_valid[0], w.kv_offset[0], 87, "21x45x80 top-87 40 heads", heads=[0, 39])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("top_k", [1, 3, 50])
def test_select_small_layouts(d, top_k):
    cq = [128, 0, 17, 1, 64, 128, 100]
    ck = [50, 128, 0, 3, 128, 16, 33, 97]
    off = [448, 0, 1024, 160, 576, 128, 320, 192]  # shuffled, with gaps
    p = make_problem(cq, ck, [[0]] * len(cq), heads=3, head_dim=d, kv_offset=off, seq_kv=1152, sort_rows=False)
    g = torch.Generator().manual_seed(d + top_k)
    q = torch.randn(1, 3, p.seq_q, d, generator=g).to(torch.bfloat16)
    k = torch.randn(1, 3, p.seq_kv, d, generator=g).to(torch.bfloat16)
    # an exact tie: key block 5 (16 rows at 128) repeats the first 16 rows of block 4 (at 576) in every head
    k[:, :, 128:144] = k[:, :, 576:592]
    ck_tie = list(ck)
    ck_tie[4] = 16
    _check(q, k, cq, ck_tie, off, top_k, f"small layout d={d} top_k={top_k}")
    _check(q, k, cq, ck, off, top_k, f"small layout d={d} top_k={top_k} (no tie)")
    _check(q[:, :, :, :], k[:, :, :1024], cq, [128] * 8, None, top_k, f"default offsets d={d} top_k={top_k}")


def test_select_then_plan_then_attention():
    """Selection and planning on the GPU give the plan of the oracle's graph: bitwise-equal O."""
    w = make_workload(4, heads=[0, 1])
    q, k, v = (x.to(DEV) for x in (w.q, w.k, w.v))
    qv = torch.as_tensor(w.q_valid[0], device=DEV)
    kvv = torch.as_tensor(w.kv_valid[0], device=DEV)
    ko = torch.as_tensor(w.kv_offset[0], device=DEV)
    plan_dev = K.plan_topk(q, k, qv, kvv, ko, 87)
    ref = oracle_select(w.q.float().numpy(), w.k.float().numpy(), w.q_valid[0], w.kv_valid[0], w.kv_offset[0], 87)
    rows = [ref[(0, h)] for h in range(2)]
    ptr = np.zeros((2, w.n_q + 1), dtype=np.int64)
    idx = []
    for h in range(2):
        ptr[h, 0] = len(idx)
        for qb in range(w.n_q):
            idx.extend(rows[h][qb])
            ptr[h, qb + 1] = len(idx)
    w.q2k_ptr, w.q2k_idx = ptr, np.asarray(idx, dtype=np.int32)
    plan_host = K.kpage_plan(w)
    o1, l1 = K.attn_fwd(plan_dev, q, k, v, w.scale)
    o2, l2 = K.attn_fwd(plan_host, q, k, v, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for t in ("fwd_walk", "q128_queue", "q64_queue"):
        assert np.array_equal(K.kpage_plan_export(plan_dev, t), K.kpage_plan_export(plan_host, t)), t


def test_select_time_full_size():
    """Not a speed assertion: selection time on the 40-head 21x45x80 layout."""
    w = make_workload(4)
    q, k = w.q.to(DEV), w.k.to(DEV)
    qv = torch.as_tensor(w.q_valid[0], device=DEV)
    kvv = torch.as_tensor(w.kv_valid[0], device=DEV)
    ko = torch.as_tensor(w.kv_offset[0], device=DEV)
    ws = torch.empty(K.kpage_select_workspace_size(q, k, qv, kvv, ko), dtype=torch.uint8, device=DEV)
    K.select_topk(q, k, qv, kvv, ko, 87, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        K.select_topk(q, k, qv, kvv, ko, 87, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    _say(f"  select top-87, 40 heads x 720 blocks: {e0.elapsed_time(e1) / 5:.3f} ms per call")
    t0 = time.perf_counter()
    K.plan_topk(q, k, qv, kvv, ko, 87)
    torch.cuda.synchronize()
    _say(f"  select + GPU plan: {(time.perf_counter() - t0) * 1e3:.2f} ms")


# ---- cluster top-p selection (independent partitions) ----

def _stack(dicts, key, dtype):
    return torch.as_tensor(np.stack([c[key] for c in dicts]), device=DEV).to(dtype).contiguous()


def _top_p_rows_gpu(clusters, B, H, top_p, scale):
    args = [_stack(clusters, k, t) for k, t in (("q_cent", torch.float32), ("k_cent", torch.float32),
                                                ("q_size", torch.int32), ("k_size", torch.int32),
                                                ("q_block_cluster", torch.int32), ("k_block_cluster", torch.int32))]
    ptr, idx = K.select_top_p(B, H, *args, top_p=top_p, scale=scale)
    torch.cuda.synchronize()
    n_q = clusters[0]["q_block_cluster"].shape[0]
    return _gpu_rows(ptr, idx, B, H, n_q), (ptr, idx)


def _check_top_p(clusters, B, H, top_p, scale, label):
    from oracle.selection import block_scores, select_top_p
    got, dev = _top_p_rows_gpu(clusters, B, H, top_p, scale)
    for g, c in enumerate(clusters):
        ref = select_top_p(c["q_cent"], c["k_cent"], c["q_size"], c["k_size"], c["q_block_cluster"],
                           c["k_block_cluster"], top_p, scale)
        rows = got[(g // H, g % H)]
        for q, (a, b) in enumerate(zip(rows, ref)):
            if a == b:
                continue
            # a different cut is only allowed where the cumulative probability sits within rounding of top_p
            cl = int(c["q_block_cluster"][q])
            s = block_scores(np.asarray(c["q_cent"], np.float64), np.asarray(c["k_cent"], np.float64))[cl] * scale
            live = np.nonzero(np.asarray(c["k_size"]) > 0)[0]
            x = np.sort(s[live])[::-1]
            e = np.exp(x - x[0])
            csum = np.cumsum(e / e.sum())
            assert np.min(np.abs(csum - top_p)) <= 1e-12, (label, g, q)
    _say(f"  {label}: {len(clusters)} slots equal")
    return dev


def test_select_top_p_svg2_like_two_heads():
    w = make_workload(5, heads=[0, 1])
    _check_top_p(w.clusters, 1, 2, 0.9, 1.0 / np.sqrt(w.head_dim), "SVG2-like clusters two heads")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("top_p", [0.3, 0.9, 1.0])
def test_select_top_p_small(d, top_p):
    rng = np.random.default_rng(d + int(10 * top_p))
    n_qc, n_kc, n_q, n_kv = 5, 9, 8, 14
    clusters = []
    for _ in range(3):
        k_cent = rng.standard_normal((n_kc, d)).astype(np.float32)
        k_cent[4] = k_cent[1]  # equal scores: the lower cluster first
        clusters.append(dict(
            q_cent=rng.standard_normal((n_qc, d)).astype(np.float32), k_cent=k_cent,
            q_size=np.array([3, 0, 7, 1, 2], dtype=np.int32), k_size=np.array([1, 4, 0, 2, 9, 3, 0, 5, 1], np.int32),
            q_block_cluster=np.array([0, 2, 2, -1, 3, 4, 1, 0], dtype=np.int32),
            k_block_cluster=rng.integers(-1, n_kc, size=n_kv).astype(np.int32)))
    _check_top_p(clusters, 1, 3, top_p, 0.25, f"small clusters d={d} top_p={top_p}")


def test_select_top_p_then_plan():
    """GPU cluster selection feeds the GPU planner: the plan equals the host plan of the
    workload's own graph (the same rule, pinned against the oracle)."""
    w = make_workload(5, heads=[0, 1])
    _, (ptr, idx) = _top_p_rows_gpu(w.clusters, 1, 2, 0.9, 1.0 / np.sqrt(w.head_dim))
    p = type("P", (), {})()
    for a in ("batch", "heads", "head_dim", "n_q", "n_kv", "seq_q", "seq_kv", "per_head", "q_valid", "kv_valid",
              "kv_offset"):
        setattr(p, a, getattr(w, a))
    p.q2k_ptr, p.q2k_idx = ptr, idx
    d = K.kpage_plan_device(p)
    h = K.kpage_plan(w)
    for t in ("fwd_walk", "fwd_walk_ptr", "q128_queue", "q64_queue", "owners", "qwalk", "adj"):
        assert np.array_equal(K.kpage_plan_export(d, t), K.kpage_plan_export(h, t)), t
