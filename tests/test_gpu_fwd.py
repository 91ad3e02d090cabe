"""Forward parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances, for bf16 inputs with fp32 accumulation:
  * LSE: relative error <= 1e-3, |L - L*| <= 1e-3 |L*| + 1e-5.  The 1e-5 absolute floor
    only matters where |L*| < 1e-2; the fp32 evaluation of m + log(l) has an absolute
    rounding error of order 2^-23 (|m| + |log l|), far below it.
  * O on the five benchmark configurations: max-abs <= 1e-2, flat.
  * O on the synthetic edge cases (rows that attend to one or a few keys of N(0,1)
    values, so |O| reaches 2-4): per element max(1e-2, E) with E the rounding bound of
    the computation (output rounded to bf16, half a bf16 ulp of the result; each
    probability rounded to bf16 before the P.V product, relative 2^-8, so at most
    2^-8 sum_j P_ij |V_jc|; 2^-12 of the same sum for fp32 accumulation).  For |O| >= 4
    no bf16 output can be within 1e-2 of every real value (half an ulp there is
    2^-6 = 0.0156), and between 2 and 4 half an ulp already takes 0.0078 of it.
    E is computed with the oracle: sum_j P_ij |V_jc| is the oracle's attention output
    for the values |V|.
  * Rows the oracle marks empty (LSE = -inf) must be exactly O = 0 and LSE = -inf.
The worst error of every check, against its bound, is printed after the run.
"""
import math
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_11_amd as K
from oracle import oracle_fwd
from tests import parity_log
from tests.tolerances import LSE_ATOL, LSE_RTOL, O_ATOL, rounding_bound
from tests.problems import make_problem, random_tensors
from workloads import make_workload

pytestmark = pytest.mark.gpu

def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_fwd(problem, q, k, v, plan=None):
    dev = torch.device("cuda", 0)
    plan = plan or K.kpage_plan(problem)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = K.attn_fwd(plan, qd, kd, vd, problem.scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def check(O, L, Oref, Lref, label, Aabs=None):
    """O against the flat 1e-2 when Aabs is None, else against max(1e-2, rounding bound)."""
    done = ~np.isnan(Lref)
    empty = done & np.isneginf(Lref)
    live = done & ~empty
    assert np.all(np.isneginf(L[empty])), f"{label}: rows without keys must have LSE = -inf"
    assert np.all(O[empty] == 0), f"{label}: rows without keys must have O = 0"
    assert np.all(np.isfinite(L[live])), f"{label}: non-finite LSE on a live row"
    if not live.any():
        return
    err = np.abs(O[live] - Oref[live])
    err_o = float(err.max())
    if Aabs is None:
        bound = np.full_like(err, O_ATOL)
        note = "flat 1e-2"
    else:
        bound = np.maximum(O_ATOL, rounding_bound(Oref[live], Aabs[live]))
        note = f"max(1e-2, rounding bound); {int((err > O_ATOL).sum())} elements above 1e-2"
    i = int(np.argmax(err / bound))
    ratio = float(err.flat[i] / bound.flat[i])
    lerr = np.abs(L[live] - Lref[live])
    lbound = LSE_RTOL * np.abs(Lref[live]) + LSE_ATOL
    j = int(np.argmax(lerr / lbound))
    lratio = float(lerr[j] / lbound[j])
    err_l = float((lerr / np.maximum(np.abs(Lref[live]), LSE_ATOL)).max())
    _say(f"  {label}: rows={int(live.sum())} empty={int(empty.sum())} O max-abs={err_o:.3e} "
         f"(max |O| {np.abs(Oref[live]).max():.2f}, worst error/bound {ratio:.3f}) LSE rel={err_l:.3e}")
    parity_log.record(label, "O", float(err.flat[i]), float(bound.flat[i]), f"{note}; max-abs {err_o:.3e}")
    parity_log.record(label, "LSE", float(lerr[j]), float(lbound[j]), f"1e-3 |L*| + 1e-5; max rel {err_l:.3e}")
    assert ratio <= 1.0, (label, err_o, ratio)
    assert lratio <= 1.0, (label, err_l)


def abs_values_attention(problem, q, k, v, items=None):
    """sum_j P_ij |V_jc| from the oracle: its attention output for the values |V|."""
    return oracle_fwd(problem, q, k, v.abs(), items=items)[0]


def padded_rows(w, side):
    """Row indices that hold no token (shared layouts: every block spans 128 rows)."""
    c = w.q_valid[0] if side == "q" else w.kv_valid[0]
    rows = [np.arange(128 * b + int(n), 128 * b + 128) for b, n in enumerate(c)]
    return torch.from_numpy(np.concatenate(rows))


def _all_rows(w, label):
    _say(f"[fwd] {label}: B={w.batch} H={w.heads} d={w.head_dim} n_q={w.n_q} n_kv={w.n_kv}")
    O, L = gpu_fwd(w, w.q, w.k, w.v)
    Oref, Lref = oracle_fwd(w, w.q, w.k, w.v)
    check(O, L, Oref, Lref, label)


def _sampled(w, label, per_head=24, seed=0):
    rng = np.random.default_rng(seed)
    items = []
    for h in range(w.heads):
        qs = rng.choice(w.n_q, size=min(per_head, w.n_q), replace=False)
        items += [(0, h, int(q)) for q in qs]
    _say(f"[fwd] {label}: B={w.batch} H={w.heads} n_q={w.n_q}, {len(items)} sampled blocks")
    O, L = gpu_fwd(w, w.q, w.k, w.v)
    Oref, Lref = oracle_fwd(w, w.q, w.k, w.v, items=items)
    check(O, L, Oref, Lref, label)


def test_fwd_tiny_3d_layout_d64_all_rows():
    _all_rows(make_workload(1), "tiny 5x6x10 d=64")


def test_fwd_padding_free_two_heads_all_rows():
    _all_rows(make_workload(2, heads=[0, 1]), "16x32x32 two heads")


def test_fwd_3d_padded_two_heads_all_rows():
    _all_rows(make_workload(3, heads=[0, 1]), "21x30x52 two heads")


def test_fwd_vsa_topk_sampled():
    _sampled(make_workload(4, heads=[0, 1]), "21x45x80 top-87, two heads", per_head=40)


def test_fwd_independent_partitions_sampled():
    _sampled(make_workload(5, heads=[0, 1]), "SVG2-like partitions, two heads", per_head=60)


def test_fwd_3d_padded_full_heads_sampled():
    """All 40 heads in one launch, as the benchmark runs it; sampled query blocks checked."""
    _sampled(make_workload(3), "21x30x52 all 40 heads", per_head=6)


def test_fwd_vsa_topk_full_heads_sampled():
    """The 21x45x80 top-87 workload at full size (40 heads, per-head graphs), as the benchmark launches it."""
    _sampled(make_workload(4), "21x45x80 top-87 all 40 heads", per_head=4)


def test_fwd_independent_partitions_full_heads_sampled():
    """The SVG2-like workload at full size (40 heads, per-head partitions), as the benchmark launches it."""
    _sampled(make_workload(5), "SVG2-like partitions all 40 heads", per_head=4)


def test_fwd_padding_free_full_heads_sampled():
    _sampled(make_workload(2), "16x32x32 all 24 heads", per_head=8)


EDGE_CASES = {
    # every tail length, both routes, walks of several stages with dummies
    "tails-1-to-15": ([128, 64, 65, 1, 127], [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 128, 16, 17],
                      [list(range(18)), list(range(0, 18, 2)), list(range(1, 18, 3)), [15, 0], list(range(17, -1, -1))]),
    # empty selections, empty blocks on both sides, a block with one valid key
    "empty-and-single": ([128, 0, 40, 128, 64], [0, 1, 128, 0],
                         [[0], [1, 2], [], [1], [0, 3]]),
    # one query block that needs many stages
    "long-walk": ([100, 30], [128] * 20 + [77] * 5, [list(range(25)), list(range(24, -1, -1))]),
}


@pytest.mark.parametrize("name", list(EDGE_CASES))
@pytest.mark.parametrize("d", [64, 128])
def test_fwd_edge_cases(name, d):
    cq, ck, rows = EDGE_CASES[name]
    p = make_problem(cq, ck, rows, heads=3, head_dim=d, sort_rows=False)
    t = random_tensors(p, seed=len(name) + d)
    _say(f"[fwd] edge case {name} d={d}")
    O, L = gpu_fwd(p, t["q"], t["k"], t["v"])
    Oref, Lref = oracle_fwd(p, t["q"], t["k"], t["v"])
    check(O, L, Oref, Lref, f"{name} d={d}", Aabs=abs_values_attention(p, t["q"], t["k"], t["v"]))


def rising_scores_problem(d):
    """Scores that rise by far more than 2^64 (base 2) after the first tile of every walk.

    Every query has a large component along one direction u; the keys of the first
    selected block have none, the keys of later blocks a large one, so the row maximum
    found on the first tile is exceeded by about q.k * scale * log2(e) ~ 100 later on.
    This drives the forward kernel's exact rescaling pass; the oracle is unaffected.
    """
    p = make_problem([128, 100, 50, 20], [128, 128, 77, 128, 33], [[0, 1, 2], [0, 3, 4, 1], [0, 2], [0, 4]],
                     heads=2, head_dim=d, sort_rows=False)
    t = random_tensors(p, seed=11)
    g = torch.Generator().manual_seed(12)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    amp = 30.0 * (128.0 / d) ** 0.5
    q = t["q"].float() + amp * u
    k = t["k"].float()
    k[:, :, 128:] += amp * u          # every key block but block 0
    for x, c in ((q, p.q_valid[0]), (k, p.kv_valid[0])):
        for b, n in enumerate(c):
            x[:, :, 128 * b + int(n):128 * (b + 1)] = 0
    return p, q.to(torch.bfloat16), k.to(torch.bfloat16), t["v"], t["do"]


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_large_score_rise_uses_exact_pass(d):
    p, q, k, v, _ = rising_scores_problem(d)
    _say(f"[fwd] large score rise d={d}")
    O, L = gpu_fwd(p, q, k, v)
    Oref, Lref = oracle_fwd(p, q, k, v)
    check(O, L, Oref, Lref, f"large score rise d={d}", Aabs=abs_values_attention(p, q, k, v))


def test_fwd_independent_offsets_with_gaps():
    """K/V blocks at shuffled Page16 offsets with unused pages between footprints."""
    ck = [50, 128, 3, 97, 16, 0, 33]
    off = [448, 0, 160, 192, 128, 0, 320]
    rows = [[0, 1, 2], [3, 4, 6], [6, 0], [1, 3, 5], [2]]
    p = make_problem([128, 64, 90, 20, 128], ck, rows, heads=2, head_dim=128, kv_offset=off, seq_kv=512,
                     sort_rows=False)
    t = random_tensors(p, seed=5)
    _say("[fwd] shuffled offsets with gaps")
    O, L = gpu_fwd(p, t["q"], t["k"], t["v"])
    Oref, Lref = oracle_fwd(p, t["q"], t["k"], t["v"])
    check(O, L, Oref, Lref, "offsets with gaps", Aabs=abs_values_attention(p, t["q"], t["k"], t["v"]))


def test_fwd_padding_contents_do_not_matter():
    """Finite garbage in padded rows gives bit-identical outputs (masking is a select before the max)."""
    w = make_workload(3, heads=[0])
    _say("[fwd] padded-row garbage invariance")
    O1, L1 = gpu_fwd(w, w.q, w.k, w.v)
    g = torch.Generator().manual_seed(3)
    q, k, v = w.q.clone(), w.k.clone(), w.v.clone()
    for x, rows in ((q, padded_rows(w, "q")), (k, padded_rows(w, "kv")), (v, padded_rows(w, "kv"))):
        garbage = (100 * torch.randn(x.shape, generator=g)).to(torch.bfloat16)
        x[:, :, rows] = garbage[:, :, rows]
    O2, L2 = gpu_fwd(w, q, k, v)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_fwd_selection_order_does_not_matter():
    w = make_workload(3, heads=[0, 1])
    _say("[fwd] K_q permutation")
    O1, L1 = gpu_fwd(w, w.q, w.k, w.v)
    rng = np.random.default_rng(1)
    idx = w.q2k_idx.copy()
    for q in range(w.n_q):
        a, b = w.q2k_ptr[0, q], w.q2k_ptr[0, q + 1]
        idx[a:b] = rng.permutation(idx[a:b])
    w.q2k_idx = idx
    O2, L2 = gpu_fwd(w, w.q, w.k, w.v)
    assert np.abs(O1 - O2).max() <= O_ATOL
    fin = np.isfinite(L1)
    assert np.array_equal(fin, np.isfinite(L2))
    assert (np.abs(L1[fin] - L2[fin]) <= 2 * (LSE_RTOL * np.abs(L1[fin]) + LSE_ATOL)).all()


def test_fwd_is_deterministic_and_plan_is_reusable():
    w = make_workload(3, heads=[0, 1])
    plan = K.kpage_plan(w)
    _say("[fwd] determinism and plan reuse")
    O1, L1 = gpu_fwd(w, w.q, w.k, w.v, plan=plan)
    O2, L2 = gpu_fwd(w, w.q, w.k, w.v, plan=plan)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_fwd_rejects_bad_arguments_before_launch():
    w = make_workload(1)
    plan = K.kpage_plan(w)
    dev = torch.device("cuda", 0)
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    with pytest.raises(K.KpageError):
        K.attn_fwd(plan, q, k, v, -1.0)
    with pytest.raises(K.KpageError):
        K.attn_fwd(plan, q[:, :1].contiguous(), k, v, w.scale)


def test_fwd_two_streams_share_one_plan():
    """Two forward calls on one plan, on two streams with different outputs, overlap safely:
    the exact re-run's marks live in each call's own LSE rows.  Uses the score-rise
    problem, where every item goes through the exact re-run."""
    p, q, k, v, _ = rising_scores_problem(128)
    dev = torch.device("cuda", 0)
    plan = K.kpage_plan(p)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    ref_o, ref_l = K.attn_fwd(plan, qd, kd, vd, p.scale)
    torch.cuda.synchronize()
    _say("[fwd] two streams, one plan")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for s in (s1, s2):
        with torch.cuda.stream(s):
            o = torch.empty_like(qd)
            lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
            outs.append((o, lse))
    for _ in range(4):
        for s, (o, lse) in zip((s1, s2), outs):
            K.kpage_attn_fwd(plan, qd, kd, vd, o, lse, p.scale, stream=s)
    torch.cuda.synchronize()
    for o, lse in outs:
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)
