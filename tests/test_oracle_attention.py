"""Pins for the fp64 attention oracle (CPU only).

Each test checks the oracle against something other than itself: dense attention
from torch over the original T x H x W tokens, pair-by-pair brute force,
torch.autograd, central finite differences, and invariants that follow from the
definition of masked softmax attention (KPage paper, section 3.2.4 and 3.3.3).
"""
import math

import numpy as np
import pytest
import torch

from oracle import brute_force_fwd, oracle_bwd, oracle_fwd
from oracle.layout import token_rows
from tests.problems import make_problem, random_tensors
from workloads import tile_layout


def _all_pairs_problem(T, H, W, d=16, heads=2):
    grid, c, _ = tile_layout(T, H, W)
    n = len(c)
    rows = [list(range(n)) for _ in range(n)]
    return make_problem(c, c, rows, heads=heads, head_dim=d)


@pytest.mark.parametrize("dims", [(5, 6, 10), (3, 5, 9), (4, 4, 8), (6, 9, 17)])
def test_all_ones_mask_equals_dense_attention_over_tokens(dims):
    """Selecting every block reduces block-sparse attention to dense attention over the unpadded tokens."""
    T, H, W = dims
    p = _all_pairs_problem(T, H, W)
    rows = token_rows(T, H, W).reshape(-1)
    g = torch.Generator().manual_seed(sum(dims))
    ntok = T * H * W
    toks = {n: torch.randn(p.heads, ntok, p.head_dim, generator=g, dtype=torch.float64) for n in "qkv"}
    phys = {n: torch.zeros(1, p.heads, p.seq_q, p.head_dim, dtype=torch.float64) for n in "qkv"}
    for n in "qkv":
        phys[n][0][:, torch.from_numpy(rows)] = toks[n]
    O, L = oracle_fwd(p, phys["q"], phys["k"], phys["v"])
    dense = torch.nn.functional.scaled_dot_product_attention(toks["q"], toks["k"], toks["v"])
    lse = torch.logsumexp(p.scale * toks["q"] @ toks["k"].transpose(-1, -2), dim=-1)
    np.testing.assert_allclose(O[0][:, rows], dense.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L[0][:, rows], lse.numpy(), rtol=1e-13, atol=0)
    # every row that holds no token is an invalid row: O = 0 and LSE = -inf
    pad = np.setdiff1d(np.arange(p.seq_q), rows)
    assert np.all(O[0][:, pad] == 0) and np.all(np.isneginf(L[0][:, pad]))


def test_brute_force_matches_vectorised_oracle():
    p = make_problem([128, 33, 64, 5, 0, 17], [128, 32, 70, 16, 3, 9],
                     [[0, 2, 5], [1], [0, 1, 2, 3, 4, 5], [3, 4], [0], []], heads=2, head_dim=8)
    t = random_tensors(p, seed=3)
    O, L = oracle_fwd(p, t["q"], t["k"], t["v"])
    Ob, Lb = brute_force_fwd(p, t["q"], t["k"], t["v"])
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-13)
    assert np.array_equal(np.isneginf(L), np.isneginf(Lb))
    fin = np.isfinite(L)
    np.testing.assert_allclose(L[fin], Lb[fin], rtol=1e-14, atol=0)


def _mixed_problem(heads=2, d=16):
    return make_problem([128, 40, 64, 100, 1, 128], [128, 17, 128, 48, 64, 100],
                        [[0, 3, 5], [1, 2], [2, 4, 0, 1], [3], [5, 1], [0, 1, 2, 3, 4, 5]],
                        heads=heads, head_dim=d, sort_rows=False)


def test_softmax_rows_sum_to_one():
    p = _mixed_problem()
    t = random_tensors(p, seed=5)
    v = t["v"].clone()
    v[:] = 1.0
    O, _ = oracle_fwd(p, t["q"], t["k"], v)
    for qb in range(p.n_q):
        c = int(p.q_valid[0, qb])
        np.testing.assert_allclose(O[:, :, 128 * qb:128 * qb + c], 1.0, rtol=0, atol=1e-14)


def test_padded_rows_do_not_contribute():
    """Finite garbage in padded Q/K/V rows leaves every valid output unchanged, exactly."""
    p = _mixed_problem()
    clean = random_tensors(p, seed=7)
    dirty = {n: x.clone() for n, x in clean.items()}
    garbage = random_tensors(p, seed=8, zero_padding=False, garbage=50.0)
    for n in "qkv":
        pad = clean[n] == 0
        dirty[n][pad] = garbage[n][pad]
    O1, L1 = oracle_fwd(p, clean["q"], clean["k"], clean["v"])
    O2, L2 = oracle_fwd(p, dirty["q"], dirty["k"], dirty["v"])
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_block_order_in_selection_does_not_matter():
    p = _mixed_problem()
    t = random_tensors(p, seed=9)
    O1, L1 = oracle_fwd(p, t["q"], t["k"], t["v"])
    rng = np.random.default_rng(0)
    idx = p.q2k_idx.copy()
    for qb in range(p.n_q):
        a, b = p.q2k_ptr[0, qb], p.q2k_ptr[0, qb + 1]
        idx[a:b] = rng.permutation(idx[a:b])
    p.q2k_idx = idx
    O2, L2 = oracle_fwd(p, t["q"], t["k"], t["v"])
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L1, L2, rtol=0, atol=1e-12)


def test_single_key_and_empty_cases():
    """One valid key: O = v and LSE = the single score; empty selections and empty blocks: O = 0, LSE = -inf."""
    p = make_problem([128, 50, 0], [1, 128, 0], [[0], [2], [0, 1]], heads=1, head_dim=16)
    t = random_tensors(p, seed=11)
    O, L = oracle_fwd(p, t["q"], t["k"], t["v"])
    q = t["q"][0, 0].double().numpy()
    k = t["k"][0, 0].double().numpy()
    v = t["v"][0, 0].double().numpy()
    np.testing.assert_allclose(O[0, 0, :128], np.broadcast_to(v[0], (128, 16)), rtol=0, atol=1e-15)
    np.testing.assert_allclose(L[0, 0, :128], p.scale * q[:128] @ k[0], rtol=1e-15, atol=1e-15)
    # block 1 selects only an empty block -> no valid key
    assert np.all(O[0, 0, 128:256] == 0) and np.all(np.isneginf(L[0, 0, 128:256]))
    # block 2 has no valid rows
    assert np.all(O[0, 0, 256:] == 0) and np.all(np.isneginf(L[0, 0, 256:]))


def _dense_mask(p, slot=0):
    M = np.zeros((p.seq_q, p.seq_kv), dtype=bool)
    for qb in range(p.n_q):
        cq = int(p.q_valid[slot, qb])
        for kb in p.row(slot, qb):
            o, ck = int(p.kv_offset[slot, kb]), int(p.kv_valid[slot, kb])
            M[128 * qb:128 * qb + cq, o:o + ck] = True
    return M


def test_backward_matches_autograd_on_dense_masked_attention():
    p = _mixed_problem(heads=2, d=16)
    t = random_tensors(p, seed=13)
    dQ, dK, dV, O, L = oracle_bwd(p, t["q"], t["k"], t["v"], t["do"])
    M = torch.from_numpy(_dense_mask(p))
    q = t["q"].double().requires_grad_()
    k = t["k"].double().requires_grad_()
    v = t["v"].double().requires_grad_()
    s = p.scale * q @ k.transpose(-1, -2)
    s = s.masked_fill(~M, -math.inf)
    has = M.any(dim=1)
    pr = torch.softmax(s.masked_fill(~has[:, None], 0.0), dim=-1) * has[:, None]
    o = pr @ v
    (o * t["do"].double()).sum().backward()
    np.testing.assert_allclose(O, o.detach().numpy(), rtol=0, atol=1e-13)
    for a, b in ((dQ, q.grad), (dK, k.grad), (dV, v.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=0, atol=1e-12)


def test_backward_matches_finite_differences():
    p = make_problem([7, 20], [5, 16, 9], [[0, 2], [1, 2]], heads=1, head_dim=4)
    t = random_tensors(p, seed=17)
    dQ, dK, dV, _, _ = oracle_bwd(p, t["q"], t["k"], t["v"], t["do"])
    base = {n: t[n].double().numpy().copy() for n in ("q", "k", "v")}
    do = t["do"].double().numpy()
    h = 1e-6

    def loss(arrs):
        O, _ = oracle_fwd(p, arrs["q"], arrs["k"], arrs["v"])
        return float((O * do).sum())

    rng = np.random.default_rng(1)
    for name, grad in (("q", dQ), ("k", dK), ("v", dV)):
        for _ in range(12):
            if name == "q":
                qb = int(rng.integers(0, p.n_q))
                row = 128 * qb + int(rng.integers(0, p.q_valid[0, qb]))
            else:
                kb = int(rng.integers(0, p.n_kv))
                row = int(p.kv_offset[0, kb]) + int(rng.integers(0, p.kv_valid[0, kb]))
            col = int(rng.integers(0, p.head_dim))
            up = {n: a.copy() for n, a in base.items()}
            dn = {n: a.copy() for n, a in base.items()}
            up[name][0, 0, row, col] += h
            dn[name][0, 0, row, col] -= h
            fd = (loss(up) - loss(dn)) / (2 * h)
            assert abs(fd - grad[0, 0, row, col]) < 1e-7, (name, row, col, fd, grad[0, 0, row, col])


def test_backward_identities():
    """sum_j dV_j = sum of dO over rows with keys; equal valid keys give dQ = 0 (score gradients sum to 0)."""
    p = _mixed_problem(heads=1)
    t = random_tensors(p, seed=19)
    dQ, dK, dV, _, _ = oracle_bwd(p, t["q"], t["k"], t["v"], t["do"])
    do = t["do"].double().numpy()
    # with every block selecting at least one valid key, each valid query row sends sum 1 of probability
    np.testing.assert_allclose(dV.sum(axis=2), do.sum(axis=2), rtol=0, atol=1e-10)
    k_same = t["k"].clone()
    k_same[:] = 0
    k_same[..., :] = torch.randn(p.head_dim, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    dQ2, _, _, _, _ = oracle_bwd(p, t["q"], k_same, t["v"], t["do"])
    np.testing.assert_allclose(dQ2, 0.0, rtol=0, atol=1e-12)
    # invalid rows receive no gradient
    for qb in range(p.n_q):
        c = int(p.q_valid[0, qb])
        assert np.all(dQ[..., 128 * qb + c:128 * qb + 128, :] == 0)
