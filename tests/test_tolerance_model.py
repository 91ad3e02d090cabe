"""The forward rounding bound used by the GPU parity tests holds for an emulation of the
rounding steps it models, and its probability term is needed.

The emulation follows the rounding reading of the forward: scores in fp32, probabilities
exp2(score * scale * log2(e) - row max) in fp32, each rounded to bf16 before the P.V
product, row sums from the fp32 probabilities, O = (sum_j bf16(P_j) V_j) / l in fp32,
rounded to bf16.  It runs on the synthetic edge cases and the per-(batch, head) graphs
that the GPU tests hold to max(1e-2, rounding bound).
"""
import math

import numpy as np
import torch

from oracle import oracle_fwd
from tests.problems import make_problem, random_tensors
from tests.tolerances import P_ROUND, rounding_bound

# the forward edge cases of the GPU tests (same layouts, graphs and seeds)
EDGE_CASES = {
    "tails-1-to-15": ([128, 64, 65, 1, 127], [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 128, 16, 17],
                      [list(range(18)), list(range(0, 18, 2)), list(range(1, 18, 3)), [15, 0], list(range(17, -1, -1))]),
    "empty-and-single": ([128, 0, 40, 128, 64], [0, 1, 128, 0], [[0], [1, 2], [], [1], [0, 3]]),
    "long-walk": ([100, 30], [128] * 20 + [77] * 5, [list(range(25)), list(range(24, -1, -1))]),
}


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def emulate_fwd(p, q, k, v):
    """O as the forward's rounding steps produce it (fp32 scores and sums, bf16 P and O)."""
    Q, K, V = (t.float().numpy().astype(np.float64) for t in (q, k, v))
    c2 = np.float32(p.scale * math.log2(math.e))
    O = np.zeros(Q.shape, dtype=np.float64)
    for b in range(p.batch):
        for h in range(p.heads):
            s = p.slot(b, h)
            for qb in range(p.n_q):
                cq = int(p.q_valid[s, qb])
                J = [np.arange(p.kv_offset[s, kb], p.kv_offset[s, kb] + p.kv_valid[s, kb])
                     for kb in p.row(s, qb)]
                J = np.concatenate(J).astype(np.int64) if J else np.zeros(0, dtype=np.int64)
                if cq == 0 or len(J) == 0:
                    continue
                I = np.arange(128 * qb, 128 * qb + cq)
                S = (Q[b, h, I] @ K[b, h, J].T).astype(np.float32) * c2
                m = S.max(axis=1, keepdims=True)
                P = np.exp2(S - m).astype(np.float32)
                l = P.sum(axis=1, keepdims=True, dtype=np.float32)
                acc = (_bf16(P).astype(np.float64) @ V[b, h, J]).astype(np.float32)
                O[b, h, I] = _bf16(acc / l)
    return O


def _case(name, d):
    if name == "batch-2-per-head":  # the per-(batch, head) graphs of the batch tests
        from tests.test_gpu_batch import per_slot_problem
        p = per_slot_problem(2, 3, d, seed=d)
        return p, random_tensors(p, seed=31 + d)
    cq, ck, rows = EDGE_CASES[name]
    p = make_problem(cq, ck, rows, heads=3, head_dim=d, sort_rows=False)
    t = random_tensors(p, seed=len(name) + d)
    return p, t


CASES = list(EDGE_CASES) + ["batch-2-per-head"]


def test_rounding_bound_holds_for_emulated_forward():
    worst = 0.0
    for name in CASES:
        for d in (64, 128):
            p, t = _case(name, d)
            Oref, Lref = oracle_fwd(p, t["q"], t["k"], t["v"])
            Aabs = oracle_fwd(p, t["q"], t["k"], t["v"].abs())[0]
            Oemu = emulate_fwd(p, t["q"], t["k"], t["v"])
            live = np.isfinite(Lref)
            err = np.abs(Oemu - Oref)[live]
            bound = rounding_bound(Oref[live], Aabs[live])
            worst = max(worst, float((err / bound).max()))
            assert (err <= bound).all(), (name, d, float((err / bound).max()))
    assert worst > 0.3, worst  # the bound is not loose by orders of magnitude


def test_probability_rounding_term_is_needed():
    """Without the 2^-8 term for the probabilities rounded to bf16 the bound fails."""
    failed = False
    for name in CASES:
        for d in (64, 128):
            p, t = _case(name, d)
            Oref, Lref = oracle_fwd(p, t["q"], t["k"], t["v"])
            Aabs = oracle_fwd(p, t["q"], t["k"], t["v"].abs())[0]
            Oemu = emulate_fwd(p, t["q"], t["k"], t["v"])
            live = np.isfinite(Lref)
            err = np.abs(Oemu - Oref)[live]
            bound = rounding_bound(Oref[live], Aabs[live]) - P_ROUND * Aabs[live]
            failed = failed or bool((err > bound).any())
    assert failed
