"""Batch > 1 through the C ABI: every kernel indexes (batch, head) as b * heads + h, and a
plan with one graph per (batch, head) looks its graph up by that slot.

Forward and backward parity with the fp64 oracle for a graph shared by every (batch, head)
and for one graph per (batch, head), both routes, d = 64 and 128 (the synthetic-case
tolerances of test_gpu_fwd and those of test_gpu_bwd); and the GPU planner's tables equal the host planner's for the
per-(batch, head) graphs.
"""
import sys

import numpy as np
import pytest

from oracle import oracle_bwd, oracle_fwd
from tests.problems import Problem, make_problem, random_tensors
from tests.test_gpu_bwd import check_grads, gpu_fwd_bwd
from tests.test_gpu_fwd import abs_values_attention, check, gpu_fwd
from tests.test_gpu_plan_device import same_plans

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def per_slot_problem(batch, heads, d, seed):
    """One seeded random layout and graph per (batch, head): block sizes on both sides
    (both routes, tails, empty blocks) and selection lists of random length and order."""
    rng = np.random.default_rng(seed)
    G, n_q, n_kv = batch * heads, 5, 7
    qv = rng.choice([128, 100, 64, 33, 20, 0, 128], size=(G, n_q)).astype(np.int32)
    kv = rng.choice([128, 128, 77, 64, 16, 3, 0], size=(G, n_kv)).astype(np.int32)
    off = np.tile(np.arange(n_kv, dtype=np.int64) * 128, (G, 1))
    ptr = np.zeros((G, n_q + 1), dtype=np.int64)
    idx = []
    for g in range(G):
        ptr[g, 0] = len(idx)
        for q in range(n_q):
            idx.extend(rng.permutation(n_kv)[:int(rng.integers(0, n_kv + 1))].tolist())
            ptr[g, q + 1] = len(idx)
    return Problem(batch=batch, heads=heads, head_dim=d, n_q=n_q, n_kv=n_kv, seq_q=128 * n_q,
                   seq_kv=128 * n_kv, per_head=True, q_valid=qv, kv_valid=kv, kv_offset=off,
                   q2k_ptr=ptr, q2k_idx=np.asarray(idx, dtype=np.int32))


def shared_problem(d):
    return make_problem([128, 64, 100, 20, 0], [128, 50, 128, 7, 128, 96],
                        [[0, 1, 2], [2, 3], [0, 4, 5, 1], [5], [1]], heads=3, batch=2, head_dim=d,
                        sort_rows=False)


def _fwd_bwd(p, seed, label):
    t = random_tensors(p, seed=seed)
    _say(f"[batch] {label}: B={p.batch} H={p.heads} d={p.head_dim} per_head={p.per_head}")
    O, L = gpu_fwd(p, t["q"], t["k"], t["v"])
    Oref, Lref = oracle_fwd(p, t["q"], t["k"], t["v"])
    check(O, L, Oref, Lref, label, Aabs=abs_values_attention(p, t["q"], t["k"], t["v"]))
    got = gpu_fwd_bwd(p, t["q"], t["k"], t["v"], t["do"])
    ref = oracle_bwd(p, t["q"], t["k"], t["v"], t["do"])[:3]
    check_grads(got, ref, label, p)


@pytest.mark.parametrize("d", [64, 128])
def test_batch2_shared_graph(d):
    _fwd_bwd(shared_problem(d), 21 + d, f"batch 2 shared graph d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_batch2_per_head_graphs(d):
    _fwd_bwd(per_slot_problem(2, 3, d, seed=d), 31 + d, f"batch 2 per-(batch, head) graphs d={d}")


def test_batch2_device_plan_equals_host_plan():
    for seed in range(3):
        same_plans(per_slot_problem(2, 3, 64, seed=100 + seed), f"batch 2 per-(batch, head) graphs, seed {seed}")
