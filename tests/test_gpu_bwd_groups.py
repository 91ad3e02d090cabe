"""Backward with Q groups (KPage paper, section 3.3.2: each owner's reverse neighbourhood
split into groups of q_group Q blocks, one work item per non-empty (owner, group)) against
the fp64 oracle, through the C ABI.  Owners split over several items sum fp32 partials in
a reduce pass; the tolerance is the one of the one-group backward (max-norm-relative
2e-2), and rows without any valid pair must still be exactly zero.
"""
import numpy as np
import pytest

import block_sparse_attention_11_amd as K
from oracle import oracle_bwd
from tests.problems import make_problem, random_tensors
from tests.test_gpu_bwd import _say, check_grads, gpu_fwd_bwd
from tests.test_gpu_fwd import EDGE_CASES
from workloads import make_workload

pytestmark = pytest.mark.gpu

CASES = {
    "tiny 5x6x10 d=64, q_group 1": (lambda: make_workload(1, with_do=True), 1),
    "tiny 5x6x10 d=64, q_group 3": (lambda: make_workload(1, with_do=True), 3),
    "21x30x52 one head, q_group 1": (lambda: make_workload(3, heads=[0], with_do=True), 1),
    "21x30x52 one head, q_group 16": (lambda: make_workload(3, heads=[0], with_do=True), 16),
    "SVG2-like partitions one head, q_group 8": (lambda: make_workload(5, heads=[1], with_do=True), 8),
}


@pytest.mark.parametrize("name", list(CASES))
def test_bwd_q_groups(name):
    make, q_group = CASES[name]
    w = make()
    plan = K.kpage_plan(w, q_group=q_group)
    base = 8 * w.batch * w.heads * w.seq_q
    ws = K.kpage_bwd_workspace_size(plan)
    _say(f"[bwd groups] {name}: {len(K.kpage_plan_export(plan, 'bwd_queue')) // 2} items, workspace {ws} B")
    assert ws > base  # some owner is split over several groups at these sizes
    got = gpu_fwd_bwd(w, w.q, w.k, w.v, w.do, plan=plan)
    ref = oracle_bwd(w, w.q, w.k, w.v, w.do)[:3]
    check_grads(got, ref, name, w)


@pytest.mark.parametrize("name", list(EDGE_CASES))
def test_bwd_q_groups_edge_cases(name):
    cq, ck, rows = EDGE_CASES[name]
    p = make_problem(cq, ck, rows, heads=2, head_dim=128, sort_rows=False)
    t = random_tensors(p, seed=len(name))
    _say(f"[bwd groups] edge case {name}, q_group 1")
    got = gpu_fwd_bwd(p, t["q"], t["k"], t["v"], t["do"], plan=K.kpage_plan(p, q_group=1))
    ref = oracle_bwd(p, t["q"], t["k"], t["v"], t["do"])[:3]
    check_grads(got, ref, f"{name} q_group 1", p)


def test_bwd_q_groups_deterministic_and_close_to_one_group():
    """Partials are summed in group order: bitwise repeatable; and equal to the one-group
    gradients up to fp32 summation order and bf16 rounding."""
    w = make_workload(3, heads=[0, 1], with_do=True)
    plan = K.kpage_plan(w, q_group=4)
    _say("[bwd groups] run-to-run, q_group 4")
    a = gpu_fwd_bwd(w, w.q, w.k, w.v, w.do, plan=plan)
    b = gpu_fwd_bwd(w, w.q, w.k, w.v, w.do, plan=plan)
    c = gpu_fwd_bwd(w, w.q, w.k, w.v, w.do)
    for name, x, y, z in zip(("dQ", "dK", "dV"), a, b, c):
        assert np.array_equal(x, y), name
        err = np.abs(x - z).max() / max(np.abs(z).max(), 1e-2)
        _say(f"  {name}: q_group 4 vs one group max-norm-rel {err:.2e}")
        assert err <= 1e-2, name
