"""kpage_attn_bwd_noalloc (workspace in the library's static device scratch) against
kpage_attn_bwd (caller workspace), through the C ABI: bit-identical gradients on two
calls in a row, the second on a smaller problem, and the size and precondition checks
(rejected before any device work)."""
import sys

import pytest
import torch

import block_sparse_attention_11_amd as K
from tests.problems import make_problem
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _both(w, label):
    dev = torch.device("cuda", 0)
    plan = K.kpage_plan(w)
    q, k, v, do = (x.to(dev) for x in (w.q, w.k, w.v, w.do))
    o, lse = K.attn_fwd(plan, q, k, v, w.scale)
    _say(f"[noalloc] {label}: B={w.batch} H={w.heads} seq_q={w.seq_q}")
    ref = K.attn_bwd(plan, q, k, v, o, lse, do, w.scale)  # builds and uploads the backward tables
    got = [torch.full_like(x, float("nan")) for x in ref]
    K.kpage_attn_bwd_noalloc(plan, q, k, v, o, lse, do, *got, w.scale)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), ref, got):
        assert torch.equal(a, b), (label, name)
    plan.close()


def test_noalloc_backward_equals_workspace_backward_twice():
    # a large problem first (13.8 MB of the 32 MiB scratch), then a smaller one reusing it
    _both(make_workload(3, with_do=True), "21x30x52, 40 heads")
    _both(make_workload(1, with_do=True), "tiny 5x6x10, 2 heads")


def test_noalloc_backward_with_q_groups():
    """Q-group partials in the scratch: the tiny layout with groups of one Q block fits;
    the 21x30x52 layout with groups of 16 needs 720 MB of partials and is rejected."""
    dev = torch.device("cuda", 0)
    for w, group, fits in ((make_workload(1, with_do=True), 1, True),
                           (make_workload(3, heads=[0, 1], with_do=True), 16, False)):
        plan = K.kpage_plan(w, q_group=group)
        q, k, v, do = (x.to(dev) for x in (w.q, w.k, w.v, w.do))
        o, lse = K.attn_fwd(plan, q, k, v, w.scale)
        _say(f"[noalloc] B={w.batch} H={w.heads} seq_q={w.seq_q}, Q groups of {group}")
        ref = K.attn_bwd(plan, q, k, v, o, lse, do, w.scale)
        got = [torch.full_like(x, float("nan")) for x in ref]
        if not fits:
            assert K.kpage_bwd_workspace_size(plan) > K.NOALLOC_SCRATCH_BYTES
            with pytest.raises(K.KpageError) as e:
                K.kpage_attn_bwd_noalloc(plan, q, k, v, o, lse, do, *got, w.scale)
            assert e.value.status == K.KPAGE_ERR_INVALID and "static scratch" in str(e.value)
            continue
        K.kpage_attn_bwd_noalloc(plan, q, k, v, o, lse, do, *got, w.scale)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), ref, got):
            assert torch.equal(a, b), name


def test_noalloc_rejects_before_device_work():
    dev = torch.device("cuda", 0)
    # tables not built yet
    w = make_workload(1, with_do=True)
    plan = K.kpage_plan(w)
    q, k, v, do = (x.to(dev) for x in (w.q, w.k, w.v, w.do))
    o = torch.zeros_like(q)
    lse = torch.zeros(q.shape[:3], dtype=torch.float32, device=dev)
    outs = [torch.empty_like(x) for x in (q, k, v)]
    with pytest.raises(K.KpageError) as e:
        K.kpage_attn_bwd_noalloc(plan, q, k, v, o, lse, do, *outs, w.scale)
    assert e.value.status == K.KPAGE_ERR_INVALID and "kpage_attn_bwd once" in str(e.value)
    # workspace above the scratch: 64 heads x 520 query blocks = 4,259,840 rows x 8 bytes
    big = make_problem([128] * 520, [128], [[0]] * 520, heads=64, head_dim=64)
    bplan = K.kpage_plan(big)
    assert K.kpage_bwd_workspace_size(bplan) > K.NOALLOC_SCRATCH_BYTES
    shape_q = (1, 64, big.seq_q, 64)
    shape_k = (1, 64, big.seq_kv, 64)
    tq = torch.zeros(shape_q, dtype=torch.bfloat16, device=dev)
    tk = torch.zeros(shape_k, dtype=torch.bfloat16, device=dev)
    tl = torch.zeros(shape_q[:3], dtype=torch.float32, device=dev)
    with pytest.raises(K.KpageError) as e:
        K.kpage_attn_bwd_noalloc(bplan, tq, tk, tk, tq, tl, tq, tq, tk, tk, big.scale)
    assert e.value.status == K.KPAGE_ERR_INVALID and "static scratch" in str(e.value)
