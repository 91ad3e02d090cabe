"""Group items on the GPU against the fp64 CPU oracle (through the C ABI).

A group item runs up to four query blocks of at most 32 valid rows over the union of
their page walks, one member per wave, each wave masking the pages its own block did
not select; it writes every member block's 128 output rows.  Checked here: forward O and
LSE and the gradients on layouts built to form groups of two, three and four members
(tails, 1- and 8-row blocks, empty blocks next to members), groups whose items take the
exact re-run, every member block of the top-87 workload, a group over both ends of a
2^21-row K/V sequence (the longest the grouping takes), and batch 2 with a shared graph
and with one graph per (batch, head) (there also the GPU planner's groups against the
host's); the same problems planned without groups agree with the oracle too.  Tolerances
as in the forward and backward parity tests.
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_11_amd as K
from oracle import oracle_bwd, oracle_fwd
from tests.problems import Problem, make_problem, random_tensors
from tests.test_gpu_bwd import check_grads, gpu_fwd_bwd
from tests.test_gpu_fwd import abs_values_attention, check, gpu_fwd
from tests.test_gpu_plan_device import same_plans
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def group_sizes(plan):
    m = K.kpage_plan_export(plan, "group_members").reshape(-1, 4)
    return sorted(int(x) for x in (m >= 0).sum(axis=1))


def small_blocks_problem(d, batch=1):
    """14 query blocks: 11 of at most 32 rows (1, 8, 16, 17, 20, 31 and 32 rows), one empty,
    two large.  K blocks 0-5 full or with tails; the small blocks select overlapping
    subsets of K blocks 0-4 (so they form groups of 2-4), two select disjoint ones."""
    cq = [128, 20, 32, 8, 32, 0, 31, 1, 17, 16, 32, 100, 32, 24]
    ck = [128, 128, 70, 128, 9, 128, 33]
    rows = [[0, 1, 2, 3], [0, 1, 2], [0, 1, 2, 4], [0, 1], [1, 2, 0], [0], [3, 4, 2], [3, 4], [2, 3, 4, 1],
            [4, 3], [5, 6], [0, 5, 6], [6, 5], [1, 0, 2, 6]]
    return make_problem(cq, ck, rows, heads=3, batch=batch, head_dim=d, sort_rows=False)


@pytest.mark.parametrize("d", [64, 128])
def test_groups_forward_and_backward(d):
    p = small_blocks_problem(d)
    t = random_tensors(p, seed=70 + d)
    plan = K.kpage_plan(p)
    sizes = group_sizes(plan)
    _say(f"[groups] small blocks d={d}: group sizes {sizes}")
    assert len(sizes) >= 2 and max(sizes) >= 3
    O, L = gpu_fwd(p, t["q"], t["k"], t["v"], plan=plan)
    Oref, Lref = oracle_fwd(p, t["q"], t["k"], t["v"])
    check(O, L, Oref, Lref, f"groups d={d}", Aabs=abs_values_attention(p, t["q"], t["k"], t["v"]))
    got = gpu_fwd_bwd(p, t["q"], t["k"], t["v"], t["do"], plan=plan)
    ref = oracle_bwd(p, t["q"], t["k"], t["v"], t["do"])[:3]
    check_grads(got, ref, f"groups d={d}", p)


def test_ungrouped_plan_matches_oracle_too():
    p = small_blocks_problem(128)
    t = random_tensors(p, seed=71)
    plan = K.kpage_plan(p, grouped=False)
    assert group_sizes(plan) == []
    _say("[groups] same problem, no groups")
    O, L = gpu_fwd(p, t["q"], t["k"], t["v"], plan=plan)
    Oref, Lref = oracle_fwd(p, t["q"], t["k"], t["v"])
    check(O, L, Oref, Lref, "ungrouped", Aabs=abs_values_attention(p, t["q"], t["k"], t["v"]))


@pytest.mark.parametrize("d", [64, 128])
def test_groups_take_the_exact_rerun(d):
    """Scores that rise by far more than 2^64 (base 2) after the first pages of every walk:
    every group item is marked and re-run by the exact kernel."""
    p = small_blocks_problem(d)
    t = random_tensors(p, seed=72 + d)
    g = torch.Generator().manual_seed(73)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    amp = 30.0 * (128.0 / d) ** 0.5
    q = t["q"].float() + amp * u
    k = t["k"].float()
    k[:, :, 128:] += amp * u  # every K block but block 0
    for x, c in ((q, p.q_valid[0]), (k, p.kv_valid[0])):
        for b, n in enumerate(c):
            x[:, :, 128 * b + int(n):128 * (b + 1)] = 0
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    plan = K.kpage_plan(p)
    assert group_sizes(plan)
    _say(f"[groups] score rise d={d}")
    O, L = gpu_fwd(p, q, k, t["v"], plan=plan)
    Oref, Lref = oracle_fwd(p, q, k, t["v"])
    check(O, L, Oref, Lref, f"groups score rise d={d}", Aabs=abs_values_attention(p, q, k, t["v"]))


def test_topk_workload_every_member_block():
    """Two heads of the 21x45x80 top-87 workload (per-head graphs): every block that runs
    inside a group item, forward; one head's gradients."""
    w = make_workload(4, heads=[0, 1], with_do=True)
    plan = K.kpage_plan(w)
    m = K.kpage_plan_export(plan, "group_members").reshape(-1, 4)
    ptr = K.kpage_plan_export(plan, "group_ptr")
    items = [(0, h, int(q)) for h in range(2) for i in range(int(ptr[h]), int(ptr[h + 1])) for q in m[i] if q >= 0]
    _say(f"[groups] top-87 two heads: {len(items)} member blocks in {m.shape[0]} groups")
    assert len(items) > 100
    O, L = gpu_fwd(w, w.q, w.k, w.v, plan=plan)
    Oref, Lref = oracle_fwd(w, w.q, w.k, w.v, items=items)
    check(O, L, Oref, Lref, "top-87 group members")
    got = gpu_fwd_bwd(w, w.q, w.k, w.v, w.do, plan=plan)
    ref = oracle_bwd(w, w.q, w.k, w.v, w.do, heads=[1])[:3]
    check_grads(got, ref, "top-87 groups head 1", w, heads=[1])


def test_groups_at_the_page_bitset_limit():
    """K/V of 2^21 rows, the longest sequence whose page bitsets (2048 words) the grouping
    takes: three small blocks form one group item whose union walk holds pages at both ends
    of the sequence (page ids up to 2^17 - 1); forward and backward against the oracle."""
    seq_kv = 2048 * 64 * 16
    p = make_problem([20, 32, 8], [128, 128, 128], [[0, 1], [0, 1], [0, 2]], heads=1, head_dim=64,
                     kv_offset=[0, 128, seq_kv - 128], seq_kv=seq_kv)
    t = random_tensors(p, seed=79)
    plan = K.kpage_plan(p)
    assert group_sizes(plan) == [3]
    assert int(K.kpage_plan_export(plan, "group_walk").max()) == seq_kv // 16 - 1
    _say(f"[groups] seq_kv {seq_kv}: one group of 3 over both ends of K/V")
    O, L = gpu_fwd(p, t["q"], t["k"], t["v"], plan=plan)
    Oref, Lref = oracle_fwd(p, t["q"], t["k"], t["v"])
    check(O, L, Oref, Lref, "groups at the page-bitset limit",
          Aabs=abs_values_attention(p, t["q"], t["k"], t["v"]))
    got = gpu_fwd_bwd(p, t["q"], t["k"], t["v"], t["do"], plan=plan)
    ref = oracle_bwd(p, t["q"], t["k"], t["v"], t["do"])[:3]
    check_grads(got, ref, "groups at the page-bitset limit", p)


def per_slot_small_blocks(batch, heads, d, seed):
    """One graph per (batch, head): mostly blocks of at most 32 rows whose selections share a
    random base set of K blocks, so that every slot forms its own groups."""
    rng = np.random.default_rng(seed)
    G, n_q, n_kv = batch * heads, 9, 7
    qv = rng.choice([20, 32, 8, 1, 31, 16, 128, 64, 0], size=(G, n_q)).astype(np.int32)
    kv = rng.choice([128, 128, 77, 64, 16, 3], size=(G, n_kv)).astype(np.int32)
    off = np.tile(np.arange(n_kv, dtype=np.int64) * 128, (G, 1))
    ptr = np.zeros((G, n_q + 1), dtype=np.int64)
    idx = []
    for g in range(G):
        base = rng.permutation(n_kv)[:3].tolist()
        ptr[g, 0] = len(idx)
        for q in range(n_q):
            extra = rng.permutation(n_kv)[:int(rng.integers(0, 3))].tolist()
            idx.extend(rng.permutation(sorted(set(base + extra))).tolist())
            ptr[g, q + 1] = len(idx)
    return Problem(batch=batch, heads=heads, head_dim=d, n_q=n_q, n_kv=n_kv, seq_q=128 * n_q,
                   seq_kv=128 * n_kv, per_head=True, q_valid=qv, kv_valid=kv, kv_offset=off,
                   q2k_ptr=ptr, q2k_idx=np.asarray(idx, dtype=np.int32))


@pytest.mark.parametrize("per_head", [False, True])
def test_groups_batch2(per_head):
    """Batch 2 x 3 heads: group items of a graph shared by every (batch, head), and of one graph
    per (batch, head); forward and backward against the oracle, and the GPU planner's groups
    equal the host's."""
    p = per_slot_small_blocks(2, 3, 128, seed=77) if per_head else small_blocks_problem(128, batch=2)
    t = random_tensors(p, seed=78)
    plan = K.kpage_plan(p)
    sizes = group_sizes(plan)
    _say(f"[groups] batch 2, per_head={per_head}: group sizes {sizes}")
    assert len(sizes) >= 3
    O, L = gpu_fwd(p, t["q"], t["k"], t["v"], plan=plan)
    Oref, Lref = oracle_fwd(p, t["q"], t["k"], t["v"])
    check(O, L, Oref, Lref, f"groups batch 2 per_head={per_head}", Aabs=abs_values_attention(p, t["q"], t["k"], t["v"]))
    got = gpu_fwd_bwd(p, t["q"], t["k"], t["v"], t["do"], plan=plan)
    ref = oracle_bwd(p, t["q"], t["k"], t["v"], t["do"])[:3]
    check_grads(got, ref, f"groups batch 2 per_head={per_head}", p)
    same_plans(p, f"groups batch 2 per_head={per_head}", bwd=False)
