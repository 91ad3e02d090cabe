"""The C++ planner behind the C ABI against the oracle planner, bit for bit (CPU only: planning
touches no device memory)."""
import numpy as np
import pytest

import block_sparse_attention_11_amd as K
from oracle import oracle_plan
from tests.problems import make_problem
from workloads import make_workload


def _assert_same(problem, **opts):
    plan = K.kpage_plan(problem, **opts)
    ref = oracle_plan(problem, **{k: v for k, v in opts.items() if v})
    for name in K.TABLES:
        if name.startswith("group_"):  # launch-level grouping, not part of the paper's tables
            continue
        got = K.kpage_plan_export(plan, name)
        want = getattr(ref, name).reshape(-1)
        assert got.dtype == want.dtype or got.dtype.kind == want.dtype.kind, name
        assert np.array_equal(got, want.astype(got.dtype)), name
    assert K.kpage_plan_stats(plan) == ref.stats
    plan.close()


@pytest.mark.parametrize("cfg,heads", [(1, None), (2, [0, 1]), (3, [0, 1, 2]), (4, [0, 5]), (5, [3, 7])])
def test_workloads_bit_exact(cfg, heads):
    _assert_same(make_workload(cfg, heads=heads))


def test_alignment_options_bit_exact():
    _assert_same(make_workload(3, heads=[0]), align_q64=32, align_q128=16)


def test_random_small_layouts_bit_exact():
    rng = np.random.default_rng(7)
    sizes = [0, 1, 2, 15, 16, 17, 31, 48, 63, 64, 65, 100, 112, 113, 127, 128]
    for _ in range(60):
        n_q, n_kv = int(rng.integers(1, 14)), int(rng.integers(1, 14))
        cq = rng.choice(sizes, size=n_q)
        ck = rng.choice(sizes, size=n_kv)
        rows = [rng.permutation(n_kv)[:int(rng.integers(0, n_kv + 1))].tolist() for _ in range(n_q)]
        # packed Page16 offsets in a shuffled block order: independent-partition style layout
        order = rng.permutation(n_kv)
        off = np.zeros(n_kv, dtype=np.int64)
        acc = 0
        for k in order:
            off[k] = acc
            acc += 16 * ((int(ck[k]) + 15) // 16) + 16 * int(rng.integers(0, 2))
        p = make_problem(cq, ck, rows, heads=int(rng.integers(1, 3)), kv_offset=off, head_dim=64,
                         seq_kv=max(16, acc), sort_rows=False)
        _assert_same(p)


@pytest.mark.parametrize("mutate,status", [
    (lambda p: setattr(p, "head_dim", 96), K.KPAGE_ERR_UNSUPPORTED),
    (lambda p: p.q_valid.__setitem__((0, 0), 129), K.KPAGE_ERR_INVALID),
    (lambda p: p.kv_valid.__setitem__((0, 1), -1), K.KPAGE_ERR_INVALID),
    (lambda p: p.kv_offset.__setitem__((0, 1), 8), K.KPAGE_ERR_INVALID),
    (lambda p: p.kv_offset.__setitem__((0, 1), 0), K.KPAGE_ERR_INVALID),        # overlapping footprints
    (lambda p: p.q2k_idx.__setitem__(0, 7), K.KPAGE_ERR_INVALID),                # block id out of range
    (lambda p: p.q2k_idx.__setitem__(1, p.q2k_idx[0]), K.KPAGE_ERR_INVALID),     # duplicate in a row
    (lambda p: setattr(p, "seq_q", 100), K.KPAGE_ERR_INVALID),
    (lambda p: setattr(p, "seq_kv", 250), K.KPAGE_ERR_INVALID),
])
def test_invalid_descriptors_are_rejected_before_device_work(mutate, status):
    p = make_problem([128, 40], [128, 64, 16], [[0, 1, 2], [2]], head_dim=128)
    mutate(p)
    with pytest.raises(K.KpageError) as e:
        K.kpage_plan(p)
    assert e.value.status == status
    assert K.kpage_last_error()


def test_negative_q_group_is_invalid():
    p = make_problem([128], [128], [[0]], head_dim=128)
    with pytest.raises(K.KpageError) as e:
        K.kpage_plan(p, q_group=-1)
    assert e.value.status == K.KPAGE_ERR_INVALID


@pytest.mark.parametrize("q_group", [1, 2, 5, 64])
@pytest.mark.parametrize("cfg,heads", [(1, None), (3, [0]), (5, [3])])
def test_q_groups_bit_exact(cfg, heads, q_group):
    _assert_same(make_workload(cfg, heads=heads), q_group=q_group)


def test_q_groups_random_small_layouts_bit_exact():
    rng = np.random.default_rng(11)
    sizes = [0, 1, 16, 17, 64, 65, 127, 128]
    for _ in range(40):
        n_q, n_kv = int(rng.integers(1, 12)), int(rng.integers(1, 12))
        rows = [rng.permutation(n_kv)[:int(rng.integers(0, n_kv + 1))].tolist() for _ in range(n_q)]
        p = make_problem(rng.choice(sizes, size=n_q), rng.choice(sizes, size=n_kv), rows, heads=2, head_dim=64,
                         sort_rows=False)
        _assert_same(p, q_group=int(rng.integers(1, n_q + 2)))


@pytest.mark.parametrize("key,q_group", [("walk_order", 0), ("queue_ties", 0), ("queue_ties", 2)])
def test_order_convention_layouts_bit_exact(key, q_group):
    """The hand-worked layouts that pin the walk, queue and work-order readings in the oracle."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "order_conventions.json")) as f:
        g = json.load(f)[key]
    p = make_problem(g["q_valid"], g["kv_valid"], g["rows"], heads=g.get("heads", 1), head_dim=64, sort_rows=False)
    _assert_same(p, q_group=q_group)
