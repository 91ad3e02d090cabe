"""Pins for the block-selection oracle (CPU only): a hand-worked example with ties, pure-Python
brute force in the same operation order, the independent top-87 selection of the 21x45x80
workload generator (numpy mean, BLAS product, stable argsort), and invariants."""
import numpy as np
import pytest

from oracle.selection import block_means, block_scores, select_topk, topk_rows
from workloads import make_workload


def _blocks(rows_per_block, d):
    x = np.zeros((128 * len(rows_per_block), d))
    for b, rows in enumerate(rows_per_block):
        for r, v in enumerate(rows):
            x[128 * b + r] = v
    return x, [len(r) for r in rows_per_block]


def test_worked_by_hand_with_ties():
    """Q means (2, 1) and (0, 1); K means (1, 1), (1, 1), none, (-1, 4).
    Scores: q0 -> 3, 3, -, 2; q1 -> 1, 1, -, 4."""
    xq, cq = _blocks([[[1, 0], [3, 2]], [[0, 1]]], 2)
    xk, ck = _blocks([[[1, 1]], [[2, 0], [0, 2]], [], [[-1, 4]]], 2)
    qbar, kbar = block_means(xq, cq), block_means(xk, ck)
    assert qbar.tolist() == [[2, 1], [0, 1]]
    assert kbar.tolist() == [[1, 1], [1, 1], [0, 0], [-1, 4]]
    s = block_scores(qbar, kbar)
    assert s[:, [0, 1, 3]].tolist() == [[3, 3, 2], [1, 1, 4]]
    assert topk_rows(s, cq, ck, 1) == [[0], [3]]        # tie 3 = 3 goes to the lower block
    assert topk_rows(s, cq, ck, 2) == [[0, 1], [0, 3]]  # tie 1 = 1 goes to the lower block
    assert topk_rows(s, cq, ck, 5) == [[0, 1, 3], [0, 1, 3]]  # block 2 (c = 0) never selected
    assert topk_rows(s, [0, 1], ck, 2) == [[], [0, 3]]  # an empty query block selects nothing


def test_brute_force_same_order():
    rng = np.random.default_rng(3)
    d, n_q, n_k = 5, 4, 6
    cq = [3, 0, 1, 128]
    ck = [2, 7, 0, 128, 1, 5]
    off = [256, 0, 0, 384, 128, 768]  # shuffled block placement
    xq = rng.standard_normal((128 * n_q, d))
    xk = rng.standard_normal((1024, d))
    qbar = block_means(xq, cq)
    kbar = block_means(xk, ck, off)
    for b in range(n_q):
        for j in range(d):
            acc = 0.0
            for r in range(cq[b]):
                acc += float(xq[128 * b + r, j])
            assert qbar[b, j] == (acc / cq[b] if cq[b] else 0.0)
    for b in range(n_k):
        for j in range(d):
            acc = 0.0
            for r in range(ck[b]):
                acc += float(xk[off[b] + r, j])
            assert kbar[b, j] == (acc / ck[b] if ck[b] else 0.0)
    s = block_scores(qbar, kbar)
    for a in range(n_q):
        for b in range(n_k):
            acc = 0.0
            for j in range(d):
                acc += float(qbar[a, j]) * float(kbar[b, j])
            assert s[a, b] == acc
    for top_k in (1, 2, 4, 10):
        rows = topk_rows(s, cq, ck, top_k)
        live = [k for k in range(n_k) if ck[k] > 0]
        for a in range(n_q):
            want = [] if cq[a] == 0 else sorted(sorted(live, key=lambda k: (-s[a, k], k))[:min(top_k, len(live))])
            assert rows[a] == want


def test_matches_the_workload_generator_top87():
    """The 21x45x80 workload's graph comes from an independent top-87 implementation; the two
    agree on every row, except where two scores tie to within 1e-9 (relative) at the cut."""
    w = make_workload(4, heads=[0, 1])
    q = w.q.float().numpy()
    k = w.k.float().numpy()
    got = select_topk(q, k, w.q_valid[0], w.kv_valid[0], w.kv_offset[0], 87)
    for g, (b, h) in enumerate([(0, 0), (0, 1)]):
        qbar = block_means(q[b, h], w.q_valid[0])
        kbar = block_means(k[b, h], w.kv_valid[0], w.kv_offset[0])
        s = block_scores(qbar, kbar)
        mism = 0
        for qb in range(w.n_q):
            ref = w.q2k_idx[w.q2k_ptr[g, qb]:w.q2k_ptr[g, qb + 1]].tolist()
            mine = got[(b, h)][qb]
            if ref != mine:
                mism += 1
                cut = np.sort(s[qb])[::-1][86]
                for kb in set(ref) ^ set(mine):
                    assert abs(s[qb, kb] - cut) <= 1e-9 * np.abs(s[qb]).max()
        assert mism <= 2, mism


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_invariants(seed):
    rng = np.random.default_rng(seed)
    n_q, n_k, d = 9, 13, 8
    cq = rng.choice([0, 1, 16, 100, 128], size=n_q)
    ck = rng.choice([0, 1, 16, 100, 128], size=n_k)
    xq = rng.standard_normal((128 * n_q, d))
    xk = rng.standard_normal((128 * n_k, d))
    s = block_scores(block_means(xq, cq), block_means(xk, ck))
    for top_k in (1, 3, 20):
        rows = topk_rows(s, cq, ck, top_k)
        # doubling K is exact in binary floating point: the selection is unchanged
        s2 = block_scores(block_means(xq, cq), block_means(2 * xk, ck))
        assert topk_rows(s2, cq, ck, top_k) == rows
        live = [k for k in range(n_k) if ck[k] > 0]
        for a in range(n_q):
            r = rows[a]
            assert r == sorted(set(r))
            assert len(r) == (0 if cq[a] == 0 else min(top_k, len(live)))
            if r:
                rest = [k for k in live if k not in r]
                assert all(s[a, x] >= s[a, y] for x in r for y in rest)


def test_top_p_worked_by_hand():
    """Scores log 6, log 3, 0 give softmax 0.6, 0.3, 0.1 (cumulative 0.6, 0.9, 1.0)."""
    from oracle.selection import top_p_clusters
    s = np.array([np.log(3.0), 0.0, np.log(6.0), -50.0])
    live = [0, 1, 2]  # cluster 3 has no tokens
    assert top_p_clusters(s, live, 0.5) == [2]
    assert top_p_clusters(s, live, 0.85) == [0, 2]
    assert top_p_clusters(s, live, 0.95) == [0, 1, 2]
    assert top_p_clusters(s, [], 0.9) == []
    # equal scores: the lower cluster comes first
    t = np.array([1.0, 1.0, 1.0, 1.0])
    assert top_p_clusters(t, [0, 1, 2, 3], 0.3) == [0, 1]   # 0.25 < 0.3 <= 0.5
    assert top_p_clusters(t, [3, 1, 2], 0.3) == [1]         # 1/3 >= 0.3


def test_top_p_block_lists_worked_by_hand():
    """Two Q clusters, three K clusters (cluster 1 empty); centroids make cluster 0 prefer K
    cluster 2 strongly and cluster 1 split evenly; K blocks 0..4 belong to clusters 0,2,2,0,-1."""
    from oracle.selection import select_top_p
    qc = np.array([[10.0, 0.0], [0.0, 0.0]])
    kc = np.array([[0.0, 1.0], [5.0, 5.0], [1.0, 0.0]])
    rows = select_top_p(qc, kc, q_size=[3, 1], k_size=[4, 0, 7], q_block_cluster=[1, 0, -1, 0],
                        k_block_cluster=[0, 2, 2, 0, -1], top_p=0.9, scale=1.0)
    # cluster 0: scores 0 (k0), 10 (k2): p(k2) = 1 / (1 + e^-10) > 0.9 -> {2}
    # cluster 1: scores 0, 0: p = 0.5 each -> both needed for 0.9 -> {0, 2}
    assert rows == [[0, 1, 2, 3], [1, 2], [], [1, 2]]


def test_top_p_matches_the_workload_generator():
    """The SVG2-like workload's graph comes from an independent implementation of the same rule
    (numpy product, division by sqrt(d)); every row agrees on two heads."""
    from oracle.selection import select_top_p
    w = make_workload(5, heads=[0, 1])
    for g in range(2):
        c = w.clusters[g]
        rows = select_top_p(c["q_cent"], c["k_cent"], c["q_size"], c["k_size"], c["q_block_cluster"],
                            c["k_block_cluster"], 0.9, 1.0 / np.sqrt(w.head_dim))
        for q in range(w.n_q):
            assert rows[q] == w.q2k_idx[w.q2k_ptr[g, q]:w.q2k_ptr[g, q + 1]].tolist(), (g, q)
