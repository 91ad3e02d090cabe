"""Block selection in front of KPage, plain and slow (TEST INFRASTRUCTURE ONLY).

KPage consumes a sparse block graph produced by a selector and is independent of which
selector produced it (KPage paper, sections 1 and 2: VSA's dynamic selection over 3D
video blocks, SSTA's window plus top-k selection; section 4.6 lists them).  The paper
does not restate a selector's formulas; the plainest reading of "dynamic selection over
blocks" taken here, for one block layout shared by all heads:

  block mean     xbar_b = (sum of the c_b valid rows of block b) / c_b, in fp64, the rows
                 added one at a time in ascending order (b with c_b = 0 has no mean)
  block score    s_qk = qbar_q . kbar_k, in fp64, the products added one at a time over
                 ascending columns (every product and every sum rounded on its own)
  selection      for each query block with c_q > 0: the min(top_k, n_live) key blocks
                 with c_k > 0 of largest s_qk, ties to the lower block index, listed in
                 ascending block order; a query block with c_q = 0 selects nothing

The fixed operation order makes the scores, and so the selected sets, a function of the
inputs alone, so a GPU implementation that follows the same order must select exactly
the same blocks.

Cluster selection (SVG2-style: Q and K tokens clustered and permuted into independent
partitions, KPage paper sections 3.4.1 and 4.6; the selection rule is SVG2's, read as):

  cluster score  s_ck = scale * (qcent_c . kcent_k), the dot product as above over the
                 fp32 centroids widened to fp64, then one rounded product with scale
  kept clusters  for each Q cluster with tokens, the K clusters with tokens ordered by
                 score descending (ties to the lower cluster); softmax probabilities
                 p = exp(s - s_max) / sum; keep the shortest prefix whose cumulative
                 probability reaches top_p (all of them if rounding never reaches it)
  block lists    a Q block of cluster c selects every K block of a kept cluster, in
                 ascending block order; a Q block without a cluster selects nothing

The exponential and the probability sums are where two correct implementations may
round differently: a cut can only move where the cumulative probability lies within
rounding of top_p.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

BLOCK = 128


def block_means(x: np.ndarray, valid: Sequence[int], offset: Optional[Sequence[int]] = None) -> np.ndarray:
    """fp64 means of the valid rows of each block of ``x`` ([rows, d], any float dtype)."""
    x = np.asarray(x, dtype=np.float64)
    n, d = len(valid), x.shape[1]
    off = [BLOCK * b for b in range(n)] if offset is None else [int(o) for o in offset]
    acc = np.zeros((n, d))
    for r in range(BLOCK):  # row r of every block that has one, blocks side by side
        live = [b for b in range(n) if int(valid[b]) > r]
        if not live:
            break
        acc[live] = acc[live] + x[[off[b] + r for b in live]]
    out = np.zeros((n, d))
    for b in range(n):
        if int(valid[b]) > 0:
            out[b] = acc[b] / float(valid[b])
    return out


def block_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """s[q, k] = sum over ascending columns j of qbar[q, j] * kbar[k, j], each step rounded."""
    s = np.zeros((qbar.shape[0], kbar.shape[0]))
    for j in range(qbar.shape[1]):
        s = s + np.multiply.outer(qbar[:, j], kbar[:, j])
    return s


def topk_rows(scores: np.ndarray, q_valid: Sequence[int], kv_valid: Sequence[int], top_k: int) -> List[List[int]]:
    """Selected key blocks of every query block (ascending), by the rule in the module header."""
    live = np.asarray([k for k in range(len(kv_valid)) if int(kv_valid[k]) > 0], dtype=np.int64)
    kk = min(top_k, len(live))
    rows = []
    for q in range(len(q_valid)):
        if int(q_valid[q]) == 0 or kk == 0:
            rows.append([])
            continue
        order = np.lexsort((live, -scores[q, live]))  # score descending, then block ascending
        rows.append(sorted(int(live[i]) for i in order[:kk]))
    return rows


def select_topk(q: np.ndarray, k: np.ndarray, q_valid, kv_valid, kv_offset, top_k: int, heads=None):
    """Per (b, h) selected lists for Q, K of shape [B, H, S, d]; returns {(b, h): rows}."""
    B, H = q.shape[0], q.shape[1]
    out = {}
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            qbar = block_means(q[b, h], q_valid)
            kbar = block_means(k[b, h], kv_valid, kv_offset)
            out[(b, h)] = topk_rows(block_scores(qbar, kbar), q_valid, kv_valid, top_k)
    return out


def top_p_clusters(scores: np.ndarray, live: Sequence[int], top_p: float) -> List[int]:
    """Kept K clusters of one Q cluster (ascending), by the rule in the module header."""
    live = np.asarray(list(live), dtype=np.int64)
    if len(live) == 0:
        return []
    x = scores[live]
    order = np.lexsort((live, -x))
    z = x[order] - x[order[0]]
    e = np.exp(z)
    csum = np.cumsum(e / e.sum())
    m = int(np.searchsorted(csum, top_p)) + 1  # first index whose cumulative probability >= top_p
    return sorted(int(c) for c in live[order[:min(m, len(order))]])


def select_top_p(q_cent, k_cent, q_size, k_size, q_block_cluster, k_block_cluster, top_p: float, scale: float):
    """Block lists of one (b, h) from its clustering (every argument as in the module header)."""
    qc = np.asarray(q_cent, dtype=np.float64)
    kc = np.asarray(k_cent, dtype=np.float64)
    s = block_scores(qc, kc) * float(scale)
    live = [k for k in range(kc.shape[0]) if int(k_size[k]) > 0]
    kept = {c: set(top_p_clusters(s[c], live, top_p)) for c in range(qc.shape[0]) if int(q_size[c]) > 0}
    rows = []
    for c in q_block_cluster:
        c = int(c)
        if c < 0 or c not in kept:
            rows.append([])
            continue
        rows.append([k for k, kc_ in enumerate(k_block_cluster) if int(kc_) in kept[c]])
    return rows
