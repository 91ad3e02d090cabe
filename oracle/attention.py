"""Plain-definition block-sparse attention in fp64 (TEST INFRASTRUCTURE ONLY).

KPage paper, section 3.2.4 (masking before the row maximum, eq. 3) and section
3.3.3 (the original sparse graph is restored exactly): the method computes
ordinary softmax attention restricted to the valid token pairs of the logical
block graph.  So the oracle is that definition written out, per (batch, head,
query block), with no paging, packing, tiling or online softmax:

  I  = valid rows of query block q: [128 q, 128 q + c_q)          (section 3.4.1)
  J  = concatenation over k in K_q of [o_k, o_k + c_k)            (section 3.4.1)
  S  = scale * Q[I] K[J]^T
  O[I]   = softmax(S) V[J],   LSE[I] = log sum_j exp(S_ij)
  rows outside I, and every row when J is empty: O = 0, LSE = -inf.

Backward is the gradient of sum(O * dO) with respect to Q, K and V under the
same definition (section 3.3), again per query block, accumulated into dK/dV.

Inputs are widened to fp64 exactly (bf16 -> fp64 is exact).
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -math.inf


def _f64(x) -> np.ndarray:
    """Widen a torch tensor or array to fp64 numpy."""
    if hasattr(x, "detach"):
        x = x.detach()
        if str(x.dtype) == "torch.bfloat16":
            x = x.float()
        x = x.cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def _slot(problem, b: int, h: int) -> int:
    return b * problem.heads + h if problem.per_head else 0


def _key_rows(problem, slot: int, q: int) -> np.ndarray:
    """Physical K/V rows of the valid tokens of every selected block, in selection order."""
    ks = problem.q2k_idx[problem.q2k_ptr[slot, q]:problem.q2k_ptr[slot, q + 1]]
    parts = [np.arange(problem.kv_offset[slot, k], problem.kv_offset[slot, k] + problem.kv_valid[slot, k])
             for k in ks]
    if not parts:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(parts).astype(np.int64)


def _query_rows(problem, slot: int, q: int) -> np.ndarray:
    c = int(problem.q_valid[slot, q])
    return np.arange(128 * q, 128 * q + c, dtype=np.int64)


def oracle_fwd_block(problem, Qh: np.ndarray, Kh: np.ndarray, Vh: np.ndarray, slot: int, q: int,
                     scale: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Forward for one query block of one head: returns (rows I, O[I], LSE[I])."""
    I = _query_rows(problem, slot, q)
    J = _key_rows(problem, slot, q)
    d = Qh.shape[1]
    if len(I) == 0:
        return I, np.zeros((0, d)), np.zeros(0)
    if len(J) == 0:
        return I, np.zeros((len(I), d)), np.full(len(I), NEG_INF)
    S = scale * (Qh[I] @ Kh[J].T)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    O = (E / l) @ Vh[J]
    lse = (m + np.log(l))[:, 0]
    return I, O, lse


def oracle_fwd(problem, q, k, v, scale: Optional[float] = None,
               items: Optional[Iterable[Tuple[int, int, int]]] = None):
    """Forward over all (b, h, q) or over the listed ``items``.

    Returns (O, LSE) as fp64 arrays shaped like the inputs ([B,H,Sq,d], [B,H,Sq]);
    rows that were not computed (when ``items`` is given) hold NaN.
    """
    scale = problem.scale if scale is None else scale
    Q, K, V = _f64(q), _f64(k), _f64(v)
    B, H, Sq, d = Q.shape
    O = np.zeros((B, H, Sq, d))
    L = np.full((B, H, Sq), NEG_INF)
    if items is None:
        todo = [(b, h, qb) for b in range(B) for h in range(H) for qb in range(problem.n_q)]
    else:
        O[:] = np.nan
        L[:] = np.nan
        todo = list(items)
    for b, h, qb in todo:
        rows = slice(128 * qb, 128 * qb + 128)
        if items is not None:
            O[b, h, rows] = 0.0
            L[b, h, rows] = NEG_INF
        I, Ob, Lb = oracle_fwd_block(problem, Q[b, h], K[b, h], V[b, h], _slot(problem, b, h), qb, scale)
        O[b, h, I] = Ob
        L[b, h, I] = Lb
    return O, L


def oracle_bwd(problem, q, k, v, do, scale: Optional[float] = None, heads: Optional[Sequence[int]] = None):
    """Gradients of sum(O * dO) w.r.t. Q, K, V in fp64, plus the oracle's own (O, LSE).

    Per query block (rows I, keys J, P the softmax probabilities):
      D  = rowsum(dO[I] * O[I])
      dV[J] += P^T dO[I];   dP = dO[I] V[J]^T;   dS = P * (dP - D)
      dQ[I] += scale dS K[J];   dK[J] += scale dS^T Q[I]
    ``heads`` restricts the computation to some head indices (others stay NaN).
    """
    scale = problem.scale if scale is None else scale
    Q, K, V, dO = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, Sq, d = Q.shape
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    O = np.zeros_like(Q)
    L = np.full((B, H, Sq), NEG_INF)
    hs = range(H) if heads is None else list(heads)
    if heads is not None:
        for arr in (dQ, dK, dV, O, L):
            arr[:] = np.nan
    for b in range(B):
        for h in hs:
            if heads is not None:
                for arr in (dQ, dK, dV, O):
                    arr[b, h] = 0.0
                L[b, h] = NEG_INF
            slot = _slot(problem, b, h)
            for qb in range(problem.n_q):
                I = _query_rows(problem, slot, qb)
                J = _key_rows(problem, slot, qb)
                if len(I) == 0 or len(J) == 0:
                    continue
                S = scale * (Q[b, h, I] @ K[b, h, J].T)
                m = S.max(axis=1, keepdims=True)
                E = np.exp(S - m)
                l = E.sum(axis=1, keepdims=True)
                P = E / l
                Ob = P @ V[b, h, J]
                O[b, h, I] = Ob
                L[b, h, I] = (m + np.log(l))[:, 0]
                Dv = (dO[b, h, I] * Ob).sum(axis=1, keepdims=True)
                dV[b, h, J] += P.T @ dO[b, h, I]
                dP = dO[b, h, I] @ V[b, h, J].T
                dS = P * (dP - Dv)
                dQ[b, h, I] += scale * (dS @ K[b, h, J])
                dK[b, h, J] += scale * (dS.T @ Q[b, h, I])
    return dQ, dK, dV, O, L


def brute_force_fwd(problem, q, k, v, scale: Optional[float] = None):
    """Pair-by-pair loops with math.exp (tiny inputs only): an independent check of ``oracle_fwd``."""
    scale = problem.scale if scale is None else scale
    Q, K, V = _f64(q), _f64(k), _f64(v)
    B, H, Sq, d = Q.shape
    O = np.zeros((B, H, Sq, d))
    L = np.full((B, H, Sq), NEG_INF)
    for b in range(B):
        for h in range(H):
            slot = _slot(problem, b, h)
            for qb in range(problem.n_q):
                cq = int(problem.q_valid[slot, qb])
                keys = []
                for kb in problem.q2k_idx[problem.q2k_ptr[slot, qb]:problem.q2k_ptr[slot, qb + 1]]:
                    o = int(problem.kv_offset[slot, kb])
                    for r in range(int(problem.kv_valid[slot, kb])):
                        keys.append(o + r)
                for i in range(128 * qb, 128 * qb + cq):
                    if not keys:
                        continue
                    s = [scale * sum(Q[b, h, i, c] * K[b, h, j, c] for c in range(d)) for j in keys]
                    mx = max(s)
                    w = [math.exp(x - mx) for x in s]
                    tot = sum(w)
                    for c in range(d):
                        O[b, h, i, c] = sum(w[t] * V[b, h, keys[t], c] for t in range(len(keys))) / tot
                    L[b, h, i] = mx + math.log(tot)
    return O, L
