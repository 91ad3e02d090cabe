"""Small hand-built block-sparse problems for the CPU tests (inputs only, no method arithmetic)."""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
import torch


@dataclass
class Problem:
    batch: int
    heads: int
    head_dim: int
    n_q: int
    n_kv: int
    seq_q: int
    seq_kv: int
    per_head: bool
    q_valid: np.ndarray
    kv_valid: np.ndarray
    kv_offset: np.ndarray
    q2k_ptr: np.ndarray
    q2k_idx: np.ndarray

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def slot(self, b, h):
        return b * self.heads + h if self.per_head else 0

    def row(self, slot, q):
        return self.q2k_idx[self.q2k_ptr[slot, q]:self.q2k_ptr[slot, q + 1]]


def make_problem(q_valid: Sequence, kv_valid: Sequence, rows: Sequence[Sequence[int]], heads=1, batch=1,
                 head_dim=16, kv_offset: Optional[Sequence[int]] = None, seq_kv: Optional[int] = None,
                 sort_rows=True) -> Problem:
    """One graph slot shared by every head."""
    q_valid = np.asarray(q_valid, dtype=np.int32)[None, :]
    kv_valid = np.asarray(kv_valid, dtype=np.int32)[None, :]
    n_q, n_kv = q_valid.shape[1], kv_valid.shape[1]
    if kv_offset is None:
        kv_offset = np.arange(n_kv, dtype=np.int64) * 128
    kv_offset = np.asarray(kv_offset, dtype=np.int64)[None, :]
    if seq_kv is None:
        seq_kv = int(max(128 * n_kv, (kv_offset + 16 * ((kv_valid + 15) // 16)).max()))
    ptr = np.zeros((1, n_q + 1), dtype=np.int64)
    idx: List[int] = []
    for q, r in enumerate(rows):
        r = sorted(r) if sort_rows else list(r)
        idx.extend(r)
        ptr[0, q + 1] = len(idx)
    return Problem(batch=batch, heads=heads, head_dim=head_dim, n_q=n_q, n_kv=n_kv, seq_q=128 * n_q,
                   seq_kv=seq_kv, per_head=False, q_valid=q_valid, kv_valid=kv_valid, kv_offset=kv_offset,
                   q2k_ptr=ptr, q2k_idx=np.asarray(idx, dtype=np.int32))


def random_tensors(p: Problem, seed=0, zero_padding=True, garbage=None):
    """bf16 Q, K, V, dO; padded rows zero, or filled with finite garbage of the given magnitude."""
    g = torch.Generator().manual_seed(seed)
    d = p.head_dim
    shapes = dict(q=p.seq_q, k=p.seq_kv, v=p.seq_kv, do=p.seq_q)
    out = {n: torch.randn(p.batch, p.heads, s, d, generator=g).to(torch.bfloat16) for n, s in shapes.items()}
    if zero_padding or garbage is not None:
        for b in range(p.batch):
            for h in range(p.heads):
                s = p.slot(b, h)
                qkeep = torch.zeros(p.seq_q, dtype=torch.bool)
                for qb in range(p.n_q):
                    qkeep[128 * qb:128 * qb + int(p.q_valid[s, qb])] = True
                kkeep = torch.zeros(p.seq_kv, dtype=torch.bool)
                for kb in range(p.n_kv):
                    o = int(p.kv_offset[s, kb])
                    kkeep[o:o + int(p.kv_valid[s, kb])] = True
                for n, keep in (("q", qkeep), ("do", qkeep), ("k", kkeep), ("v", kkeep)):
                    x = out[n][b, h]
                    if garbage is None:
                        x[~keep] = 0
                    else:
                        x[~keep] = (garbage * torch.randn(int((~keep).sum()), d, generator=g)).to(torch.bfloat16)
    return out
