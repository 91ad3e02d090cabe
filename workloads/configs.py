"""Seeded generators for the five block-sparse attention workloads.

Every workload is a flattened T x H x W video token grid cut into 4 x 4 x 8 tiles.
A tile becomes one 128-row logical block; a boundary tile keeps fewer valid rows
(KPage paper, section 1 and section 3.2.1: valid-row counts c_b in [0, 128]).
Valid rows are stored as a prefix of the block's 128-row span; rows past the
prefix are padding and are written as zeros (the paper zeroes unused page rows,
section 3.2.4).

Block order: blocks raster over (bt, bh, bw) with bw fastest.  Token order inside
a tile: (t, h, w) with w fastest.  These two orders are a reading of the word
"flattened" in the paper's introduction; the CPU oracle re-derives them on its
own when it checks block-sparse attention against dense attention.

Graphs (the sparse-selection step, which the paper keeps outside the method,
section 3.4):
  1  tiny 3D layout, 2 heads, d=64: diagonal plus Bernoulli(0.5) off-diagonal
     blocks, one mask shared by both heads;
  2  padding-free 16x32x32, 24 heads: 3D block window of radius (1,1,1);
  3  3D-padded 21x30x52, 40 heads: window radius (1,2,2) plus 4 distinct seeded
     random blocks outside the window per query block;
  4  21x45x80, 40 heads, Q/K carry a smooth per-block offset: per head, top-87
     key blocks by the dot product of mean-pooled valid query/key rows;
  5  same tokens, independent partitions: per head, k-means of Q tokens into 200
     clusters and K tokens into 600, tokens permuted cluster by cluster, clusters
     split into blocks of at most 128 rows, K/V blocks placed at 16-row-aligned
     offsets, and each Q cluster keeps the K clusters that cover 0.9 of the
     softmax mass of its centroid scores.

Seeds: workload i uses base seed 1000 + i.  Each head draws from generators
seeded by (base seed, batch, head, tensor), so generating a subset of heads
yields exactly the same data as the full problem restricted to those heads.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

TILE = (4, 4, 8)
BLOCK_ROWS = 128
PAGE_ROWS = 16

CONFIG_NAMES = {
    1: "tiny-3d-5x6x10-d64",
    2: "padding-free-16x32x32-h24",
    3: "3d-padded-21x30x52-h40",
    4: "vsa-top87-21x45x80-h40",
    5: "svg2-independent-21x45x80-h40",
}

_SPECS = {
    1: dict(T=5, H=6, W=10, heads=2, d=64),
    2: dict(T=16, H=32, W=32, heads=24, d=128),
    3: dict(T=21, H=30, W=52, heads=40, d=128),
    4: dict(T=21, H=45, W=80, heads=40, d=128),
    5: dict(T=21, H=45, W=80, heads=40, d=128),
}

_TENSOR_ID = {"q": 1, "k": 2, "v": 3, "do": 4}


def base_seed(cfg: int) -> int:
    return 1000 + cfg


@dataclass
class Workload:
    cfg: int
    name: str
    batch: int
    heads: int                 # heads present in the tensors
    head_dim: int
    n_q: int
    n_kv: int
    seq_q: int
    seq_kv: int
    per_head: bool
    q_valid: np.ndarray        # int32 [G, n_q]
    kv_valid: np.ndarray       # int32 [G, n_kv]
    kv_offset: np.ndarray      # int64 [G, n_kv]
    q2k_ptr: np.ndarray        # int64 [G, n_q + 1], absolute offsets into q2k_idx
    q2k_idx: np.ndarray        # int32 [nnz]
    q: torch.Tensor            # bf16 [B, H, seq_q, d]
    k: torch.Tensor            # bf16 [B, H, seq_kv, d]
    v: torch.Tensor            # bf16 [B, H, seq_kv, d]
    do: Optional[torch.Tensor] = None   # bf16 [B, H, seq_q, d]
    head_ids: List[int] = field(default_factory=list)
    layout: Optional[dict] = None
    # independent partitions only: per slot, the clustering the graph was selected from
    # (q_cent / k_cent fp32 [n_clusters, d], q_size / k_size tokens per cluster,
    # q_block_cluster [n_q] / k_block_cluster [n_kv] cluster of each block, -1 none)
    clusters: Optional[list] = None

    @property
    def n_slots(self) -> int:
        return self.q_valid.shape[0]

    def slot(self, b: int, h: int) -> int:
        return b * self.heads + h if self.per_head else 0

    def row(self, slot: int, q: int) -> np.ndarray:
        return self.q2k_idx[self.q2k_ptr[slot, q]:self.q2k_ptr[slot, q + 1]]

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# ----------------------------------------------------------------------------
# layout


def tile_layout(T: int, H: int, W: int, tile=TILE):
    """Blocks of a T x H x W grid cut into tiles: returns (grid, counts, coords)."""
    tt, th, tw = tile
    grid = (-(-T // tt), -(-H // th), -(-W // tw))
    counts, coords = [], []
    for bt in range(grid[0]):
        for bh in range(grid[1]):
            for bw in range(grid[2]):
                n = min(tt, T - tt * bt) * min(th, H - th * bh) * min(tw, W - tw * bw)
                counts.append(n)
                coords.append((bt, bh, bw))
    return grid, np.asarray(counts, dtype=np.int32), np.asarray(coords, dtype=np.int64)


def _csr(rows: Sequence[Sequence[int]]):
    ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    for i, r in enumerate(rows):
        ptr[i + 1] = ptr[i] + len(r)
    idx = np.concatenate([np.asarray(sorted(r), dtype=np.int32) for r in rows]) if ptr[-1] else \
        np.zeros(0, dtype=np.int32)
    return ptr, idx


def _window_rows(coords: np.ndarray, radius):
    r = np.asarray(radius)
    diff = np.abs(coords[:, None, :] - coords[None, :, :])
    inside = np.all(diff <= r[None, None, :], axis=2)
    return [list(np.nonzero(inside[qb])[0]) for qb in range(len(coords))], inside


# ----------------------------------------------------------------------------
# tensors


def _gen(cfg: int, b: int, h: int, name: str) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(((base_seed(cfg) * 1_000_003 + b) * 4099 + h) * 8 + _TENSOR_ID[name])
    return g


def _randn(cfg, b, h, name, rows, d) -> torch.Tensor:
    return torch.randn(rows, d, generator=_gen(cfg, b, h, name), dtype=torch.float32)


def _zero_padding_rows(x: torch.Tensor, starts, counts, span: int):
    keep = torch.zeros(x.shape[0], dtype=torch.bool)
    for s, c in zip(starts, counts):
        keep[int(s):int(s) + int(c)] = True
    x[~keep] = 0
    return x


def _smooth_offset(cfg: int, b: int, h: int, coords: np.ndarray, d: int) -> torch.Tensor:
    """Per-block offset: sum of 4 cosine waves over block coordinates along random unit directions."""
    rng = np.random.default_rng([base_seed(cfg), 7, b, h])
    u = rng.standard_normal((4, d))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    f = rng.uniform(0.5, 2.0, size=(4, 3))
    phi = rng.uniform(0.0, 2 * math.pi, size=4)
    pos = coords / np.array([6.0, 12.0, 10.0])
    waves = np.cos(2 * math.pi * pos @ f.T + phi[None, :])          # [n_blk, 4]
    off = waves @ u * (math.sqrt(d) / 2.0)                          # [n_blk, d]
    return torch.from_numpy(off.astype(np.float32))


# ----------------------------------------------------------------------------
# workload builders


def _shared_layout_tensors(cfg, spec, counts, head_ids, batch, with_do, offsets=None, coords=None):
    n = len(counts)
    S = BLOCK_ROWS * n
    d = spec["d"]
    starts = np.arange(n) * BLOCK_ROWS
    out = {nm: torch.empty(batch, len(head_ids), S, d, dtype=torch.bfloat16)
           for nm in (["q", "k", "v"] + (["do"] if with_do else []))}
    for b in range(batch):
        for hi, h in enumerate(head_ids):
            off_rows = None
            if offsets:
                off = _smooth_offset(cfg, b, h, coords, d)
                off_rows = off.repeat_interleave(BLOCK_ROWS, dim=0)
            for nm in out:
                x = _randn(cfg, b, h, nm, S, d)
                if off_rows is not None and nm in ("q", "k"):
                    x += off_rows
                out[nm][b, hi] = _zero_padding_rows(x, starts, counts, S).to(torch.bfloat16)
    return out


def _make_shared(cfg: int, head_ids, batch, with_do):
    spec = _SPECS[cfg]
    grid, counts, coords = tile_layout(spec["T"], spec["H"], spec["W"])
    n = len(counts)
    rng = np.random.default_rng(base_seed(cfg))
    if cfg == 1:
        keep = rng.random((n, n)) < 0.5
        np.fill_diagonal(keep, True)
        rows = [list(np.nonzero(keep[qb])[0]) for qb in range(n)]
    elif cfg == 2:
        rows, _ = _window_rows(coords, (1, 1, 1))
    elif cfg == 3:
        rows, inside = _window_rows(coords, (1, 2, 2))
        for qb in range(n):
            outside = np.nonzero(~inside[qb])[0]
            extra = rng.choice(outside, size=4, replace=False)
            rows[qb] = rows[qb] + [int(x) for x in extra]
    else:
        raise ValueError(cfg)
    ptr, idx = _csr(rows)
    t = _shared_layout_tensors(cfg, spec, counts, head_ids, batch, with_do)
    S = BLOCK_ROWS * n
    return Workload(
        cfg=cfg, name=CONFIG_NAMES[cfg], batch=batch, heads=len(head_ids), head_dim=spec["d"],
        n_q=n, n_kv=n, seq_q=S, seq_kv=S, per_head=False,
        q_valid=counts[None, :].copy(), kv_valid=counts[None, :].copy(),
        kv_offset=(np.arange(n, dtype=np.int64) * BLOCK_ROWS)[None, :],
        q2k_ptr=ptr[None, :], q2k_idx=idx, q=t["q"], k=t["k"], v=t["v"], do=t.get("do"),
        head_ids=list(head_ids), layout=dict(T=spec["T"], H=spec["H"], W=spec["W"], tile=TILE, grid=grid),
    )


def _make_topk(cfg: int, head_ids, batch, with_do, topk=87):
    spec = _SPECS[cfg]
    grid, counts, coords = tile_layout(spec["T"], spec["H"], spec["W"])
    n = len(counts)
    t = _shared_layout_tensors(cfg, spec, counts, head_ids, batch, with_do, offsets=True, coords=coords)
    G = batch * len(head_ids)
    ptrs, idxs, base = [], [], 0
    for b in range(batch):
        for hi in range(len(head_ids)):
            qm = _block_means(t["q"][b, hi], counts)
            km = _block_means(t["k"][b, hi], counts)
            score = qm @ km.T
            rows = []
            for qb in range(n):
                order = np.argsort(-score[qb], kind="stable")   # ties keep the lower block index first
                rows.append(sorted(int(x) for x in order[:topk]))
            p, i = _csr(rows)
            ptrs.append(p + base)
            idxs.append(i)
            base += len(i)
    return Workload(
        cfg=cfg, name=CONFIG_NAMES[cfg], batch=batch, heads=len(head_ids), head_dim=spec["d"],
        n_q=n, n_kv=n, seq_q=BLOCK_ROWS * n, seq_kv=BLOCK_ROWS * n, per_head=True,
        q_valid=np.tile(counts, (G, 1)), kv_valid=np.tile(counts, (G, 1)),
        kv_offset=np.tile(np.arange(n, dtype=np.int64) * BLOCK_ROWS, (G, 1)),
        q2k_ptr=np.stack(ptrs), q2k_idx=np.concatenate(idxs),
        q=t["q"], k=t["k"], v=t["v"], do=t.get("do"), head_ids=list(head_ids),
        layout=dict(T=spec["T"], H=spec["H"], W=spec["W"], tile=TILE, grid=grid),
    )


def _block_means(x: torch.Tensor, counts) -> np.ndarray:
    xs = x.to(torch.float64).numpy()
    out = np.zeros((len(counts), xs.shape[1]))
    for bi, c in enumerate(counts):
        if c:
            out[bi] = xs[bi * BLOCK_ROWS: bi * BLOCK_ROWS + c].mean(axis=0)
    return out


def _kmeans(x: torch.Tensor, k: int, iters: int, rng: np.random.Generator):
    """Lloyd's k-means (fp32) from k distinct random tokens; empty clusters keep their centre."""
    n = x.shape[0]
    cent = x[torch.from_numpy(rng.choice(n, size=k, replace=False))].clone()
    lab = None
    for _ in range(iters):
        dist = (cent * cent).sum(1)[None, :] - 2.0 * (x @ cent.T)
        lab = torch.argmin(dist, dim=1)
        sums = torch.zeros_like(cent).index_add_(0, lab, x)
        cnt = torch.bincount(lab, minlength=k)
        nz = cnt > 0
        cent[nz] = sums[nz] / cnt[nz, None].to(x.dtype)
    return lab.numpy(), cent.numpy(), torch.bincount(lab, minlength=k).numpy()


def _split_clusters(labels: np.ndarray, k: int):
    """Cluster-contiguous token order and blocks (<= 128 rows) per cluster."""
    perm = np.argsort(labels, kind="stable")
    sizes = np.bincount(labels, minlength=k)
    blocks, block_cluster, start = [], [], 0
    for ci in range(k):
        n = int(sizes[ci])
        while n > 0:
            c = min(BLOCK_ROWS, n)
            blocks.append((start, c))
            block_cluster.append(ci)
            start += c
            n -= c
    return perm, blocks, np.asarray(block_cluster, dtype=np.int64)


def _make_svg2(cfg: int, head_ids, batch, with_do, n_qc=200, n_kc=600, top_p=0.9, iters=10):
    spec = _SPECS[cfg]
    d = spec["d"]
    grid, counts, coords = tile_layout(spec["T"], spec["H"], spec["W"])
    n_blk = len(counts)
    S_base = BLOCK_ROWS * n_blk
    starts = np.arange(n_blk) * BLOCK_ROWS
    valid_rows = np.concatenate([np.arange(s, s + c) for s, c in zip(starts, counts)])
    per = []
    for b in range(batch):
        for h in head_ids:
            off = _smooth_offset(cfg, b, h, coords, d).repeat_interleave(BLOCK_ROWS, dim=0)
            qt = (_randn(cfg, b, h, "q", S_base, d) + off).to(torch.bfloat16)[valid_rows]
            kt = (_randn(cfg, b, h, "k", S_base, d) + off).to(torch.bfloat16)[valid_rows]
            vt = _randn(cfg, b, h, "v", S_base, d).to(torch.bfloat16)[valid_rows]
            rng = np.random.default_rng([base_seed(cfg), 11, b, h])
            lq, cq, nq_sz = _kmeans(qt.float(), n_qc, iters, rng)
            lk, ck, nk_sz = _kmeans(kt.float(), n_kc, iters, rng)
            pq, qblocks, qcl = _split_clusters(lq, n_qc)
            pk, kblocks, kcl = _split_clusters(lk, n_kc)
            # centroid scores over non-empty K clusters, softmax, keep the top-p prefix
            live_k = np.nonzero(nk_sz > 0)[0]
            sc = cq.astype(np.float64) @ ck[live_k].astype(np.float64).T / math.sqrt(d)
            keep = {}
            for ci in np.nonzero(nq_sz > 0)[0]:
                z = sc[ci] - sc[ci].max()
                p = np.exp(z) / np.exp(z).sum()
                order = np.argsort(-p, kind="stable")
                csum = np.cumsum(p[order])
                m = int(np.searchsorted(csum, top_p) + 1)
                keep[int(ci)] = set(int(x) for x in live_k[order[:min(m, len(order))]])
            kb_of_cluster: Dict[int, List[int]] = {}
            for kb, ci in enumerate(kcl):
                kb_of_cluster.setdefault(int(ci), []).append(kb)
            rows = []
            for qb, ci in enumerate(qcl):
                sel = []
                for kc in keep[int(ci)]:
                    sel.extend(kb_of_cluster.get(kc, []))
                rows.append(sorted(sel))
            kvalid = np.asarray([c for _, c in kblocks], dtype=np.int32)
            koff = np.zeros(len(kblocks), dtype=np.int64)
            acc = 0
            for i, c in enumerate(kvalid):
                koff[i] = acc
                acc += PAGE_ROWS * (-(-int(c) // PAGE_ROWS))
            per.append(dict(cq=cq, ck=ck, nq_sz=nq_sz, nk_sz=nk_sz, qcl=qcl, kcl=kcl,
                            qt=qt[pq], kt=kt[pk], vt=vt[pk], qblocks=qblocks, kblocks=kblocks,
                            qvalid=np.asarray([c for _, c in qblocks], dtype=np.int32),
                            kvalid=kvalid, koff=koff, kfoot=acc, rows=rows, b=b, h=h))
    n_q = max(len(p["qblocks"]) for p in per)
    n_kv = max(len(p["kblocks"]) for p in per)
    S_q = BLOCK_ROWS * n_q
    S_kv = max(p["kfoot"] for p in per)
    S_kv = max(PAGE_ROWS, S_kv)
    G = len(per)
    q_valid = np.zeros((G, n_q), dtype=np.int32)
    kv_valid = np.zeros((G, n_kv), dtype=np.int32)
    kv_offset = np.zeros((G, n_kv), dtype=np.int64)
    names = ["q", "k", "v"] + (["do"] if with_do else [])
    out = {nm: torch.zeros(batch, len(head_ids), (S_q if nm in ("q", "do") else S_kv), d,
                           dtype=torch.bfloat16) for nm in names}
    ptrs, idxs, base = [], [], 0
    clusters = []
    for g, p in enumerate(per):
        b, hi = g // len(head_ids), g % len(head_ids)
        nq, nk = len(p["qblocks"]), len(p["kblocks"])
        qbc = np.full(n_q, -1, dtype=np.int32)
        kbc = np.full(n_kv, -1, dtype=np.int32)
        qbc[:nq] = p["qcl"]
        kbc[:nk] = p["kcl"]
        clusters.append(dict(q_cent=np.asarray(p["cq"], dtype=np.float32), k_cent=np.asarray(p["ck"], dtype=np.float32),
                             q_size=np.asarray(p["nq_sz"], dtype=np.int32), k_size=np.asarray(p["nk_sz"], dtype=np.int32),
                             q_block_cluster=qbc, k_block_cluster=kbc))
        q_valid[g, :nq] = p["qvalid"]
        kv_valid[g, :nk] = p["kvalid"]
        kv_offset[g, :nk] = p["koff"]
        kv_offset[g, nk:] = p["kfoot"]
        for qb, (s, c) in enumerate(p["qblocks"]):
            out["q"][b, hi, BLOCK_ROWS * qb: BLOCK_ROWS * qb + c] = p["qt"][s:s + c]
        for kb, (s, c) in enumerate(p["kblocks"]):
            o = int(p["koff"][kb])
            out["k"][b, hi, o:o + c] = p["kt"][s:s + c]
            out["v"][b, hi, o:o + c] = p["vt"][s:s + c]
        if with_do:
            x = _randn(cfg, p["b"], p["h"], "do", S_q, d)
            out["do"][b, hi] = _zero_padding_rows(
                x, np.arange(n_q) * BLOCK_ROWS, q_valid[g], S_q).to(torch.bfloat16)
        rows = p["rows"] + [[] for _ in range(n_q - nq)]
        pp, ii = _csr(rows)
        ptrs.append(pp + base)
        idxs.append(ii)
        base += len(ii)
    return Workload(
        cfg=cfg, name=CONFIG_NAMES[cfg], batch=batch, heads=len(head_ids), head_dim=d,
        n_q=n_q, n_kv=n_kv, seq_q=S_q, seq_kv=S_kv, per_head=True,
        q_valid=q_valid, kv_valid=kv_valid, kv_offset=kv_offset,
        q2k_ptr=np.stack(ptrs), q2k_idx=np.concatenate(idxs),
        q=out["q"], k=out["k"], v=out["v"], do=out.get("do"), head_ids=list(head_ids),
        layout=dict(T=spec["T"], H=spec["H"], W=spec["W"], tile=TILE, grid=grid), clusters=clusters,
    )


def make_workload(cfg: int, heads: Optional[Sequence[int]] = None, batch: int = 1,
                  with_do: bool = False) -> Workload:
    """Build workload ``cfg`` (1..5) for the given head indices (default: all heads)."""
    spec = _SPECS[cfg]
    head_ids = list(range(spec["heads"])) if heads is None else [int(h) for h in heads]
    torch.set_num_threads(max(1, torch.get_num_threads()))
    if cfg in (1, 2, 3):
        return _make_shared(cfg, head_ids, batch, with_do)
    if cfg == 4:
        return _make_topk(cfg, head_ids, batch, with_do)
    if cfg == 5:
        return _make_svg2(cfg, head_ids, batch, with_do)
    raise ValueError(f"unknown workload {cfg}")
