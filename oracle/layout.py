"""Where each token of a T x H x W grid lands after blocking (TEST INFRASTRUCTURE ONLY).

KPage paper, section 1: video latents have a T x H x W token organisation that
is flattened before attention and cut into 128-row logical blocks; boundary
blocks hold fewer valid rows.  Reading taken (the paper fixes no order):
4 x 4 x 8 tiles, blocks in raster order over (tile_t, tile_h, tile_w) with
tile_w fastest, tokens inside a tile in raster order over (t, h, w) with w
fastest, valid tokens at the start of their block's 128-row span.

This is written per token and does not use the generators' block counting, so a
test can check the two against each other.
"""
from __future__ import annotations

import numpy as np


def token_rows(T: int, H: int, W: int, tile=(4, 4, 8)) -> np.ndarray:
    """Physical row of every token, as an int64 array shaped [T, H, W]."""
    tt, th, tw = tile
    nbh, nbw = -(-H // th), -(-W // tw)
    rows = np.zeros((T, H, W), dtype=np.int64)
    for t in range(T):
        for h in range(H):
            for w in range(W):
                bt, bh, bw = t // tt, h // th, w // tw
                block = (bt * nbh + bh) * nbw + bw
                # extent of this token's tile along each axis (boundary tiles are cut short)
                et = min(tt, T - bt * tt)
                eh = min(th, H - bh * th)
                ew = min(tw, W - bw * tw)
                local = ((t - bt * tt) * eh + (h - bh * th)) * ew + (w - bw * tw)
                assert local < et * eh * ew
                rows[t, h, w] = 128 * block + local
    return rows
