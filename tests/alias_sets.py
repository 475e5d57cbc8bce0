"""Predicted alias sets of unguarded padded-row stores (host-side arithmetic).

A tile of ``tile_m`` rows that runs past the end of its row range still holds
``tile_m - (n % tile_m)`` padded rows.  If the epilogue stored them, the
addresses they would hit are fully determined by the output mapping; the
FlyDSL conv3d fp8 page ("Root cause", "Verification") predicts that set for
its fast path and checks that the clobbered offsets match it exactly.  The same
prediction for packed variable-length attention rows tells the bounds tests
which rows of which sequence an unguarded store would overwrite.
"""
import numpy as np


def conv_fast_path_alias(npq: int, tile_m: int, columns: int, dhw: int) -> np.ndarray:
    """Live output offsets hit by padded rows under off = col * dhw + row."""
    grid_m = -(-npq // tile_m)
    rows = np.arange(npq, grid_m * tile_m)
    off = (np.arange(columns)[:, None] * dhw + rows[None, :]).ravel()
    live = (off < columns * dhw) & ((off % dhw) < npq)
    return np.unique(off[live])


def packed_alias_rows(seqlens, tile_m: int):
    """For packed rows [cu[b], cu[b] + n_b) per sequence, the global rows that the
    padded rows of each sequence's last tile would hit: a list per sequence of
    (rows inside the tensor, number of rows past its end)."""
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    total = int(cu[-1])
    out = []
    for b, n in enumerate(seqlens):
        tiles = -(-int(n) // tile_m)
        pad = np.arange(cu[b] + n, cu[b] + tiles * tile_m)
        out.append((pad[pad < total], int((pad >= total).sum())))
    return out
