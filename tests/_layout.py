"""Expected per-rank blocks of a (mesh, placements) layout, from torch.chunk.

Rank l of the mesh (row-major coordinates c) holds, for every Shard(d) mesh
axis k, piece c[k] of torch.chunk(tensor, dims[k], dim=d); torch.chunk yields
ceil(D/m)-sized pieces and may yield fewer than m, in which case the missing
pieces are empty.
"""
from __future__ import annotations

import itertools

import numpy as np
import torch


def chunk_piece(a: np.ndarray, m: int, axis: int, c: int) -> np.ndarray:
    pieces = torch.chunk(torch.from_numpy(np.ascontiguousarray(a)), m, dim=axis)
    if c < len(pieces):
        return pieces[c].numpy()
    shape = list(a.shape)
    shape[axis] = 0
    return np.zeros(shape, a.dtype)


def local_blocks(G: np.ndarray, layout) -> list[np.ndarray]:
    dims, _start, pl = layout
    out = []
    for c in itertools.product(*[range(m) for m in dims]):
        blk = G
        for k, p in enumerate(pl):
            if p != "R":
                blk = chunk_piece(blk, dims[k], p[1], c[k])
        out.append(np.ascontiguousarray(blk).ravel())
    return out
