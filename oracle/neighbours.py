"""Padded neighbour list by brute force (oracle, float64, test infrastructure).

The attention takes each target's neighbours as a padded index list plus mask
(E2Former-V2 write-up, section 3.2: padded slots are skipped; section 5.1:
the edge cutoff).  The pages do not spell the list out; the reading here,
which the GPU builder implements too, is:

* the neighbours of i are the atoms j != i with d2_ij < rc^2, where
  d2_ij = ((dx*dx + dy*dy) + dz*dz) in float64 with d_ = p_i - p_j formed
  from the float32 positions in float64, each operation rounded once (no
  fused multiply-add), and rc^2 = rc * rc in float64: a strict cutoff;
* a row lists them by increasing (d2, j): nearest first, equal distances
  by atom index;
* the first K are kept (valid slots first, mask 1); the rest of the row is
  index -1, mask 0;
* n_within_i counts all of them, before truncation.

Every pair is examined (O(N^2) in chunks): obviously correct, slow.
"""

from __future__ import annotations

from typing import Optional

import numpy as np


def pair_d2(pi: np.ndarray, pj: np.ndarray) -> np.ndarray:
    """d2 of every (i, j) pair of the two float32 position blocks, as defined above."""
    a = np.asarray(pi, dtype=np.float32).astype(np.float64)
    b = np.asarray(pj, dtype=np.float32).astype(np.float64)
    dx = a[:, None, 0] - b[None, :, 0]
    dy = a[:, None, 1] - b[None, :, 1]
    dz = a[:, None, 2] - b[None, :, 2]
    return (dx * dx + dy * dy) + dz * dz      # numpy rounds each product and sum once


def neighbour_list(pos: np.ndarray, cutoff: float, K: int, targets: Optional[np.ndarray] = None,
                   chunk: int = 256):
    """(idx [T, K] int32, mask [T, K] uint8, n_within [T] int64) for the given targets."""
    pos = np.asarray(pos, dtype=np.float32)
    n = pos.shape[0]
    tg = np.arange(n) if targets is None else np.asarray(targets, dtype=np.int64)
    rc2 = float(cutoff) * float(cutoff)
    idx = np.full((tg.size, K), -1, dtype=np.int32)
    mask = np.zeros((tg.size, K), dtype=np.uint8)
    n_within = np.zeros(tg.size, dtype=np.int64)
    js = np.arange(n, dtype=np.int64)
    for t0 in range(0, tg.size, chunk):
        rows = tg[t0:t0 + chunk]
        d2 = pair_d2(pos[rows], pos)                       # [r, n]
        ok = d2 < rc2
        ok[np.arange(rows.size), rows] = False             # j != i
        for r in range(rows.size):
            sel = np.nonzero(ok[r])[0]
            order = np.lexsort((js[sel], d2[r, sel]))      # by d2, then j
            sel = sel[order]
            n_within[t0 + r] = sel.size
            k = min(K, sel.size)
            idx[t0 + r, :k] = sel[:k]
            mask[t0 + r, :k] = 1
    return idx, mask, n_within
