"""Shared test helpers: the parity metric and host-side array conversions."""

from __future__ import annotations

import numpy as np

TOL_F32 = 1e-4   # max block-relative error, fp32 storage
TOL_BF16 = 2e-2  # max block-relative error, bf16 storage with fp32 accumulation


def block_rel_err(got: np.ndarray, ref: np.ndarray, lmax: int) -> float:
    """max over (atom, degree block) of max|got - ref| / max|ref| within the block.

    Blocks are normalised separately because degree l scales like |r|^l.
    0/0 counts as 0; a non-zero result where the reference block is all zero
    counts as infinite.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    worst = 0.0
    for l in range(lmax + 1):
        sl = slice(l * l, (l + 1) ** 2)
        num = np.abs(got[:, sl] - ref[:, sl]).max(axis=(1, 2))
        den = np.abs(ref[:, sl]).max(axis=(1, 2))
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
        if not np.isfinite(got[:, sl]).all():
            return float("inf")
        worst = max(worst, float(r.max()))
    return worst


HEAD_FLOOR = 1e-3   # a head's scale never counts below this share of its block's scale


def head_rel_err(got: np.ndarray, ref: np.ndarray, lmax: int, heads: int) -> float:
    """max over (atom, degree block, head) of max|got - ref| / max|ref| within that head's
    channels of the block, the denominator floored at HEAD_FLOOR times the block's max|ref|.

    Stricter than block_rel_err: a head whose values are small next to the rest of its block
    is measured against its own scale (down to the floor), not the block's.  0/0 counts as 0.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    if not np.isfinite(got).all():
        return float("inf")
    n, S, C = ref.shape
    d = C // heads
    worst = 0.0
    for l in range(lmax + 1):
        sl = slice(l * l, (l + 1) ** 2)
        dg = np.abs(got[:, sl] - ref[:, sl]).reshape(n, -1, heads, d)   # [n, 2l+1, H, d]
        rr = np.abs(ref[:, sl]).reshape(n, -1, heads, d)
        num = dg.max(axis=(1, 3))                                        # [n, H]
        block = rr.max(axis=(1, 2, 3))[:, None]                          # [n, 1]
        den = np.maximum(rr.max(axis=(1, 3)), HEAD_FLOOR * block)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
        worst = max(worst, float(r.max()))
    return worst


def to_host(t) -> np.ndarray:
    """A torch tensor (fp32 or bf16, any device) as float64 numpy."""
    import torch
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)
