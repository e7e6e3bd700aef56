"""Gradients of the attention output (oracle, float64, torch autograd on the CPU).

The "Conservative" E2Former-V2 variant (write-up section 4.2; gist.science
summary, section 4) takes forces as derivatives of an energy with respect to
positions, so the attention layer needs its vector-Jacobian product: for an
upstream gradient G = dL/d out, the gradients dL/dh and dL/dpos.

This module restates the forward definition of ``oracle.attn`` in torch
(float64, CPU) with the same coupling tensors (``oracle.cg``) and closed-form
harmonics, and lets autograd differentiate it.  It is pinned by central finite
differences of the numpy oracle (tests/test_oracle_grad.py).
"""

from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from .cg import real_cg
from .tp import paths

SQRT3 = 3.0 ** 0.5


def _harmonic(l: int, r: torch.Tensor) -> torch.Tensor:
    x, y, z = r[..., 0], r[..., 1], r[..., 2]
    if l == 0:
        return torch.ones(r.shape[:-1] + (1,), dtype=r.dtype)
    if l == 1:
        return torch.stack([y, z, x], dim=-1)
    rr = x * x + y * y + z * z
    return torch.stack([SQRT3 * x * y, SQRT3 * y * z, 0.5 * (3.0 * z * z - rr), SQRT3 * x * z,
                        0.5 * SQRT3 * (x * x - y * y)], dim=-1)


def tp_dense_torch(x: torch.Tensor, r: torch.Tensor, lmax: int,
                   path_w: Optional[np.ndarray] = None) -> torch.Tensor:
    """Same contraction as ``oracle.tp.tp_dense``, differentiable in x and r."""
    P = paths(lmax)
    w = np.ones(len(P)) if path_w is None else np.asarray(path_w, dtype=np.float64)
    blocks = [torch.zeros(x.shape[0], 2 * l + 1, x.shape[2], dtype=x.dtype) for l in range(lmax + 1)]
    for p, (li, lf, lo) in enumerate(P):
        if w[p] == 0.0:
            continue
        T = torch.from_numpy(real_cg(li, lf, lo))
        Y = _harmonic(lf, r)
        t = torch.einsum("ifo,nf->nio", T, Y)
        blocks[lo] = blocks[lo] + w[p] * torch.einsum("nio,nic->noc", t, x[:, li * li:(li + 1) ** 2])
    return torch.cat(blocks, dim=1)


def envelope_torch(x: torch.Tensor) -> torch.Tensor:
    """``oracle.attn.envelope`` in torch: 1 - 21 x^5 + 35 x^6 - 15 x^7 below 1, else 0,
    in the same factored form (1 - x)^3 (1 + 3x + 6x^2 + 10x^3 + 15x^4)."""
    y = 1.0 - x
    u = y ** 3 * (1.0 + x * (3.0 + x * (6.0 + x * (10.0 + 15.0 * x))))
    return torch.where(x < 1.0, u, torch.zeros_like(u))


def attn_forward_torch(pos: torch.Tensor, h: torch.Tensor, nbr_idx: np.ndarray, nbr_mask: np.ndarray,
                       heads: int, lmax: int, scale: Optional[float] = None,
                       path_w: Optional[np.ndarray] = None,
                       env_cutoff: Optional[float] = None, proj=None) -> torch.Tensor:
    """The three steps of ``oracle.attn.attn_forward`` for all targets, in torch.

    ``proj`` = (W_Q, W_K, W_V) torch tensors: the learned projections of
    ``oracle.attn.project`` (q = h[l=0] W_Q, k = h[l=0] W_K, v[l] = h[l] W_V[l], h' = v (x) R).
    """
    N, S, C = h.shape
    d = C // heads
    if scale is None:
        scale = 1.0 / d ** 0.5
    e_row, e_slot = np.nonzero(np.asarray(nbr_mask) != 0)
    e_src = np.asarray(nbr_idx)[e_row, e_slot].astype(np.int64)
    er = torch.from_numpy(e_row)
    es = torch.from_numpy(e_src)
    if proj is None:
        v, q0, k0 = h, h[:, 0, :], h[:, 0, :]
    else:
        w_q, w_k, w_v = proj
        q0, k0 = h[:, 0, :] @ w_q, h[:, 0, :] @ w_k
        v = torch.cat([h[:, l * l:(l + 1) ** 2, :] @ w_v[l] for l in range(lmax + 1)], dim=1)
    hp = tp_dense_torch(v, pos, lmax, path_w)                      # step 1
    q = q0.reshape(N, heads, d)
    k = k0.reshape(N, heads, d)
    s = scale * (q[er] * k[es]).sum(-1)                            # [E, H]
    mx_np = np.full((N, heads), -np.inf)
    np.maximum.at(mx_np, e_row, s.detach().numpy())
    mx = torch.from_numpy(np.where(np.isfinite(mx_np), mx_np, 0.0))  # stabiliser, no gradient
    p = torch.exp(s - mx[er])
    if env_cutoff is not None:
        dist = torch.linalg.vector_norm(pos[er] - pos[es], dim=-1)
        p = p * envelope_torch(dist / float(env_cutoff))[:, None]
    z = torch.zeros((N, heads), dtype=h.dtype).index_add(0, er, p)
    zr = z[er]
    alpha = p / torch.where(zr > 0, zr, torch.ones_like(zr))
    a = alpha.repeat_interleave(d, dim=1)                          # channel c -> head c // d
    msg = torch.zeros((N, S, C), dtype=h.dtype).index_add(0, er, a[:, None, :] * hp[es])
    return tp_dense_torch(msg, pos, lmax, path_w)                  # step 3


def attn_backward(pos: np.ndarray, h: np.ndarray, nbr_idx: np.ndarray, nbr_mask: np.ndarray,
                  heads: int, lmax: int, grad_out: np.ndarray, scale: Optional[float] = None,
                  path_w: Optional[np.ndarray] = None, env_cutoff: Optional[float] = None):
    """(dL/dh [N,S,C], dL/dpos [N,3]) for L = <grad_out, out>, float64."""
    pt = torch.tensor(np.asarray(pos, dtype=np.float64), requires_grad=True)
    ht = torch.tensor(np.asarray(h, dtype=np.float64), requires_grad=True)
    out = attn_forward_torch(pt, ht, nbr_idx, nbr_mask, heads, lmax, scale, path_w, env_cutoff)
    g = torch.from_numpy(np.asarray(grad_out, dtype=np.float64))
    dh, dpos = torch.autograd.grad((out * g).sum(), (ht, pt), allow_unused=True)
    if dpos is None:            # lmax = 0: the harmonics are constant, positions do not enter
        dpos = torch.zeros_like(pt)
    return dh.numpy(), dpos.numpy()


def attn_backward_proj(pos: np.ndarray, h: np.ndarray, nbr_idx: np.ndarray, nbr_mask: np.ndarray,
                       heads: int, lmax: int, grad_out: np.ndarray, proj, scale: Optional[float] = None,
                       path_w: Optional[np.ndarray] = None, env_cutoff: Optional[float] = None):
    """(dL/dh, dL/dpos, dL/dW_Q, dL/dW_K, dL/dW_V) of the projected layer, float64."""
    pt = torch.tensor(np.asarray(pos, dtype=np.float64), requires_grad=True)
    ht = torch.tensor(np.asarray(h, dtype=np.float64), requires_grad=True)
    ws = [torch.tensor(np.asarray(w, dtype=np.float64), requires_grad=True) for w in proj]
    out = attn_forward_torch(pt, ht, nbr_idx, nbr_mask, heads, lmax, scale, path_w, env_cutoff,
                             proj=tuple(ws))
    g = torch.from_numpy(np.asarray(grad_out, dtype=np.float64))
    grads = torch.autograd.grad((out * g).sum(), (ht, pt, *ws), allow_unused=True)
    grads = [torch.zeros_like(t) if d is None else d for d, t in zip(grads, (ht, pt, *ws))]
    return tuple(d.numpy() for d in grads)


def eaas_vjp(x: np.ndarray, r: np.ndarray, g: np.ndarray, lmax: int,
             path_w: Optional[np.ndarray] = None):
    """(dL/dx, dL/dr) of L = <g, x (x) R(r)> for the channel-wise coupling alone."""
    xt = torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)
    rt = torch.tensor(np.asarray(r, dtype=np.float64), requires_grad=True)
    y = tp_dense_torch(xt, rt, lmax, path_w)
    dx, dr = torch.autograd.grad((y * torch.from_numpy(np.asarray(g, dtype=np.float64))).sum(),
                                 (xt, rt), allow_unused=True)
    if dr is None:
        dr = torch.zeros_like(rt)
    return dx.numpy(), dr.numpy()
