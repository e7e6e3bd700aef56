"""Node-centric equivariant attention with every edge materialised (oracle, float64).

Follows the three steps of the E2Former-V2 write-up (stapisi.com, section 3.1)
and the attention description of the gist.science summary of arXiv 2601.16622
(technical summary 2.2):

1. source pre-coupling  h'_j = h_j (x) R(r_j)                     (tp_dense)
2. aggregation           m_i = sum_j alpha_ij h'_j over the neighbours j of i
3. target coupling       out_i = m_i (x) R(r_i)                     (tp_dense)

Only the values carry direction; the logits use SO(3)-invariant scalars.
Readings of what the pages leave open:

* q_i = h_i[l=0, :], k_j = h_j[l=0, :] (the input features, no learned
  projection); head h owns channels [h d, (h+1) d) with d = C / H for Q, K
  and V; the logit is scale * <q_i, k_j> over the head's channels, with
  scale = 1/sqrt(d) unless given.
* V = h'_j, so alpha_ijh weights all (lmax+1)^2 components of head h's
  channels.
* the softmax runs over the valid (mask = 1) slots of row i only; the fused
  kernel's online softmax (write-up section 3.2; gist.science summary 2.2)
  equals this plain softmax up to rounding.  A row with no valid slot gives
  m_i = 0 and out_i = 0.  Repeated indices count once per slot.
* r_j, r_i are the atoms' own position vectors as passed.

Optional learned projections (``project``).  The gist.science summary (2.2,
Eq. 6) builds Q and K with SO(3)-invariant scalar projections; the equation
itself is not printed.  Reading: q_i = h_i[l=0] W_Q and k_j = h_j[l=0] W_K
with W_Q, W_K [C, C] acting on the channel axis from the right.  For the
values the pages print no projection; the reading is per-degree channel
mixing v_j[l] = h_j[l] W_V[l] (W_V [lmax+1, C, C]), the most general linear
map of irrep features that commutes with rotations (Schur's lemma), applied
before the pre-coupling: h'_j = v_j (x) R(r_j).

Optional smooth envelope (``env_cutoff``).  The EquiformerV3 page (method
details, attention) multiplies the softmax numerator and denominator by an
envelope e(|r_ij|) of the pair distance so that the weights fade out smoothly
at the cutoff; it prints no formula for e.  Reading: the weights become

    alpha_ijh = e_ij exp(s_ijh) / sum_k e_ik exp(s_ikh),
    e_ij = u(|r_i - r_j| / r_env),  u(x) = 1 - 21 x^5 + 35 x^6 - 15 x^7 (x < 1), 0 (x >= 1),

the polynomial smooth cutoff with u(0) = 1 and u = u' = u'' = 0 at x = 1
(so the weights, and forces derived from them, stay continuous as a
neighbour crosses r_env).  A slot with e_ij = 0 contributes nothing; a row
whose every valid slot has e = 0 gives m_i = 0 like an empty row.  The
distance is taken in float64 from the float32 positions.

This function materialises logits [E, H] and messages [E, S, C]: it is the
edge-centric form the pages contrast the fused kernel with.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .sh import n_comp
from .tp import tp_dense


def project(h: np.ndarray, w_q: np.ndarray, w_k: np.ndarray, w_v: np.ndarray):
    """(q [N, C], k [N, C], v [N, S, C]) of the learned projections (reading in the header)."""
    h = np.asarray(h, dtype=np.float64)
    N, S, C = h.shape
    lmax = int(round(S ** 0.5)) - 1
    w_v = np.asarray(w_v, dtype=np.float64)
    if w_v.shape != (lmax + 1, C, C):
        raise ValueError("w_v must be [lmax + 1, C, C]")
    q = h[:, 0, :] @ np.asarray(w_q, dtype=np.float64)
    k = h[:, 0, :] @ np.asarray(w_k, dtype=np.float64)
    v = np.empty_like(h)
    for l in range(lmax + 1):
        v[:, l * l:(l + 1) ** 2, :] = h[:, l * l:(l + 1) ** 2, :] @ w_v[l]
    return q, k, v


def envelope(x: np.ndarray) -> np.ndarray:
    """u(x) = 1 - 21 x^5 + 35 x^6 - 15 x^7 for 0 <= x < 1, 0 for x >= 1 (reading in the header).

    Evaluated as (1 - x)^3 (1 + 3x + 6x^2 + 10x^3 + 15x^4), the same polynomial.  Its
    factors are positive on [0, 1), so u keeps its relative precision up to the cutoff;
    the expanded sum cancels there (within 1e-5 of x = 1 no digit of it is left in
    float64), and weights and gradients of pairs near the cutoff are relative to u.
    """
    x = np.asarray(x, dtype=np.float64)
    y = 1.0 - x
    u = y ** 3 * (1.0 + x * (3.0 + x * (6.0 + x * (10.0 + 15.0 * x))))
    return np.where(x < 1.0, u, 0.0)


def pair_distance(pos: np.ndarray, i: np.ndarray, j: np.ndarray) -> np.ndarray:
    """|r_i - r_j| in float64 from the positions as given."""
    p = np.asarray(pos, dtype=np.float64)
    return np.linalg.norm(p[np.asarray(i)] - p[np.asarray(j)], axis=-1)


def attention_weights(h: np.ndarray, nbr_idx: np.ndarray, nbr_mask: np.ndarray, heads: int,
                      scale: Optional[float] = None, targets: Optional[np.ndarray] = None,
                      qk: Optional[tuple] = None, env: Optional[tuple] = None):
    """Edge list and softmax weights: (e_row, e_src, alpha [E, H]).

    e_row indexes the target list, e_src the source atom of each valid slot.
    ``qk`` = (q [N, C], k [N, C]) replaces the default q = k = h[:, l=0, :].
    ``env`` = (pos [N, 3], r_env) multiplies each pair's exp(logit) by the
    envelope of its distance, numerator and denominator alike.
    """
    h = np.asarray(h, dtype=np.float64)
    N, _, C = h.shape
    if C % heads != 0:
        raise ValueError("channels must divide into heads")
    d = C // heads
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    tgt = np.arange(N) if targets is None else np.asarray(targets, dtype=np.int64)
    T = tgt.shape[0]

    # edge list (target row t, source j) from the mask; masked slots are never read
    mask = np.asarray(nbr_mask)[tgt] != 0
    idx = np.asarray(nbr_idx)[tgt]
    e_row, e_slot = np.nonzero(mask)
    e_src = idx[e_row, e_slot].astype(np.int64)
    if e_src.size and (e_src.min() < 0 or e_src.max() >= N):
        raise IndexError("a valid neighbour slot holds an out-of-range index")
    E = e_src.shape[0]

    # invariant per-head logits [E, H]
    qa, ka = (h[:, 0, :], h[:, 0, :]) if qk is None else (np.asarray(qk[0], dtype=np.float64),
                                                         np.asarray(qk[1], dtype=np.float64))
    q = qa[tgt].reshape(T, heads, d)
    k = ka[e_src].reshape(E, heads, d)
    logits = scale * np.einsum("ehc,ehc->eh", q[e_row], k)

    # softmax per (target, head) over that target's valid slots
    mx = np.full((T, heads), -np.inf)
    np.maximum.at(mx, e_row, logits)
    p = np.exp(logits - mx[e_row])
    if env is not None:
        pos, r_env = env
        p = p * envelope(pair_distance(pos, tgt[e_row], e_src) / float(r_env))[:, None]
    z = np.zeros((T, heads))
    np.add.at(z, e_row, p)
    zr = z[e_row]
    return e_row, e_src, np.divide(p, zr, out=np.zeros_like(p), where=zr > 0)


def attn_forward(pos: np.ndarray, h: np.ndarray, nbr_idx: np.ndarray, nbr_mask: np.ndarray,
                 heads: int, lmax: int, scale: Optional[float] = None,
                 path_w: Optional[np.ndarray] = None, targets: Optional[np.ndarray] = None,
                 return_msg: bool = False, chunk_edges: int = 1 << 16,
                 proj: Optional[tuple] = None, env_cutoff: Optional[float] = None):
    """Output [T, S, C] for the given targets (all atoms if None); optionally also m [T, S, C].

    ``proj`` = (W_Q, W_K, W_V) switches on the learned projections (see ``project``);
    ``env_cutoff`` = r_env switches on the smooth envelope (see ``envelope``).
    """
    pos = np.asarray(pos, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    N, S, C = h.shape
    if S != n_comp(lmax):
        raise ValueError("component axis does not match lmax")
    d = C // heads
    tgt = np.arange(N) if targets is None else np.asarray(targets, dtype=np.int64)
    T = tgt.shape[0]

    if proj is None:
        qk, v = None, h
    else:
        q, k, v = project(h, *proj)
        qk = (q, k)
    env = None if env_cutoff is None else (pos, env_cutoff)
    e_row, e_src, alpha = attention_weights(h, nbr_idx, nbr_mask, heads, scale, tgt, qk, env)
    E = e_src.shape[0]

    # step 1 on every source that some edge reads
    src, src_inv = np.unique(e_src, return_inverse=True)
    hp_src = tp_dense(v[src], pos[src], lmax, path_w)           # [n_src, S, C]

    # messages alpha_ijh * h'_j, materialised in chunks, summed into m_i
    msg = np.zeros((T, S, C))
    for e0 in range(0, E, chunk_edges):
        e1 = min(E, e0 + chunk_edges)
        a = np.repeat(alpha[e0:e1], d, axis=1)                  # [e, C], channel c -> head c // d
        m_e = a[:, None, :] * hp_src[src_inv[e0:e1]]            # [e, S, C]
        np.add.at(msg, e_row[e0:e1], m_e)

    # step 3 with the target's own harmonics
    out = tp_dense(msg, pos[tgt], lmax, path_w)
    if return_msg:
        return out, msg
    return out
