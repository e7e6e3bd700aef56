"""Channel-wise tensor product h (x) R(r) and the reference EAAS (oracle, float64).

Definition followed (E2Former-V2 write-up, stapisi.com, sections 2.3 and 3.1):
a node feature h, one irrep block h^(l_i) per degree, is coupled with the
solid harmonics R^(l_f)(r) of a vector r into output degree l_o.  Readings,
since the pages print no weights or path list:

* the paths are every (l_i, l_f, l_o) with all three <= lmax that obey the
  triangle rule |l_i - l_f| <= l_o <= l_i + l_f, in lexicographic order
  (5 paths at lmax = 1, 15 at lmax = 2);
* coupling is channel-wise (no mixing between channels) with one weight per
  path (default 1), and all paths that reach the same l_o are summed;
* output degrees are truncated to l_o <= lmax, so h and the result have the
  same shape [n, (lmax+1)^2, C].

``tp_dense`` is the definition: a dense contraction with the real coupling
tensors of ``oracle.cg``.  It produces every graded oracle output.

``eaas_reference`` is a second, independent route used only to check
Proposition 4.3 (write-up section 2.3; gist.science summary, technical
summary 2.1): rotate h into the frame whose z axis lies along r, apply the
sparse reindex of section 2.2 (l_i + l_f + l_o even: keep m_i = m_o; odd:
keep m_i = -m_o with a sign), then rotate back.  In the aligned frame the
harmonics reduce to |r|^l_f at m_f = 0 (Lemma 4.1), so the reindex weights
are the Condon-Shortley coefficients <l_i m l_f 0 | l_o m>; the sign of the
odd case follows from the real-basis phase of ``oracle.cg``: for m >= 1,
y[l_o, +m] gets +c_m h[l_i, -m] and y[l_o, -m] gets -c_m h[l_i, +m], and
y[l_o, 0] gets nothing.
"""

from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np

from .cg import cg_coefficient, real_cg
from .sh import block, n_comp, solid_harmonic
from .wigner import alignment_rotation, wigner_d_full

Path = Tuple[int, int, int]


def paths(lmax: int) -> List[Path]:
    """Triangle-allowed (l_i, l_f, l_o), each <= lmax, lexicographic."""
    out = []
    for li in range(lmax + 1):
        for lf in range(lmax + 1):
            for lo in range(lmax + 1):
                if abs(li - lf) <= lo <= li + lf:
                    out.append((li, lf, lo))
    return out


def _weights(lmax: int, path_w: Optional[np.ndarray]) -> np.ndarray:
    P = len(paths(lmax))
    if path_w is None:
        return np.ones(P)
    w = np.asarray(path_w, dtype=np.float64).reshape(-1)
    if w.shape[0] != P:
        raise ValueError(f"path_w needs {P} entries at lmax={lmax}")
    return w


def tp_dense(x: np.ndarray, r: np.ndarray, lmax: int,
             path_w: Optional[np.ndarray] = None) -> np.ndarray:
    """sum_p w_p CG_p(x[l_i], R_{l_f}(r)) into block l_o; x [n,S,C], r [n,3] -> [n,S,C]."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    n, S, C = x.shape
    if S != n_comp(lmax):
        raise ValueError("component axis does not match lmax")
    w = _weights(lmax, path_w)
    out = np.zeros((n, S, C))
    for p, (li, lf, lo) in enumerate(paths(lmax)):
        if w[p] == 0.0:
            continue
        Y = solid_harmonic(lf, r)                                # [n, 2lf+1]
        T = real_cg(li, lf, lo)                                  # [2li+1, 2lf+1, 2lo+1]
        t = np.einsum("ifo,nf->nio", T, Y)                       # [n, 2li+1, 2lo+1]
        out[:, block(lo), :] += w[p] * np.einsum("nio,nic->noc", t, x[:, block(li), :])
    return out


def sparse_rule(lmax: int):
    """Nonzeros of the aligned-frame reindex: (path, l_o, m_o, l_i, m_i, coefficient).

    The coefficient excludes the |r|^l_f factor and the path weight.
    """
    entries = []
    for p, (li, lf, lo) in enumerate(paths(lmax)):
        even = (li + lf + lo) % 2 == 0
        for m in range(0, min(li, lo) + 1):
            c = cg_coefficient(li, m, lf, 0, lo, m)
            if c == 0.0:
                continue
            if even:
                entries.append((p, lo, m, li, m, c))
                if m > 0:
                    entries.append((p, lo, -m, li, -m, c))
            elif m > 0:
                entries.append((p, lo, m, li, -m, c))
                entries.append((p, lo, -m, li, m, -c))
    return entries


def eaas_reference(x: np.ndarray, r: np.ndarray, lmax: int,
                   path_w: Optional[np.ndarray] = None) -> np.ndarray:
    """Rotate into the r-aligned frame, sparse reindex, rotate back (per atom loop)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    n, S, C = x.shape
    w = _weights(lmax, path_w)
    rule = sparse_rule(lmax)
    out = np.zeros((n, S, C))
    for a in range(n):
        Q = alignment_rotation(r[a])
        D = wigner_d_full(lmax, Q)
        xt = D @ x[a]                                   # features in the aligned frame
        rn = float(np.linalg.norm(r[a]))
        yt = np.zeros((S, C))
        for p, lo, mo, li, mi, c in rule:
            lf = paths(lmax)[p][1]
            yt[lo * lo + lo + mo] += w[p] * c * rn ** lf * xt[li * li + li + mi]
        out[a] = D.T @ yt                               # back to the global frame
    return out
