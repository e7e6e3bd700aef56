"""Real solid harmonics R_l(r) = |r|^l C_l(r_hat), l = 0, 1, 2 (oracle, float64).

E2Former-V2 write-up (stapisi.com), section 2.3: the tensor product couples a
node feature h^(l_i) with a geometric encoding R^(l_f)(r); the gist.science
summary of arXiv 2601.16622 (technical summary 2.1, Lemma 4.1) calls these
solid spherical harmonics and states that, in a frame whose z axis lies along
r, only their m = 0 component is non-zero.

Reading (the pages fix no normalisation): Racah normalisation, so that
C_l0(z_hat) = 1 and sum_m C_lm(r_hat)^2 = 1; real components ordered
m = -l..l at flat index l^2 + l + m, with the usual real combinations of the
Condon-Shortley complex harmonics:

    l = 1 : (y, z, x)
    l = 2 : (sqrt3 xy, sqrt3 yz, (3z^2 - r^2)/2, sqrt3 xz, sqrt3/2 (x^2 - y^2))

Positions are used as given, in angstrom, without rescaling.
"""

from __future__ import annotations

import numpy as np

SQRT3 = np.sqrt(3.0)


def n_comp(lmax: int) -> int:
    """Number of irrep components S = (lmax + 1)^2."""
    return (lmax + 1) ** 2


def block(l: int) -> slice:
    """Slice of degree l in the flat component axis."""
    return slice(l * l, (l + 1) * (l + 1))


def solid_harmonic(l: int, r: np.ndarray) -> np.ndarray:
    """R_l(r) for r of shape [..., 3]; returns [..., 2l+1] in float64."""
    r = np.asarray(r, dtype=np.float64)
    x, y, z = r[..., 0], r[..., 1], r[..., 2]
    if l == 0:
        return np.ones(r.shape[:-1] + (1,))
    if l == 1:
        return np.stack([y, z, x], axis=-1)
    if l == 2:
        rr = x * x + y * y + z * z
        return np.stack([SQRT3 * x * y,
                         SQRT3 * y * z,
                         0.5 * (3.0 * z * z - rr),
                         SQRT3 * x * z,
                         0.5 * SQRT3 * (x * x - y * y)], axis=-1)
    raise ValueError(f"solid harmonics implemented for l <= 2, got {l}")


def solid_harmonics(lmax: int, r: np.ndarray) -> np.ndarray:
    """All R_l(r), l = 0..lmax, concatenated: [..., (lmax+1)^2]."""
    return np.concatenate([solid_harmonic(l, r) for l in range(lmax + 1)], axis=-1)
