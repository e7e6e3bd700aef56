"""Wigner-D matrices and the alignment rotation (oracle, float64).

The E2Former-V2 write-up (stapisi.com, section 2.1) builds, per node, a
rotation that aligns the z axis with the node's vector r and rotates the
features with its Wigner-D matrix; section 5.2 asks that such rotations have
determinant 1 to within 1e-6.

Definitions used here:

* D^l(R) is the matrix with R_l(R r) = D^l(R) R_l(r) for every r, where R_l
  are the real solid harmonics of ``oracle.sh``.  Since the harmonics of
  degree l span a (2l+1)-dimensional space, D^l(R) is obtained exactly (up
  to rounding) by least squares from harmonics sampled at a few points.
* The alignment rotation of r = |r| (sin t cos p, sin t sin p, cos t) is
  Q = R_y(-t) R_z(-p), which maps r_hat to z_hat.  At r = 0 it is the
  identity, and on the z axis p = 0.
"""

from __future__ import annotations

import numpy as np

from .sh import solid_harmonic

# fixed, well-spread sample directions for the least-squares fit
_SAMPLES = np.random.default_rng(12345).standard_normal((32, 3))


def rot_z(a: float) -> np.ndarray:
    c, s = np.cos(a), np.sin(a)
    return np.array([[c, -s, 0.0], [s, c, 0.0], [0.0, 0.0, 1.0]])


def rot_y(a: float) -> np.ndarray:
    c, s = np.cos(a), np.sin(a)
    return np.array([[c, 0.0, s], [0.0, 1.0, 0.0], [-s, 0.0, c]])


def random_rotation(rng: np.random.Generator) -> np.ndarray:
    """A random proper rotation (QR of a Gaussian matrix, sign-fixed)."""
    A = rng.standard_normal((3, 3))
    Q, Rm = np.linalg.qr(A)
    Q = Q * np.sign(np.diag(Rm))
    if np.linalg.det(Q) < 0:
        Q[:, 0] = -Q[:, 0]
    return Q


def wigner_d(l: int, R: np.ndarray) -> np.ndarray:
    """D^l(R), [2l+1, 2l+1], defined by R_l(R r) = D^l(R) R_l(r)."""
    R = np.asarray(R, dtype=np.float64)
    Y = solid_harmonic(l, _SAMPLES)            # [n, 2l+1]
    YR = solid_harmonic(l, _SAMPLES @ R.T)     # [n, 2l+1]  rows: R_l(R r_k)
    # YR^T = D Y^T  ->  Y D^T = YR
    Dt, *_ = np.linalg.lstsq(Y, YR, rcond=None)
    return Dt.T


def wigner_d_full(lmax: int, R: np.ndarray) -> np.ndarray:
    """Block-diagonal D over all degrees 0..lmax: [(lmax+1)^2, (lmax+1)^2]."""
    S = (lmax + 1) ** 2
    D = np.zeros((S, S))
    for l in range(lmax + 1):
        sl = slice(l * l, (l + 1) ** 2)
        D[sl, sl] = wigner_d(l, R)
    return D


def alignment_rotation(r: np.ndarray) -> np.ndarray:
    """Q = R_y(-theta) R_z(-phi) with Q r_hat = z_hat (identity at r = 0)."""
    r = np.asarray(r, dtype=np.float64)
    rho = np.hypot(r[0], r[1])
    if rho == 0.0 and r[2] == 0.0:
        return np.eye(3)
    theta = np.arctan2(rho, r[2])
    phi = np.arctan2(r[1], r[0]) if rho > 0.0 else 0.0
    return rot_y(-theta) @ rot_z(-phi)
