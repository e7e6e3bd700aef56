"""Clebsch-Gordan coefficients and real-basis coupling tensors (oracle, float64).

The dense SO(3) tensor product that EAAS replaces is a contraction with
Clebsch-Gordan coefficients (gist.science summary of arXiv 2601.16622,
technical summary 2.1; EquiformerV3 page on paper.rainbus.top, background on
irreps and CG products).  The write-up (stapisi.com, section 5.2) warns that
the CG normalisation matters.  Readings used here, none of which the pages fix:

* Condon-Shortley coefficients <l1 m1 l2 m2 | L M> from Racah's closed
  formula (orthonormal: sum over m1, m2 of the squares is 1 for each M).
* Real components x relate to spherical components T by
  T_0 = x_0,  T_{+m} = (-1)^m (x_m + i x_{-m}) / sqrt2,
  T_{-m} = (x_m - i x_{-m}) / sqrt2   (m > 0),
  which matches the real harmonics of ``oracle.sh``.
* The real coupling tensor of a path (l_i, l_f, l_o) is the spherical one
  transformed by these maps; it is real when l_i + l_f + l_o is even and
  purely imaginary when it is odd, in which case it is multiplied by -i.
* Factor order is feature (x) harmonic: index order [m_i, m_f, m_o].
"""

from __future__ import annotations

import functools
from math import factorial, sqrt

import numpy as np


def cg_coefficient(j1: int, m1: int, j2: int, m2: int, J: int, M: int) -> float:
    """<j1 m1 j2 m2 | J M> (Condon-Shortley) from Racah's formula, integer spins."""
    if M != m1 + m2:
        return 0.0
    if not (abs(j1 - j2) <= J <= j1 + j2):
        return 0.0
    if abs(m1) > j1 or abs(m2) > j2 or abs(M) > J:
        return 0.0
    pre = sqrt((2 * J + 1) * factorial(J + j1 - j2) * factorial(J - j1 + j2)
               * factorial(j1 + j2 - J) / factorial(j1 + j2 + J + 1))
    pre *= sqrt(factorial(J + M) * factorial(J - M) * factorial(j1 - m1) * factorial(j1 + m1)
                * factorial(j2 - m2) * factorial(j2 + m2))
    total = 0.0
    for k in range(0, j1 + j2 + J + 1):
        args = (k, j1 + j2 - J - k, j1 - m1 - k, j2 + m2 - k, J - j2 + m1 + k, J - j1 - m2 + k)
        if min(args) < 0:
            continue
        den = 1
        for a in args:
            den *= factorial(a)
        total += (-1) ** k / den
    return pre * total


def cg_spherical(l1: int, l2: int, L: int) -> np.ndarray:
    """Spherical CG tensor [2l1+1, 2l2+1, 2L+1] indexed by (m1+l1, m2+l2, M+L)."""
    out = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * L + 1))
    for m1 in range(-l1, l1 + 1):
        for m2 in range(-l2, l2 + 1):
            M = m1 + m2
            if abs(M) <= L:
                out[m1 + l1, m2 + l2, M + L] = cg_coefficient(l1, m1, l2, m2, L, M)
    return out


def real_to_spherical(l: int) -> np.ndarray:
    """Unitary U with T = U x (rows: spherical mu = -l..l, columns: real m = -l..l)."""
    U = np.zeros((2 * l + 1, 2 * l + 1), dtype=np.complex128)
    U[l, l] = 1.0
    s = 1.0 / sqrt(2.0)
    for m in range(1, l + 1):
        sign = (-1) ** m
        U[l + m, l + m] = sign * s          # T_{+m} from x_m
        U[l + m, l - m] = 1j * sign * s     # T_{+m} from x_{-m}
        U[l - m, l + m] = s                 # T_{-m} from x_m
        U[l - m, l - m] = -1j * s           # T_{-m} from x_{-m}
    return U


@functools.lru_cache(maxsize=None)
def _real_cg_complex(li: int, lf: int, lo: int) -> np.ndarray:
    C = cg_spherical(li, lf, lo)
    Ui, Uf, Uo = real_to_spherical(li), real_to_spherical(lf), real_to_spherical(lo)
    # x_out[mo] = sum conj(Uo[mu_o, mo]) C[mu_i, mu_f, mu_o] Ui[mu_i, mi] a[mi] Uf[mu_f, mf] b[mf]
    return np.einsum("ai,bf,co,abc->ifo", Ui, Uf, Uo.conj(), C)


@functools.lru_cache(maxsize=None)
def real_cg(li: int, lf: int, lo: int) -> np.ndarray:
    """Real coupling tensor [2li+1, 2lf+1, 2lo+1] of path (li, lf, lo), float64."""
    T = _real_cg_complex(li, lf, lo)
    if (li + lf + lo) % 2 == 1:
        T = -1j * T
    return np.ascontiguousarray(T.real)


def real_cg_imag_residue(li: int, lf: int, lo: int) -> float:
    """Largest imaginary part left after the phase; zero up to rounding for every path."""
    T = _real_cg_complex(li, lf, lo)
    if (li + lf + lo) % 2 == 1:
        T = -1j * T
    return float(np.abs(T.imag).max())
