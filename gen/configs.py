"""Seeded workloads shaped like the E2Former-V2 pages' systems.

The pages (E2Former-V2 news write-up on stapisi.com, sections 1.1, 3.2, 4.3
and 5.1; the gist.science summary of arXiv 2601.16622, technical summary
section 4) describe liquid water boxes of 216 molecules, a 32,768-atom
latency point, a K=256 memory point and 100,000-atom systems, with 16 heads,
128 channels and a 5.0 A cutoff at lmax=2.  None of their datasets ships
here, so these generators stand in for them:

* uniform-random atoms at 0.1 atoms/A^3 (about the atom density of liquid
  water) in a cube centred at the origin, open boundaries;
* 216 rigid water molecules (O-H 0.96 A, H-O-H 104.5 deg) on a jittered
  6x6x6 lattice with uniformly random orientations;
* irrep features drawn i.i.d. from N(0, 1) in float32, optionally rounded
  to bfloat16 storage (round to nearest, ties to even);
* a padded neighbour list: j != i with |r_i - r_j| < r_c (strict), sorted by
  (distance, j), truncated to the K nearest, padded with index -1 and
  mask 0.

Periodic boundaries are listed as future work on the pages (section 6), so
every box here is open.  Nothing in this module computes any part of the
attention or the tensor product.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
from scipy.spatial import cKDTree

DENSITY = 0.1  # atoms per cubic angstrom


# --------------------------------------------------------------------------
# bfloat16 storage helpers (format conversion only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to exactly equal float32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# geometry
# --------------------------------------------------------------------------

def uniform_box(rng: np.random.Generator, n: int, density: float = DENSITY) -> np.ndarray:
    """n points uniform in a cube of volume n/density centred at the origin (float32)."""
    side = (n / density) ** (1.0 / 3.0)
    return ((rng.random((n, 3)) - 0.5) * side).astype(np.float32)


def _random_rotations(rng: np.random.Generator, n: int) -> np.ndarray:
    """Uniformly random rotation matrices from uniform unit quaternions (Shoemake, 1992)."""
    u1, u2, u3 = rng.random((3, n))
    a = np.sqrt(1.0 - u1)
    b = np.sqrt(u1)
    w = a * np.sin(2 * np.pi * u2)
    x = a * np.cos(2 * np.pi * u2)
    y = b * np.sin(2 * np.pi * u3)
    z = b * np.cos(2 * np.pi * u3)
    R = np.empty((n, 3, 3))
    R[:, 0, 0] = 1 - 2 * (y * y + z * z)
    R[:, 0, 1] = 2 * (x * y - z * w)
    R[:, 0, 2] = 2 * (x * z + y * w)
    R[:, 1, 0] = 2 * (x * y + z * w)
    R[:, 1, 1] = 1 - 2 * (x * x + z * z)
    R[:, 1, 2] = 2 * (y * z - x * w)
    R[:, 2, 0] = 2 * (x * z - y * w)
    R[:, 2, 1] = 2 * (y * z + x * w)
    R[:, 2, 2] = 1 - 2 * (x * x + y * y)
    return R


def water_box(rng: np.random.Generator, n_side: int = 6, spacing: float = 3.1,
              bond: float = 0.96, angle_deg: float = 104.5, jitter: float = 0.2) -> np.ndarray:
    """Rigid water molecules on a jittered cubic lattice, ordered O, H, H (float32)."""
    ii = (np.arange(n_side) + 0.5) * spacing - 0.5 * n_side * spacing
    ox = np.stack(np.meshgrid(ii, ii, ii, indexing="ij"), axis=-1).reshape(-1, 3)
    nmol = ox.shape[0]
    ox = ox + rng.uniform(-jitter, jitter, size=(nmol, 3))
    half = math.radians(angle_deg) / 2.0
    local = np.array([[0.0, 0.0, 0.0],
                      [bond * math.sin(half), 0.0, bond * math.cos(half)],
                      [-bond * math.sin(half), 0.0, bond * math.cos(half)]])
    R = _random_rotations(rng, nmol)
    atoms = ox[:, None, :] + np.einsum("nab,kb->nka", R, local)
    return atoms.reshape(-1, 3).astype(np.float32)


def unit_vectors(rng: np.random.Generator, n: int) -> np.ndarray:
    """n unit vectors uniform on the sphere (normalised Gaussian draws), float32."""
    g = rng.standard_normal((n, 3))
    return (g / np.linalg.norm(g, axis=1, keepdims=True)).astype(np.float32)


# --------------------------------------------------------------------------
# neighbour list
# --------------------------------------------------------------------------

@dataclasses.dataclass
class NeighbourList:
    idx: np.ndarray        # [N, K] int32, -1 at padded slots
    mask: np.ndarray       # [N, K] uint8, 1 at valid slots
    n_within: np.ndarray   # [N] number of j != i strictly inside the cutoff

    @property
    def n_edges(self) -> int:
        return int(self.mask.sum(dtype=np.int64))

    @property
    def truncated_fraction(self) -> float:
        k = self.idx.shape[1]
        return float((self.n_within > k).mean()) if self.n_within.size else 0.0


def neighbour_list(pos: np.ndarray, cutoff: float, K: int) -> NeighbourList:
    """Padded list of the K nearest j != i with |r_i - r_j| < cutoff, valid slots first."""
    pos = np.asarray(pos)
    n = pos.shape[0]
    idx = np.full((n, K), -1, dtype=np.int32)
    mask = np.zeros((n, K), dtype=np.uint8)
    if n == 0:
        return NeighbourList(idx, mask, np.zeros(0, dtype=np.int64))
    p64 = pos.astype(np.float64)
    tree = cKDTree(p64)
    kq = min(K + 1, n)
    _, cand = tree.query(p64, k=kq, distance_upper_bound=cutoff)
    cand = np.asarray(cand).reshape(n, kq)
    rows = np.repeat(np.arange(n), kq).reshape(n, kq)
    ok = (cand < n) & (cand != rows)
    cj = np.where(ok, cand, 0)
    d = np.linalg.norm(p64[rows] - p64[cj], axis=-1)
    ok &= d < cutoff
    # order each row by (distance, j); invalid entries go last
    dkey = np.where(ok, d, np.inf)
    jkey = np.where(ok, cand, np.iinfo(np.int64).max)
    flat = np.lexsort((jkey.ravel(), dkey.ravel(), rows.ravel()))
    order = (flat % kq).reshape(n, kq)
    cand_s = np.take_along_axis(cand, order, axis=1)
    ok_s = np.take_along_axis(ok, order, axis=1)
    take = min(K, kq)
    sel_ok = ok_s[:, :take]
    idx[:, :take] = np.where(sel_ok, cand_s[:, :take], -1)
    mask[:, :take] = sel_ok
    n_within = tree.query_ball_point(p64, r=np.nextafter(cutoff, 0.0), return_length=True)
    n_within = np.asarray(n_within, dtype=np.int64) - 1
    return NeighbourList(idx, mask, n_within)


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class ConfigSpec:
    name: str
    kind: str            # "uniform" | "water"
    n_atoms: int
    cutoff: float
    K: int
    lmax: int
    C: int
    H: int
    dtype: str           # "f32" | "bf16"  (storage of h, workspace and out)
    seed: int
    description: str


CONFIGS = {
    "tiny": ConfigSpec("tiny", "uniform", 64, 5.0, 32, 1, 16, 2, "f32", 0,
                       "N=64 uniform at 0.1/A^3, r_c 5.0 A, K=32, lmax=1, C=16, H=2, fp32"),
    "water": ConfigSpec("water", "water", 648, 5.0, 64, 2, 128, 16, "f32", 1,
                        "216 rigid H2O (648 atoms), 18.6 A box, r_c 5.0 A, K=64, lmax=2, "
                        "C=128, H=16, fp32"),
    "large": ConfigSpec("large", "uniform", 32768, 8.4, 256, 2, 128, 16, "f32", 2,
                        "N=32768 uniform at 0.1/A^3, r_c 8.4 A, K=256, lmax=2, C=128, H=16, fp32"),
    "scaleout": ConfigSpec("scaleout", "uniform", 100000, 5.0, 64, 2, 128, 16, "bf16", 4,
                           "N=100000 uniform at 0.1/A^3, r_c 5.0 A, K=64, lmax=2, C=128, H=16, "
                           "bf16 storage"),
}

MICRO_SEED = 3
MICRO_B = 1 << 20


@dataclasses.dataclass
class Config:
    spec: ConfigSpec
    pos: np.ndarray              # [N, 3] float32
    h: np.ndarray                # [N, S, C] float32 (bf16-representable for bf16 configs)
    h_bits: Optional[np.ndarray] # [N, S, C] uint16 for bf16 configs, else None
    nl: NeighbourList

    @property
    def N(self) -> int:
        return self.pos.shape[0]

    @property
    def S(self) -> int:
        return (self.spec.lmax + 1) ** 2

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.spec.C / self.spec.H)

    @property
    def idx(self) -> np.ndarray:
        return self.nl.idx

    @property
    def mask(self) -> np.ndarray:
        return self.nl.mask


def features(rng: np.random.Generator, n: int, S: int, C: int, dtype: str):
    """i.i.d. N(0,1) float32 features; bf16 storage rounds them (RNE)."""
    h = rng.standard_normal((n, S, C), dtype=np.float32)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(h)
        return bf16_bits_to_f32(bits), bits
    if dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return h, None


def make_config(name: str, n_atoms: Optional[int] = None, K: Optional[int] = None,
                seed: Optional[int] = None, dtype: Optional[str] = None) -> Config:
    """Build one named workload; n_atoms / K / seed / dtype override for small test variants."""
    spec = CONFIGS[name]
    if n_atoms is not None or K is not None or seed is not None or dtype is not None:
        spec = dataclasses.replace(
            spec,
            n_atoms=spec.n_atoms if n_atoms is None else n_atoms,
            K=spec.K if K is None else K,
            seed=spec.seed if seed is None else seed,
            dtype=spec.dtype if dtype is None else dtype,
        )
    rng = np.random.default_rng(spec.seed)
    if spec.kind == "uniform":
        pos = uniform_box(rng, spec.n_atoms)
    elif spec.kind == "water":
        if spec.n_atoms % 3 != 0:
            raise ValueError("water config needs a multiple of 3 atoms")
        n_side = round((spec.n_atoms // 3) ** (1.0 / 3.0))
        if 3 * n_side ** 3 != spec.n_atoms:
            raise ValueError("water config needs 3*n^3 atoms")
        pos = water_box(rng, n_side=n_side)
    else:
        raise ValueError(spec.kind)
    S = (spec.lmax + 1) ** 2
    h, bits = features(rng, pos.shape[0], S, spec.C, spec.dtype)
    nl = neighbour_list(pos, spec.cutoff, spec.K)
    return Config(spec, pos, h, bits, nl)


def make_micro(B: int = MICRO_B, C: int = 128, lmax: int = 2, seed: int = MICRO_SEED,
               dtype: str = "f32"):
    """EAAS tensor-product workload: B unit vectors uniform on S^2 and features [B, S, C]."""
    rng = np.random.default_rng(seed)
    r = unit_vectors(rng, B)
    h, bits = features(rng, B, (lmax + 1) ** 2, C, dtype)
    return r, h, bits


def proj_weights(lmax: int, C: int, seed: int, dtype: str = "f32"):
    """Random projection weights (W_Q [C, C], W_K [C, C], W_V [lmax + 1, C, C]), i.i.d.
    N(0, 1/C) so that projected features keep unit scale; bf16 rounds them (RNE).
    Returns float32 arrays (already rounded for bf16)."""
    rng = np.random.default_rng(seed)
    scale = np.float32(1.0 / np.sqrt(C))
    ws = [rng.standard_normal((C, C), dtype=np.float32) * scale,
          rng.standard_normal((C, C), dtype=np.float32) * scale,
          rng.standard_normal((lmax + 1, C, C), dtype=np.float32) * scale]
    if dtype == "bf16":
        ws = [bf16_bits_to_f32(f32_to_bf16_bits(w)) for w in ws]
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return tuple(ws)
