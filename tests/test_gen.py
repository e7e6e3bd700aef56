"""Checks of the seeded input generators (shared by the oracle and the HIP path)."""

import numpy as np
import pytest

from gen import bf16_bits_to_f32, f32_to_bf16_bits, make_config, make_micro, neighbour_list
from gen.configs import water_box


def _brute_force_list(pos, cutoff, K):
    p = pos.astype(np.float64)
    d = np.linalg.norm(p[:, None, :] - p[None, :, :], axis=-1)
    n = pos.shape[0]
    idx = np.full((n, K), -1, dtype=np.int32)
    for i in range(n):
        js = [j for j in range(n) if j != i and d[i, j] < cutoff]
        js.sort(key=lambda j: (d[i, j], j))
        js = js[:K]
        idx[i, :len(js)] = js
    return idx


@pytest.mark.parametrize("n,cut,K", [(64, 5.0, 32), (200, 4.0, 8), (50, 100.0, 60), (1, 5.0, 4)])
def test_neighbour_list_matches_brute_force(n, cut, K):
    rng = np.random.default_rng(n)
    pos = ((rng.random((n, 3)) - 0.5) * (n / 0.1) ** (1 / 3)).astype(np.float32)
    nl = neighbour_list(pos, cut, K)
    ref = _brute_force_list(pos, cut, K)
    np.testing.assert_array_equal(nl.idx, ref)
    np.testing.assert_array_equal(nl.mask, (ref >= 0).astype(np.uint8))


def test_neighbour_list_strict_cutoff_and_empty():
    pos = np.array([[0, 0, 0], [1.0, 0, 0], [3.0, 0, 0]], dtype=np.float32)
    nl = neighbour_list(pos, 1.0, 4)
    assert nl.n_edges == 0          # distance exactly at the cutoff is excluded
    nl = neighbour_list(pos, 2.5, 4)
    assert nl.idx[0].tolist() == [1, -1, -1, -1]
    assert nl.idx[1].tolist() == [0, 2, -1, -1]
    nl = neighbour_list(np.zeros((0, 3), np.float32), 2.0, 3)
    assert nl.idx.shape == (0, 3)


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32),
                        np.array([1.0, -0.0, 0.0, 3.0e38, 1e-40, 1.00390625, 1.01171875], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(x), ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(
        torch.bfloat16).float().numpy())


def test_tiny_config_shape_and_determinism():
    a = make_config("tiny")
    b = make_config("tiny")
    assert a.pos.shape == (64, 3) and a.h.shape == (64, 4, 16)
    assert a.idx.shape == (64, 32) and a.idx.dtype == np.int32 and a.mask.dtype == np.uint8
    np.testing.assert_array_equal(a.h, b.h)
    np.testing.assert_array_equal(a.idx, b.idx)
    # valid slots first, within the cutoff, never self
    for i in range(64):
        k = int(a.mask[i].sum())
        assert a.mask[i, :k].all() and not a.mask[i, k:].any()
        js = a.idx[i, :k]
        assert (js != i).all()
        d = np.linalg.norm(a.pos[js].astype(np.float64) - a.pos[i], axis=1)
        assert (d < 5.0).all() and (np.diff(d) >= 0).all()


def test_water_geometry():
    pos = water_box(np.random.default_rng(1)).astype(np.float64)
    assert pos.shape == (648, 3)
    o, h1, h2 = pos[0::3], pos[1::3], pos[2::3]
    np.testing.assert_allclose(np.linalg.norm(h1 - o, axis=1), 0.96, atol=1e-5)
    np.testing.assert_allclose(np.linalg.norm(h2 - o, axis=1), 0.96, atol=1e-5)
    cosang = np.einsum("ij,ij->i", h1 - o, h2 - o) / 0.96 ** 2
    np.testing.assert_allclose(np.degrees(np.arccos(cosang)), 104.5, atol=1e-3)
    assert np.abs(o).max() < 9.3


def test_bf16_config_and_micro():
    c = make_config("scaleout", n_atoms=500)
    assert c.h_bits is not None and c.h_bits.dtype == np.uint16
    np.testing.assert_array_equal(bf16_bits_to_f32(c.h_bits), c.h)
    r, h, bits = make_micro(B=1000)
    np.testing.assert_allclose(np.linalg.norm(r.astype(np.float64), axis=1), 1.0, atol=1e-6)
    assert h.shape == (1000, 9, 128) and bits is None
