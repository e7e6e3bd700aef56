"""Pins for the oracle's envelope-weighted softmax (oracle/attn.py, ``env_cutoff``).

Sources of truth other than the oracle itself: the polynomial's defining
integral (scipy quadrature), its smoothness at the cutoff, torch's
scaled-dot-product attention with an additive float mask (log of the
envelope), reductions to the plain softmax (far cutoff, equidistant
neighbours), to masking (neighbours at or beyond the cutoff), continuity as a
neighbour crosses the cutoff, rotation equivariance, and finite differences of
the numpy oracle for the torch gradient.
"""

import math

import numpy as np
import pytest

from oracle import wigner
from oracle.attn import attn_forward, envelope
from oracle.grad import attn_backward, attn_forward_torch


def test_envelope_is_the_integral_of_its_derivative():
    from scipy.integrate import quad
    rng = np.random.default_rng(0)
    for x in np.r_[rng.random(20), 0.0, 0.5, 0.999]:
        want = quad(lambda t: 105.0 * t ** 4 * (1.0 - t) ** 2, x, 1.0, epsabs=1e-15)[0]
        assert abs(envelope(x) - want) < 1e-13, x
    assert envelope(0.0) == 1.0
    assert np.all(envelope([1.0, 1.5, 7.0]) == 0.0)


def test_envelope_keeps_its_relative_precision_up_to_the_cutoff():
    """Against the defining polynomial 1 - 21 x^5 + 35 x^6 - 15 x^7 evaluated exactly (rational
    arithmetic on each float x): relative error at float64 rounding level, right up to x -> 1,
    where the pair weights and their gradients are relative to u."""
    from fractions import Fraction
    xs = [1.0 - 10.0 ** -k for k in range(1, 12)] + [0.0, 0.25, 0.5, 0.75, 0.9999999999]
    xs += list(np.random.default_rng(3).random(20))
    for x in xs:
        f = Fraction(x)
        exact = 1 - 21 * f ** 5 + 35 * f ** 6 - 15 * f ** 7
        got = float(envelope(x))
        assert abs(Fraction(got) - exact) <= Fraction(1, 10 ** 13) * abs(exact), x


def test_envelope_is_smooth_and_monotone_at_the_cutoff():
    x = np.linspace(0.0, 1.0, 2001)
    u = envelope(x)
    assert np.all(np.diff(u) <= 0.0) and np.all(u >= 0.0)
    # a triple zero at x = 1 (u, u' and u'' all vanish there, so the junction with
    # 0 beyond the cutoff is C^2): u(1 - y) / y^3 tends to a finite limit (35)
    y = np.array([1e-2, 1e-3, 1e-4])
    ratio = envelope(1.0 - y) / y ** 3
    np.testing.assert_allclose(ratio, 35.0, rtol=0.25)
    assert abs(ratio[-1] - 35.0) < abs(ratio[0] - 35.0)


def _graph(rng, N, K, p=0.8):
    """K distinct sources j != i per row (a dense mask counts each pair once), ~p valid."""
    idx = np.empty((N, K), np.int32)
    for i in range(N):
        others = np.delete(np.arange(N), i)
        idx[i] = rng.choice(others, K, replace=False)
    mask = (rng.random((N, K)) < p).astype(np.uint8)
    return idx, mask


def _sdpa_logmask(h_q, v, idx, mask, heads, scale, addmask):
    """torch SDPA with an additive float mask: -inf off the graph, `addmask` on it."""
    import torch
    N, C = h_q.shape
    d = C // heads
    M = np.full((N, N), -np.inf)
    rows = np.repeat(np.arange(N), idx.shape[1])
    ok = mask.ravel() != 0
    M[rows[ok], idx.ravel()[ok]] = addmask[rows[ok], idx.ravel()[ok]]
    q = torch.from_numpy(h_q.reshape(N, heads, d).transpose(1, 0, 2).copy())
    Sv = v.shape[1]
    vv = torch.from_numpy(v.reshape(N, Sv, heads, d).transpose(2, 0, 1, 3).reshape(heads, N, Sv * d).copy())
    out = torch.nn.functional.scaled_dot_product_attention(q, q, vv, attn_mask=torch.from_numpy(M),
                                                           scale=scale)
    return out.numpy().reshape(heads, N, Sv, d).transpose(1, 2, 0, 3).reshape(N, Sv, C)


def test_lmax0_envelope_equals_sdpa_with_log_envelope_mask():
    rng = np.random.default_rng(1)
    N, K, C, H = 40, 12, 16, 4
    pos = rng.random((N, 3)) * 6
    h = rng.standard_normal((N, 1, C))
    idx, mask = _graph(rng, N, K)
    r_env = 5.0
    dist = np.linalg.norm(pos[:, None, :] - pos[None, :, :], axis=-1)
    with np.errstate(divide="ignore"):
        logu = np.log(envelope(dist / r_env))
    # keep only slots strictly inside the envelope (SDPA would give NaN on an all -inf row)
    inside = np.take_along_axis(dist, idx.astype(np.int64), axis=1) < r_env
    m2 = (mask.astype(bool) & inside).astype(np.uint8)
    assert m2.sum() < mask.sum()                      # some slots do fall outside
    rows_ok = m2.any(axis=1)
    out = attn_forward(pos, h, idx, mask, H, 0, env_cutoff=r_env)
    ref = _sdpa_logmask(h[:, 0, :], h, idx, m2, H, 1 / math.sqrt(C // H), logu)
    np.testing.assert_allclose(out[rows_ok], ref[rows_ok], atol=1e-12)
    assert np.all(out[~rows_ok] == 0.0)


def test_far_cutoff_and_equidistant_neighbours_reduce_to_plain_softmax():
    rng = np.random.default_rng(2)
    N, K, C, H, lmax = 24, 8, 8, 2, 2
    pos = rng.standard_normal((N, 3)) * 2
    h = rng.standard_normal((N, 9, C))
    idx, mask = _graph(rng, N, K)
    plain = attn_forward(pos, h, idx, mask, H, lmax)
    far = attn_forward(pos, h, idx, mask, H, lmax, env_cutoff=1e7)
    np.testing.assert_allclose(far, plain, atol=1e-12 * np.abs(plain).max())
    # target 0 at the centre of a sphere of sources: the envelope cancels out
    dirs = rng.standard_normal((N, 3))
    p2 = 2.5 * dirs / np.linalg.norm(dirs, axis=1, keepdims=True)
    p2[0] = 0.0
    idx2 = np.tile(np.arange(1, K + 1, dtype=np.int32), (N, 1))
    mask2 = np.ones((N, K), np.uint8)
    a = attn_forward(p2, h, idx2, mask2, H, lmax, targets=np.array([0]))
    b = attn_forward(p2, h, idx2, mask2, H, lmax, targets=np.array([0]), env_cutoff=4.0)
    np.testing.assert_allclose(b, a, atol=1e-12 * np.abs(a).max())


def test_neighbours_beyond_the_cutoff_act_as_masked_and_fade_continuously():
    rng = np.random.default_rng(3)
    N, K, C, H, lmax = 10, 4, 8, 2, 2
    h = rng.standard_normal((N, 9, C))
    pos = np.zeros((N, 3))
    pos[0] = [0.3, -0.2, 0.1]
    pos[1] = pos[0] + [1.0, 0.0, 0.0]
    pos[2] = pos[0] + [0.0, 1.5, 0.0]
    pos[3] = pos[0] + [0.0, 0.0, 3.0]       # this neighbour moves across r_env = 3
    idx = np.array([[1, 2, 3, 9]] + [[0, 0, 0, 0]] * (N - 1), np.int32)
    mask = np.array([[1, 1, 1, 0]] + [[1, 0, 0, 0]] * (N - 1), np.uint8)
    masked = mask.copy()
    masked[0, 2] = 0
    ref = attn_forward(pos, h, idx, masked, H, lmax, env_cutoff=3.0, targets=np.array([0]))
    for dz in (0.0, 0.5):                    # at and beyond the cutoff: the masked result
        p = pos.copy()                       # (up to the rounding of a different softmax max)
        p[3, 2] += dz
        got = attn_forward(p, h, idx, mask, H, lmax, env_cutoff=3.0, targets=np.array([0]))
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14 * np.abs(ref).max())
    prev = None
    for eps in (1e-1, 1e-2, 1e-3):           # just inside: converges like eps^3
        p = pos.copy()
        p[3, 2] -= eps
        gap = np.abs(attn_forward(p, h, idx, mask, H, lmax, env_cutoff=3.0,
                                  targets=np.array([0])) - ref).max()
        if prev is not None:
            assert gap < prev * 2e-2
        prev = gap
    # every neighbour beyond the cutoff: the row is zero, like an empty row
    got = attn_forward(pos, h, idx, mask, H, lmax, env_cutoff=0.5, targets=np.array([0]))
    assert np.all(got == 0.0)


def test_envelope_attention_stays_equivariant():
    rng = np.random.default_rng(4)
    N, K, C, H, lmax = 26, 9, 8, 2, 2
    h = rng.standard_normal((N, 9, C))
    pos = rng.standard_normal((N, 3)) * 2
    idx, mask = _graph(rng, N, K)
    out = attn_forward(pos, h, idx, mask, H, lmax, env_cutoff=3.5)
    R = wigner.random_rotation(rng)
    D = wigner.wigner_d_full(lmax, R)
    out_r = attn_forward(pos @ R.T, np.einsum("ab,nbc->nac", D, h), idx, mask, H, lmax,
                         env_cutoff=3.5)
    np.testing.assert_allclose(out_r, np.einsum("ab,nbc->nac", D, out), atol=1e-10 * np.abs(out).max())


@pytest.mark.parametrize("lmax", [0, 2])
def test_envelope_gradients_match_finite_differences(lmax):
    import torch
    rng = np.random.default_rng(20 + lmax)
    N, K, C, H = 7, 5, 4, 2
    S = (lmax + 1) ** 2
    pos = rng.random((N, 3)) * 3
    h = rng.standard_normal((N, S, C))
    idx, mask = _graph(rng, N, K)
    g = rng.standard_normal((N, S, C))
    r_env = 2.5
    ref = attn_forward(pos, h, idx, mask, H, lmax, env_cutoff=r_env)
    got = attn_forward_torch(torch.from_numpy(pos), torch.from_numpy(h), idx, mask, H, lmax,
                             env_cutoff=r_env)
    np.testing.assert_allclose(got.numpy(), ref, atol=1e-12 * np.abs(ref).max())
    dh, dpos = attn_backward(pos, h, idx, mask, H, lmax, g, env_cutoff=r_env)
    assert np.abs(dpos).max() > 0             # positions enter through the envelope even at l = 0

    def loss(p, hh):
        return float((attn_forward(p, hh, idx, mask, H, lmax, env_cutoff=r_env) * g).sum())

    eps = 1e-6
    for i in range(N):
        for a in range(3):
            e = np.zeros_like(pos)
            e[i, a] = eps
            fd = (loss(pos + e, h) - loss(pos - e, h)) / (2 * eps)
            assert abs(fd - dpos[i, a]) <= 1e-6 * (1 + abs(fd)), (i, a, fd, dpos[i, a])
    for i, s, c in [(0, 0, 0), (3, S - 1, 2), (5, 0, 3), (6, S // 2, 1)]:
        e = np.zeros_like(h)
        e[i, s, c] = eps
        fd = (loss(pos, h + e) - loss(pos, h - e)) / (2 * eps)
        assert abs(fd - dh[i, s, c]) <= 1e-6 * (1 + abs(fd)), (i, s, c, fd, dh[i, s, c])
