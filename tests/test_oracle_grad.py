"""Pins for the oracle's gradients: central finite differences of the numpy oracle."""

import numpy as np
import pytest

from oracle import tp
from oracle.attn import attn_forward
from oracle.grad import attn_backward, attn_forward_torch, eaas_vjp


def _graph(rng, N, K, p=0.7):
    idx = rng.integers(0, N, size=(N, K)).astype(np.int32)
    mask = (rng.random((N, K)) < p).astype(np.uint8)
    for i in range(N):
        idx[i][idx[i] == i] = (i + 1) % N
    return idx, mask


def test_torch_forward_matches_numpy_oracle():
    import torch
    rng = np.random.default_rng(0)
    N, K, C, H, lmax = 12, 6, 8, 2, 2
    pos = rng.standard_normal((N, 3)) * 2
    h = rng.standard_normal((N, 9, C))
    idx, mask = _graph(rng, N, K)
    mask[4] = 0
    ref = attn_forward(pos, h, idx, mask, H, lmax)
    got = attn_forward_torch(torch.from_numpy(pos), torch.from_numpy(h), idx, mask, H, lmax)
    np.testing.assert_allclose(got.numpy(), ref, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("lmax", [1, 2])
def test_attention_gradients_match_finite_differences(lmax):
    rng = np.random.default_rng(10 + lmax)
    N, K, C, H = 7, 5, 4, 2
    S = (lmax + 1) ** 2
    pos = rng.standard_normal((N, 3)) * 1.5
    h = rng.standard_normal((N, S, C))
    idx, mask = _graph(rng, N, K)
    g = rng.standard_normal((N, S, C))
    dh, dpos = attn_backward(pos, h, idx, mask, H, lmax, g)

    def loss(p, hh):
        return float((attn_forward(p, hh, idx, mask, H, lmax) * g).sum())

    eps = 1e-6
    for i in range(N):
        for a in range(3):
            e = np.zeros_like(pos)
            e[i, a] = eps
            fd = (loss(pos + e, h) - loss(pos - e, h)) / (2 * eps)
            assert abs(fd - dpos[i, a]) <= 1e-6 * (1 + abs(fd)), (i, a, fd, dpos[i, a])
    picks = [(i, s, c) for i in range(N) for s in range(S) for c in range(C)]
    for i, s, c in [picks[k] for k in rng.choice(len(picks), 40, replace=False)]:
        e = np.zeros_like(h)
        e[i, s, c] = eps
        fd = (loss(pos, h + e) - loss(pos, h - e)) / (2 * eps)
        assert abs(fd - dh[i, s, c]) <= 1e-6 * (1 + abs(fd)), (i, s, c, fd, dh[i, s, c])


def test_coupling_vjp_matches_finite_differences_and_adjoint():
    rng = np.random.default_rng(3)
    n, C, lmax = 5, 3, 2
    x = rng.standard_normal((n, 9, C))
    r = rng.standard_normal((n, 3)) * 2
    r[0] = 0.0                      # gradient at the origin (only the l_f = 1 paths move)
    g = rng.standard_normal((n, 9, C))
    dx, dr = eaas_vjp(x, r, g, lmax)
    eps = 1e-6
    for a in range(n):
        for k in range(3):
            e = np.zeros_like(r)
            e[a, k] = eps
            fd = ((tp.tp_dense(x, r + e, lmax) - tp.tp_dense(x, r - e, lmax)) * g).sum() / (2 * eps)
            assert abs(fd - dr[a, k]) <= 1e-6 * (1 + abs(fd))
    # dL/dx is the adjoint map applied to g: <g, T y> = <T^T g, y> for any y
    y = rng.standard_normal(x.shape)
    np.testing.assert_allclose((g * tp.tp_dense(y, r, lmax)).sum(), (dx * y).sum(), rtol=1e-12)


def test_lmax0_position_gradient_is_zero():
    rng = np.random.default_rng(4)
    N, K, C, H = 6, 4, 4, 2
    idx, mask = _graph(rng, N, K)
    _, dpos = attn_backward(rng.standard_normal((N, 3)), rng.standard_normal((N, 1, C)), idx, mask,
                            H, 0, rng.standard_normal((N, 1, C)))
    assert np.all(dpos == 0)


@pytest.mark.parametrize("lmax", [0, 2])
def test_projected_gradients_match_finite_differences(lmax):
    """dL/dW_Q, dL/dW_K, dL/dW_V, dL/dh and dL/dpos of the projected layer against central finite
    differences of the numpy oracle's projected forward."""
    from oracle.grad import attn_backward_proj
    rng = np.random.default_rng(40 + lmax)
    N, K, C, H = 7, 5, 4, 2
    S = (lmax + 1) ** 2
    pos = rng.standard_normal((N, 3)) * 1.5
    h = rng.standard_normal((N, S, C))
    w = (rng.standard_normal((C, C)) / 2, rng.standard_normal((C, C)) / 2,
         rng.standard_normal((lmax + 1, C, C)) / 2)
    idx, mask = _graph(rng, N, K)
    g = rng.standard_normal((N, S, C))
    dh, dpos, dwq, dwk, dwv = attn_backward_proj(pos, h, idx, mask, H, lmax, g, w)

    def loss(p, hh, ww):
        return float((attn_forward(p, hh, idx, mask, H, lmax, proj=ww) * g).sum())

    eps = 1e-6

    def fd_check(arr_index, grad, make):
        for k in arr_index:
            plus, minus = make(k, eps), make(k, -eps)
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            assert abs(fd - grad[k]) <= 1e-6 * (1 + abs(fd)), (k, fd, grad[k])

    def w_at(which, k, e):
        ww = [x.copy() for x in w]
        ww[which][k] += e
        return pos, h, tuple(ww)

    for which, grad in ((0, dwq), (1, dwk), (2, dwv)):
        keys = list(np.ndindex(grad.shape))
        picks = [keys[i] for i in rng.choice(len(keys), min(12, len(keys)), replace=False)]
        fd_check(picks, grad, lambda k, e, which=which: w_at(which, k, e))
    hk = list(np.ndindex(h.shape))
    fd_check([hk[i] for i in rng.choice(len(hk), 12, replace=False)], dh,
             lambda k, e: (pos, h + np.where(np.arange(h.size).reshape(h.shape) ==
                                             np.ravel_multi_index(k, h.shape), e, 0.0), w))
    if lmax > 0:
        fd_check([(i, a) for i in range(N) for a in range(3)], dpos,
                 lambda k, e: (pos + np.where(np.arange(pos.size).reshape(pos.shape) ==
                                              np.ravel_multi_index(k, pos.shape), e, 0.0), h, w))
    else:
        assert np.all(dpos == 0)
