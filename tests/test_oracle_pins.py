"""Pins for the CPU oracle: each check ties it to something other than itself.

Sources of truth used here: sympy's Clebsch-Gordan routine and scipy's
spherical harmonics (library routines), textbook coupling tables and
identities (tests/golden), group properties of rotations, Proposition 4.3
of the E2Former-V2 write-up (EAAS equals the dense product), rotation
equivariance, and torch's scaled-dot-product attention.
"""

import math
import os

import numpy as np
import pytest

from oracle import cg, sh, tp, wigner
from oracle.attn import attention_weights, attn_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- harmonics

def _real_from_scipy(l, r):
    """Racah-normalised real harmonics built from scipy's complex Y_l^m."""
    from scipy.special import sph_harm_y
    r = np.asarray(r, dtype=np.float64)
    rn = np.linalg.norm(r, axis=-1)
    theta = np.arccos(np.clip(r[:, 2] / rn, -1, 1))
    phi = np.mod(np.arctan2(r[:, 1], r[:, 0]), 2 * np.pi)
    k = math.sqrt(4 * math.pi / (2 * l + 1))
    out = np.zeros((r.shape[0], 2 * l + 1))
    for m in range(-l, l + 1):
        Y = sph_harm_y(l, abs(m), theta, phi)
        if m == 0:
            v = Y.real
        elif m > 0:
            v = math.sqrt(2) * (-1) ** m * Y.real
        else:
            v = math.sqrt(2) * (-1) ** m * Y.imag
        out[:, m + l] = k * v * rn ** l
    return out


@pytest.mark.parametrize("l", [0, 1, 2])
def test_solid_harmonics_match_scipy(l):
    r = np.random.default_rng(1).standard_normal((50, 3)) * 3.0
    np.testing.assert_allclose(sh.solid_harmonic(l, r), _real_from_scipy(l, r), rtol=1e-12, atol=1e-12)


def test_solid_harmonics_addition_theorem_and_axis():
    rng = np.random.default_rng(2)
    u = rng.standard_normal((100, 3))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    for l in range(3):
        np.testing.assert_allclose((sh.solid_harmonic(l, u) ** 2).sum(-1), 1.0, atol=1e-13)
        z = sh.solid_harmonic(l, np.array([[0.0, 0.0, 2.5]]))[0]
        expect = np.zeros(2 * l + 1)
        expect[l] = 2.5 ** l          # only m = 0 survives on the z axis (Lemma 4.1)
        np.testing.assert_allclose(z, expect, atol=1e-13)


# --------------------------------------------------------- Clebsch-Gordan

def test_cg_matches_golden_table():
    path = os.path.join(GOLDEN, "cg_textbook.txt")
    n = 0
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        j1, m1, j2, m2, J, M, v = line.split()
        got = cg.cg_coefficient(int(j1), int(m1), int(j2), int(m2), int(J), int(M))
        assert abs(got - float(v)) < 1e-12, (line, got)
        n += 1
    assert n >= 15


def test_cg_matches_sympy():
    from sympy.physics.wigner import clebsch_gordan
    for j1 in range(3):
        for j2 in range(3):
            for J in range(abs(j1 - j2), min(j1 + j2, 3) + 1):
                for m1 in range(-j1, j1 + 1):
                    for m2 in range(-j2, j2 + 1):
                        M = m1 + m2
                        if abs(M) > J:
                            continue
                        ref = float(clebsch_gordan(j1, j2, J, m1, m2, M))
                        got = cg.cg_coefficient(j1, m1, j2, m2, J, M)
                        assert abs(got - ref) < 1e-13, (j1, m1, j2, m2, J, M, got, ref)


def test_cg_orthonormal():
    for l1 in range(3):
        for l2 in range(3):
            rows = []
            for L in range(abs(l1 - l2), l1 + l2 + 1):
                T = cg.cg_spherical(l1, l2, L)
                for M in range(2 * L + 1):
                    rows.append(T[:, :, M].ravel())
            A = np.array(rows)          # complete orthonormal change of basis
            np.testing.assert_allclose(A @ A.T, np.eye(A.shape[0]), atol=1e-13)


@pytest.mark.parametrize("p", tp.paths(2))
def test_real_cg_is_real_and_equivariant(p):
    li, lf, lo = p
    assert cg.real_cg_imag_residue(li, lf, lo) < 1e-12
    T = cg.real_cg(li, lf, lo)
    R = wigner.random_rotation(np.random.default_rng(7))
    Di, Df, Do = (wigner.wigner_d(l, R) for l in (li, lf, lo))
    # coupling commutes with rotation: T(Di a, Df b) = Do T(a, b)
    lhs = np.einsum("ifo,ia,fb->abo", T, Di, Df)
    rhs = np.einsum("abp,op->abo", T, Do)
    np.testing.assert_allclose(lhs, rhs, atol=1e-12)


def test_textbook_vector_couplings():
    rng = np.random.default_rng(3)
    a = rng.standard_normal(3)    # Cartesian (x, y, z)
    b = rng.standard_normal(3)
    yzx = [1, 2, 0]
    ar, br = a[yzx], b[yzx]       # real l = 1 components (y, z, x)
    s0 = np.einsum("ifo,i,f->o", cg.real_cg(1, 1, 0), ar, br)
    np.testing.assert_allclose(s0, [-a @ b / math.sqrt(3)], atol=1e-14)
    v1 = np.einsum("ifo,i,f->o", cg.real_cg(1, 1, 1), ar, br)
    np.testing.assert_allclose(v1, np.cross(a, b)[yzx] / math.sqrt(2), atol=1e-14)
    # rank 2 of two vectors: symmetric traceless part, normalised like R_2
    t2 = np.einsum("ifo,i,f->o", cg.real_cg(1, 1, 2), ar, br)
    np.testing.assert_allclose(np.einsum("ifo,i,f->o", cg.real_cg(1, 1, 2), a[yzx], a[yzx]),
                               sh.solid_harmonic(2, a) * math.sqrt(2.0 / 3.0), atol=1e-13)
    assert np.isfinite(t2).all()
    # scalar feature times harmonic, and feature times the l = 0 harmonic
    for l in range(3):
        T = cg.real_cg(0, l, l)
        np.testing.assert_allclose(T[0], np.eye(2 * l + 1), atol=1e-14)
        T = cg.real_cg(l, 0, l)
        np.testing.assert_allclose(T[:, 0, :], np.eye(2 * l + 1), atol=1e-14)


# ---------------------------------------------------------------- Wigner-D

def test_wigner_group_properties():
    rng = np.random.default_rng(4)
    P = np.array([[0, 1, 0], [0, 0, 1], [1, 0, 0]], dtype=float)   # (x,y,z) -> (y,z,x)
    for _ in range(5):
        R1, R2 = wigner.random_rotation(rng), wigner.random_rotation(rng)
        np.testing.assert_allclose(wigner.wigner_d(1, R1), P @ R1 @ P.T, atol=1e-13)
        for l in range(3):
            D1, D2 = wigner.wigner_d(l, R1), wigner.wigner_d(l, R2)
            np.testing.assert_allclose(D1 @ D1.T, np.eye(2 * l + 1), atol=1e-12)
            assert abs(np.linalg.det(D1) - 1.0) < 1e-12
            np.testing.assert_allclose(wigner.wigner_d(l, R1 @ R2), D1 @ D2, atol=1e-12)


def test_alignment_rotation():
    rng = np.random.default_rng(5)
    rs = list(rng.standard_normal((20, 3)) * 10) + [np.array([0, 0, 3.0]), np.array([0, 0, -2.0]),
                                                     np.array([1e-30, 0, 1.0]), np.zeros(3)]
    for r in rs:
        Q = wigner.alignment_rotation(r)
        assert abs(np.linalg.det(Q) - 1.0) < 1e-6     # write-up section 5.2 bound
        np.testing.assert_allclose(Q @ Q.T, np.eye(3), atol=1e-14)
        n = np.linalg.norm(r)
        if n > 0:
            np.testing.assert_allclose(Q @ (r / n), [0, 0, 1.0], atol=1e-14)


# ------------------------------------------------- tensor product and EAAS

def test_path_enumeration():
    assert tp.paths(0) == [(0, 0, 0)]
    assert tp.paths(1) == [(0, 0, 0), (0, 1, 1), (1, 0, 1), (1, 1, 0), (1, 1, 1)]
    assert len(tp.paths(2)) == 15
    for li, lf, lo in tp.paths(2):
        assert abs(li - lf) <= lo <= li + lf


def test_sparse_rule_is_mf0_slice_of_dense():
    """The section 2.2 reindex rule equals the m_f = 0 slice of the dense coupling."""
    rule = tp.sparse_rule(2)
    assert len(rule) == 37
    for p, (li, lf, lo) in enumerate(tp.paths(2)):
        dense = cg.real_cg(li, lf, lo)[:, lf, :]        # m_f = 0 column: [2li+1, 2lo+1]
        sparse = np.zeros_like(dense)
        for pp, lo_, mo, li_, mi, c in rule:
            if pp == p:
                assert (li_, lo_) == (li, lo)
                even = (li + lf + lo) % 2 == 0
                assert (mi == mo) if even else (mi == -mo)
                sparse[mi + li, mo + lo] += c
        np.testing.assert_allclose(sparse, dense, atol=1e-14)


@pytest.mark.parametrize("lmax", [0, 1, 2])
def test_prop43_eaas_equals_dense(lmax):
    """Proposition 4.3: rotate, sparse reindex and rotate back equals the dense product."""
    rng = np.random.default_rng(10 + lmax)
    n, C = 12, 5
    S = (lmax + 1) ** 2
    x = rng.standard_normal((n, S, C))
    r = rng.standard_normal((n, 3)) * 4.0
    r[0] = [0, 0, 2.0]
    r[1] = [0, 0, -3.0]
    r[2] = [0, 0, 0.0]
    r[3] = [1e-9, -2e-9, 1.5]
    P = len(tp.paths(lmax))
    for p in range(P):
        w = np.zeros(P)
        w[p] = 1.0
        d = tp.tp_dense(x, r, lmax, w)
        e = tp.eaas_reference(x, r, lmax, w)
        scale = np.abs(d).max() + 1e-300
        assert np.abs(d - e).max() <= 1e-12 * scale, tp.paths(lmax)[p]
    w = rng.standard_normal(P)
    d = tp.tp_dense(x, r, lmax, w)
    e = tp.eaas_reference(x, r, lmax, w)
    assert np.abs(d - e).max() <= 1e-12 * np.abs(d).max()


def test_eaas_gauge_independence():
    """Any extra rotation about z in the aligned frame leaves the result unchanged."""
    rng = np.random.default_rng(6)
    lmax, C = 2, 3
    x = rng.standard_normal((1, 9, C))
    r = rng.standard_normal(3) * 2
    rule = tp.sparse_rule(lmax)
    outs = []
    for gamma in [0.0, 0.7, 2.5]:
        Q = wigner.rot_z(gamma) @ wigner.alignment_rotation(r)
        D = wigner.wigner_d_full(lmax, Q)
        xt = D @ x[0]
        yt = np.zeros_like(xt)
        for p, lo, mo, li, mi, c in rule:
            lf = tp.paths(lmax)[p][1]
            yt[lo * lo + lo + mo] += c * np.linalg.norm(r) ** lf * xt[li * li + li + mi]
        outs.append(D.T @ yt)
    np.testing.assert_allclose(outs[1], outs[0], atol=1e-12)
    np.testing.assert_allclose(outs[2], outs[0], atol=1e-12)
    np.testing.assert_allclose(outs[0], tp.tp_dense(x, r[None], lmax)[0], atol=1e-12)


def test_tp_dense_equivariant():
    rng = np.random.default_rng(8)
    lmax = 2
    x = rng.standard_normal((6, 9, 4))
    r = rng.standard_normal((6, 3)) * 3
    R = wigner.random_rotation(rng)
    D = wigner.wigner_d_full(lmax, R)
    lhs = tp.tp_dense(np.einsum("ab,nbc->nac", D, x), r @ R.T, lmax)
    rhs = np.einsum("ab,nbc->nac", D, tp.tp_dense(x, r, lmax))
    np.testing.assert_allclose(lhs, rhs, atol=1e-10 * np.abs(rhs).max())


# ---------------------------------------------------------------- attention

def _random_graph(rng, N, K, p_valid=0.7, allow_empty=False):
    idx = np.full((N, K), -1, dtype=np.int32)
    mask = np.zeros((N, K), dtype=np.uint8)
    for i in range(N):
        cand = np.setdiff1d(np.arange(N), [i])
        k = rng.binomial(K, p_valid)
        if not allow_empty:
            k = max(k, 1)
        k = min(k, cand.size)
        js = rng.choice(cand, size=k, replace=False)
        slots = rng.choice(K, size=k, replace=False)     # valid slots anywhere in the row
        idx[i, slots] = js
        mask[i, slots] = 1
    return idx, mask


def _sdpa(h_q, v, idx, mask, heads, scale):
    """torch's scaled-dot-product attention with a dense boolean adjacency."""
    import torch
    N, C = h_q.shape
    d = C // heads
    adj = np.zeros((N, N), dtype=bool)
    rows = np.repeat(np.arange(N), idx.shape[1])
    ok = mask.ravel() != 0
    adj[rows[ok], idx.ravel()[ok]] = True
    q = torch.from_numpy(h_q.reshape(N, heads, d).transpose(1, 0, 2).copy())
    Sv = v.shape[1]
    vv = torch.from_numpy(v.reshape(N, Sv, heads, d).transpose(2, 0, 1, 3).reshape(heads, N, Sv * d).copy())
    out = torch.nn.functional.scaled_dot_product_attention(
        q, q, vv, attn_mask=torch.from_numpy(adj), scale=scale)
    return out.numpy().reshape(heads, N, Sv, d).transpose(1, 2, 0, 3).reshape(N, Sv, C)


def test_softmax_weights_sum_to_one():
    rng = np.random.default_rng(20)
    N, K, C, H = 30, 12, 16, 4
    h = rng.standard_normal((N, 9, C))
    idx, mask = _random_graph(rng, N, K)
    e_row, _, alpha = attention_weights(h, idx, mask, H)
    z = np.zeros((N, H))
    np.add.at(z, e_row, alpha)
    np.testing.assert_allclose(z, 1.0, atol=1e-12)
    # equal logits give uniform weights
    h0 = h.copy()
    h0[:, 0, :] = 0.0
    e_row, _, alpha = attention_weights(h0, idx, mask, H)
    cnt = np.bincount(e_row, minlength=N)
    np.testing.assert_allclose(alpha, np.broadcast_to(1.0 / cnt[e_row][:, None], alpha.shape), atol=1e-14)


def test_lmax0_reduces_to_sdpa():
    rng = np.random.default_rng(21)
    N, K, C, H = 40, 10, 32, 4
    pos = rng.standard_normal((N, 3)) * 5
    h = rng.standard_normal((N, 1, C))
    idx, mask = _random_graph(rng, N, K)
    out = attn_forward(pos, h, idx, mask, H, 0)
    ref = _sdpa(h[:, 0, :], h, idx, mask, H, 1 / math.sqrt(C // H))
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_origin_positions_reduce_to_sdpa_on_every_component():
    """With all atoms at r = 0 both couplings are the identity; V spans all rows."""
    rng = np.random.default_rng(22)
    N, K, C, H, lmax = 32, 9, 24, 3, 2
    h = rng.standard_normal((N, 9, C))
    idx, mask = _random_graph(rng, N, K)
    out, msg = attn_forward(np.zeros((N, 3)), h, idx, mask, H, lmax, return_msg=True)
    ref = _sdpa(h[:, 0, :], h, idx, mask, H, 1 / math.sqrt(C // H))
    np.testing.assert_allclose(msg, ref, atol=1e-12)
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_source_and_target_harmonics_are_the_right_atoms():
    """Step 1 uses each source's own r_j, step 3 the target's own r_i."""
    rng = np.random.default_rng(23)
    N, K, C, H, lmax = 30, 8, 16, 2, 2
    h = rng.standard_normal((N, 9, C))
    pos = rng.standard_normal((N, 3)) * 3
    idx, mask = _random_graph(rng, N, K)
    scale = 1 / math.sqrt(C // H)
    # targets 0..9 sit at the origin, sources elsewhere: out_i = sum_j a_ij (h_j (x) R(r_j))
    p1 = pos.copy()
    p1[:10] = 0.0
    out = attn_forward(p1, h, idx, mask, H, lmax, targets=np.arange(10))
    ref = _sdpa(h[:, 0, :], tp.tp_dense(h, p1, lmax), idx, mask, H, scale)[:10]
    np.testing.assert_allclose(out, ref, atol=1e-10 * np.abs(ref).max())
    # only atom 5 away from the origin: its sources are all at r = 0, so
    # out_5 = (sum_j a_5j h_j) (x) R(r_5)
    pos2 = np.zeros((N, 3))
    pos2[5] = [1.0, -2.0, 0.5]
    m_ref = _sdpa(h[:, 0, :], h, idx, mask, H, scale)
    # sources of target 5 are at the origin unless they are atom 5 itself (never listed)
    out5 = attn_forward(pos2, h, idx, mask, H, lmax, targets=np.array([5]))
    np.testing.assert_allclose(out5[0], tp.tp_dense(m_ref[5:6], pos2[5:6], lmax)[0],
                               atol=1e-10 * np.abs(out5).max())


def test_attention_equivariant_and_permutation():
    rng = np.random.default_rng(24)
    N, K, C, H, lmax = 28, 10, 16, 2, 2
    h = rng.standard_normal((N, 9, C))
    pos = rng.standard_normal((N, 3)) * 3
    idx, mask = _random_graph(rng, N, K)
    out = attn_forward(pos, h, idx, mask, H, lmax)
    R = wigner.random_rotation(rng)
    D = wigner.wigner_d_full(lmax, R)
    out_r = attn_forward(pos @ R.T, np.einsum("ab,nbc->nac", D, h), idx, mask, H, lmax)
    np.testing.assert_allclose(out_r, np.einsum("ab,nbc->nac", D, out), atol=1e-10 * np.abs(out).max())
    perm = rng.permutation(N)
    inv = np.argsort(perm)
    idx_p = np.where(mask[perm] != 0, inv[np.maximum(idx[perm], 0)], -1).astype(np.int32)
    out_p = attn_forward(pos[perm], h[perm], idx_p, mask[perm], H, lmax)
    np.testing.assert_allclose(out_p, out[perm], atol=1e-12 * np.abs(out).max())


def test_masked_slots_ignored_and_empty_rows_zero():
    rng = np.random.default_rng(25)
    N, K, C, H, lmax = 20, 8, 8, 2, 1
    h = rng.standard_normal((N, 4, C))
    pos = rng.standard_normal((N, 3))
    idx, mask = _random_graph(rng, N, K, allow_empty=True)
    mask[3] = 0
    out = attn_forward(pos, h, idx, mask, H, lmax)
    idx_g = np.where(mask != 0, idx, rng.integers(-10**6, 10**6, size=idx.shape)).astype(np.int32)
    out_g = attn_forward(pos, h, idx_g, mask, H, lmax)
    assert np.array_equal(out, out_g)
    assert np.all(out[3] == 0.0)
    sub = attn_forward(pos, h, idx, mask, H, lmax, targets=np.array([7, 3, 1]))
    np.testing.assert_array_equal(sub, out[[7, 3, 1]])


# ------------------------------------------------------- learned projections

def _torch_mha(x_qk, x_v, idx, mask, heads, w_q, w_k, w_v):
    """torch's multi-head attention with separate input projections and an identity output map.

    torch's linear maps compute x @ weight.T, so the oracle's right-multiplied weights
    go in transposed; a transposed operand on the oracle side fails this comparison.
    """
    import torch
    N, C = x_qk.shape
    adj = np.zeros((N, N), dtype=bool)
    rows = np.repeat(np.arange(N), idx.shape[1])
    ok = mask.ravel() != 0
    adj[rows[ok], idx.ravel()[ok]] = True
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))  # noqa: E731
    out, _ = torch.nn.functional.multi_head_attention_forward(
        t(x_qk)[:, None, :], t(x_qk)[:, None, :], t(x_v)[:, None, :], C, heads,
        in_proj_weight=None, in_proj_bias=None, bias_k=None, bias_v=None, add_zero_attn=False,
        dropout_p=0.0, out_proj_weight=torch.eye(C, dtype=torch.float64), out_proj_bias=None,
        training=False, need_weights=False, attn_mask=torch.from_numpy(~adj),
        use_separate_proj_weight=True, q_proj_weight=t(w_q.T), k_proj_weight=t(w_k.T),
        v_proj_weight=t(w_v.T))
    return out[:, 0, :].numpy()


def _weights(rng, lmax, C):
    return (rng.standard_normal((C, C)) / math.sqrt(C), rng.standard_normal((C, C)) / math.sqrt(C),
            rng.standard_normal((lmax + 1, C, C)) / math.sqrt(C))


def test_projections_lmax0_match_torch_mha():
    rng = np.random.default_rng(26)
    N, K, C, H = 36, 10, 32, 4
    pos = rng.standard_normal((N, 3)) * 4
    h = rng.standard_normal((N, 1, C))
    idx, mask = _random_graph(rng, N, K)
    wq, wk, wv = _weights(rng, 0, C)
    out = attn_forward(pos, h, idx, mask, H, 0, proj=(wq, wk, wv))
    ref = _torch_mha(h[:, 0, :], h[:, 0, :], idx, mask, H, wq, wk, wv[0])
    np.testing.assert_allclose(out[:, 0, :], ref, atol=1e-12 * np.abs(ref).max())


def test_projections_at_origin_match_torch_mha_per_component():
    """All atoms at r = 0: each component s is multi-head attention over v = h[:, s] W_V[l(s)]."""
    rng = np.random.default_rng(27)
    N, K, C, H, lmax = 30, 9, 16, 2, 2
    h = rng.standard_normal((N, 9, C))
    idx, mask = _random_graph(rng, N, K)
    wq, wk, wv = _weights(rng, lmax, C)
    out = attn_forward(np.zeros((N, 3)), h, idx, mask, H, lmax, proj=(wq, wk, wv))
    for s in range(9):
        l = int(math.isqrt(s))
        ref = _torch_mha(h[:, 0, :], h[:, s, :], idx, mask, H, wq, wk, wv[l])
        np.testing.assert_allclose(out[:, s, :], ref, atol=1e-12 * np.abs(ref).max())


def test_projections_keep_equivariance_and_identity_weights_change_nothing():
    rng = np.random.default_rng(28)
    N, K, C, H, lmax = 24, 8, 16, 2, 2
    h = rng.standard_normal((N, 9, C))
    pos = rng.standard_normal((N, 3)) * 3
    idx, mask = _random_graph(rng, N, K)
    w = _weights(rng, lmax, C)
    out = attn_forward(pos, h, idx, mask, H, lmax, proj=w)
    R = wigner.random_rotation(rng)
    D = wigner.wigner_d_full(lmax, R)
    out_r = attn_forward(pos @ R.T, np.einsum("ab,nbc->nac", D, h), idx, mask, H, lmax, proj=w)
    np.testing.assert_allclose(out_r, np.einsum("ab,nbc->nac", D, out), atol=1e-10 * np.abs(out).max())
    eye = np.eye(C)
    same = attn_forward(pos, h, idx, mask, H, lmax, proj=(eye, eye, np.stack([eye] * 3)))
    np.testing.assert_allclose(same, attn_forward(pos, h, idx, mask, H, lmax), atol=1e-13)
