"""GPU parity of the learned projections (MFMA, fused with the pre-coupling) against the oracle.

The oracle (oracle.attn.project / attn_forward(proj=...)) computes q = h[l=0] W_Q,
k = h[l=0] W_K and v[l] = h[l] W_V[l] in float64; bf16 cases feed it the same
bf16-rounded features and weights the GPU reads.  Tolerances as for the path
without projections: 1e-4 (fp32), 2e-2 (bf16 storage, fp32 accumulation).
"""

import sys

import numpy as np
import pytest

from gen import bf16_bits_to_f32, f32_to_bf16_bits, make_config, proj_weights
from oracle import tp
from oracle.attn import attn_forward as oracle_attn
from oracle.attn import project as oracle_project
from tests.helpers import TOL_BF16, TOL_F32, block_rel_err, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def e2f():
    import interatomic_potentials_amd as m
    return m


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def T(x, dev, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    return t if dtype is None else t.to(dtype)


def _r256(n):
    return (n + 255) // 256 * 256


def _inputs(rng, N, lmax, C, dt):
    S = (lmax + 1) ** 2
    pos = (rng.standard_normal((N, 3)) * 4).astype(np.float32)
    pos[0] = 0.0                                           # an atom at the origin
    h = rng.standard_normal((N, S, C)).astype(np.float32)
    if dt == "bf16":
        h = bf16_bits_to_f32(f32_to_bf16_bits(h))
    return pos, h


def _tdt(dt):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def _weights_dev(w, dev, dt):
    return tuple(T(x, dev, _tdt(dt)) for x in w)


CASES = [(0, 16, "f32"), (1, 32, "f32"), (2, 64, "f32"), (2, 128, "f32"), (1, 128, "f32"),
         (2, 16, "f32"), (2, 32, "bf16"), (1, 64, "bf16"), (2, 128, "bf16"), (0, 128, "bf16"),
         # widths the matrix-core kernel is not built for: the vector-ALU kernel
         (2, 48, "f32"), (2, 96, "f32"), (1, 80, "bf16"), (2, 256, "f32"), (2, 16, "bf16"),
         (0, 48, "bf16"), (2, 20, "f32")]


@pytest.mark.parametrize("lmax,C,dt", CASES)
@pytest.mark.parametrize("N", [1, 5, 16, 77])
def test_projected_workspace_rows_vs_oracle(e2f, dev, lmax, C, dt, N):
    """q rows, k row and h' rows of the workspace; N covers one partial tile, exact tiles, a tail."""
    say(f"projected precouple: lmax={lmax} C={C} {dt} N={N}")
    rng = np.random.default_rng(lmax * 100 + C + N)
    S = (lmax + 1) ** 2
    pos, h = _inputs(rng, N, lmax, C, dt)
    w = proj_weights(lmax, C, seed=C + lmax, dtype=dt)
    ws = e2f.attn_precouple(T(pos, dev), T(h, dev, _tdt(dt)), proj=_weights_dev(w, dev, dt))
    torch.cuda.synchronize()
    b = 2 if dt == "bf16" else 4
    rows = ws[:N * (S + 1) * C * b].view(_tdt(dt)).reshape(N, S + 1, C)
    qoff = _r256(N * (S + 1) * C * b)
    q = ws[qoff:qoff + N * C * b].view(_tdt(dt)).reshape(N, 1, C)
    rq, rk, rv = oracle_project(h, *w)
    ref_hp = tp.tp_dense(rv, pos, lmax)
    tol = TOL_BF16 if dt == "bf16" else TOL_F32
    assert block_rel_err(to_host(q), rq[:, None, :], 0) <= tol
    assert block_rel_err(to_host(rows[:, :1]), rk[:, None, :], 0) <= tol
    assert block_rel_err(to_host(rows[:, 1:]), ref_hp, lmax) <= tol


@pytest.mark.parametrize("lmax,C,dt", [(2, 128, "bf16"), (2, 64, "f32"), (1, 64, "bf16"),
                                        (2, 32, "f32")])
def test_projected_workspace_rows_many_tiles(e2f, dev, lmax, C, dt):
    """Enough atoms (20,003: 1,251 tiles of 16, the last partial) that each persistent
    workgroup runs several tiles, so every tile's rows come from the register sets
    loaded one or two tile periods ahead."""
    N = 20003
    say(f"projected precouple, many tiles: lmax={lmax} C={C} {dt} N={N}")
    rng = np.random.default_rng(lmax * 100 + C + 7)
    S = (lmax + 1) ** 2
    pos, h = _inputs(rng, N, lmax, C, dt)
    w = proj_weights(lmax, C, seed=C + lmax + 1, dtype=dt)
    ws = e2f.attn_precouple(T(pos, dev), T(h, dev, _tdt(dt)), proj=_weights_dev(w, dev, dt))
    torch.cuda.synchronize()
    b = 2 if dt == "bf16" else 4
    rows = ws[:N * (S + 1) * C * b].view(_tdt(dt)).reshape(N, S + 1, C)
    qoff = _r256(N * (S + 1) * C * b)
    q = ws[qoff:qoff + N * C * b].view(_tdt(dt)).reshape(N, 1, C)
    rq, rk, rv = oracle_project(h, *w)
    ref_hp = tp.tp_dense(rv, pos, lmax)
    tol = TOL_BF16 if dt == "bf16" else TOL_F32
    assert block_rel_err(to_host(q), rq[:, None, :], 0) <= tol
    assert block_rel_err(to_host(rows[:, :1]), rk[:, None, :], 0) <= tol
    assert block_rel_err(to_host(rows[:, 1:]), ref_hp, lmax) <= tol


@pytest.mark.parametrize("lmax,C,H,dt,K", [(0, 16, 2, "f32", 12), (1, 32, 4, "f32", 40),
                                           (2, 128, 16, "f32", 64), (2, 64, 8, "f32", 300),
                                           (2, 128, 16, "bf16", 64), (1, 64, 8, "bf16", 30)])
def test_projected_attention_vs_oracle(e2f, dev, lmax, C, H, dt, K):
    say(f"projected attention: lmax={lmax} C={C} H={H} {dt} K={K}")
    rng = np.random.default_rng(5000 + lmax * 100 + C + K)
    N = 130
    pos, h = _inputs(rng, N, lmax, C, dt)
    idx = rng.integers(0, N, size=(N, K)).astype(np.int32)
    mask = (rng.random((N, K)) < 0.6).astype(np.uint8)
    mask[9] = 0                                            # a target with no valid slot
    w = proj_weights(lmax, C, seed=7 + C, dtype=dt)
    out, msg = e2f.attn_forward(T(pos, dev), T(h, dev, _tdt(dt)), T(idx, dev), T(mask, dev), H,
                                return_msg=True, proj=_weights_dev(w, dev, dt))
    ref, ref_msg = oracle_attn(pos, h, idx, mask, H, lmax, return_msg=True, proj=w)
    tol = TOL_BF16 if dt == "bf16" else TOL_F32
    assert block_rel_err(to_host(msg), ref_msg, lmax) <= tol
    assert block_rel_err(to_host(out), ref, lmax) <= tol
    assert (out[9].float() == 0).all()


@pytest.mark.parametrize("name", ["tiny", "water"])
def test_projected_small_configs_full(e2f, dev, name):
    cfg = make_config(name)
    s = cfg.spec
    say(f"projected attention {name}: N={cfg.N} E={cfg.nl.n_edges}")
    w = proj_weights(s.lmax, s.C, seed=11)
    out, msg = e2f.attn_forward(T(cfg.pos, dev), T(cfg.h, dev), T(cfg.idx, dev), T(cfg.mask, dev),
                                s.H, return_msg=True, proj=_weights_dev(w, dev, "f32"))
    ref, ref_msg = oracle_attn(cfg.pos, cfg.h, cfg.idx, cfg.mask, s.H, s.lmax, return_msg=True,
                               chunk_edges=4096, proj=w)
    assert block_rel_err(to_host(msg), ref_msg, s.lmax) <= TOL_F32
    assert block_rel_err(to_host(out), ref, s.lmax) <= TOL_F32


@pytest.mark.parametrize("name", ["large", "scaleout"])
def test_projected_big_configs_sampled(e2f, dev, name):
    """Full sizes in the launch configuration the benchmark times; sampled targets."""
    cfg = make_config(name)
    s = cfg.spec
    say(f"projected attention {name}: N={cfg.N} K={s.K} {s.dtype} (sampled targets)")
    w = proj_weights(s.lmax, s.C, seed=13, dtype=s.dtype)
    out, msg = e2f.attn_forward(T(cfg.pos, dev), T(cfg.h, dev, _tdt(s.dtype)), T(cfg.idx, dev),
                                T(cfg.mask, dev), s.H, return_msg=True,
                                proj=_weights_dev(w, dev, s.dtype))
    torch.cuda.synchronize()
    rng = np.random.default_rng(17)
    tg = np.unique(np.concatenate([rng.choice(cfg.N, 64, replace=False), [0, cfg.N - 1]]))
    tgt = torch.from_numpy(tg).to(dev)
    ref, ref_msg = oracle_attn(cfg.pos, cfg.h, cfg.idx, cfg.mask, s.H, s.lmax, targets=tg,
                               return_msg=True, chunk_edges=4096, proj=w)
    tol = TOL_BF16 if s.dtype == "bf16" else TOL_F32
    assert block_rel_err(to_host(msg[tgt]), ref_msg, s.lmax) <= tol
    assert block_rel_err(to_host(out[tgt]), ref, s.lmax) <= tol
    assert torch.isfinite(out.float()).all()


def test_identity_weights_reproduce_the_unprojected_path(e2f, dev):
    cfg = make_config("water")
    s = cfg.spec
    say("identity projections vs no projections")
    eye = torch.eye(s.C, device=dev)
    proj = (eye, eye.clone(), eye.expand(s.lmax + 1, s.C, s.C).contiguous())
    args = (T(cfg.pos, dev), T(cfg.h, dev), T(cfg.idx, dev), T(cfg.mask, dev), s.H)
    a = e2f.attn_forward(*args, proj=proj)
    b = e2f.attn_forward(*args)
    assert block_rel_err(to_host(a), to_host(b), s.lmax) <= 1e-6


def test_unsupported_projection_width_is_reported(e2f, dev):
    h = torch.zeros((4, 9, 2048), device=dev)
    w = torch.zeros((2048, 2048), device=dev)
    with pytest.raises(e2f.E2FError) as ei:
        e2f.attn_precouple(torch.zeros((4, 3), device=dev), h,
                           proj=(w, w, torch.zeros((3, 2048, 2048), device=dev)))
    assert ei.value.name == "E2F_ERR_UNSUPPORTED"
