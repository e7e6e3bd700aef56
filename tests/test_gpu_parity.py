"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerances (max block-relative error, see helpers.block_rel_err): 1e-4 for
fp32 storage, 2e-2 for bf16 storage with fp32 arithmetic.  Integer work (which
slots are used, masking, empty rows, permutations) is checked bit-exactly.
"""

import math
import sys

import numpy as np
import pytest

from gen import bf16_bits_to_f32, f32_to_bf16_bits, make_config, make_micro
from oracle import tp
from oracle import wigner as owig
from oracle.attn import attn_forward as oracle_attn
from tests.helpers import TOL_BF16, TOL_F32, block_rel_err, head_rel_err, to_host

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


# ------------------------------------------------------------------ frames

def test_frames_match_oracle(e2f, dev):
    say("frames: 500 vectors incl. axis and zero cases")
    rng = np.random.default_rng(0)
    r = (rng.standard_normal((500, 3)) * 20).astype(np.float32)
    r[0] = [0, 0, 3]
    r[1] = [0, 0, -2]
    r[2] = [0, 0, 0]
    r[3] = [1e-20, 0, 1]
    Q, D = e2f.frames(T(r, dev), 2)
    Q = Q.cpu().numpy().astype(np.float64).reshape(-1, 3, 3)
    D = D.cpu().numpy().astype(np.float64)
    for a in range(r.shape[0]):
        assert abs(np.linalg.det(Q[a]) - 1.0) < 1e-6           # write-up section 5.2 bound
        np.testing.assert_allclose(Q[a] @ Q[a].T, np.eye(3), atol=1e-6)
        n = np.linalg.norm(r[a].astype(np.float64))
        if n > 0:
            np.testing.assert_allclose(Q[a] @ (r[a] / n), [0, 0, 1], atol=2e-6)
        np.testing.assert_allclose(Q[a], owig.alignment_rotation(r[a]), atol=2e-6)
        # D blocks equal the oracle's Wigner-D of the kernel's own Q
        assert abs(D[a, 0] - 1.0) < 1e-7
        np.testing.assert_allclose(D[a, 1:10].reshape(3, 3), owig.wigner_d(1, Q[a]), atol=2e-6)
        np.testing.assert_allclose(D[a, 10:35].reshape(5, 5), owig.wigner_d(2, Q[a]), atol=2e-6)


# -------------------------------------------------------------------- EAAS

@pytest.mark.parametrize("lmax,C,n", [(0, 16, 37), (1, 16, 37), (2, 128, 37), (2, 5, 9),
                                      (2, 6, 300), (1, 128, 1), (2, 300, 17)])
def test_eaas_each_path_fp32(e2f, dev, lmax, C, n):
    say(f"eaas per path: lmax={lmax} C={C} n={n}")
    rng = np.random.default_rng(100 + lmax * 7 + C + n)
    S = (lmax + 1) ** 2
    r = (rng.standard_normal((n, 3)) * 6).astype(np.float32)
    r[0] = [0, 0, 0]
    if n > 2:
        r[1] = [0, 0, -4.0]
    h = rng.standard_normal((n, S, C)).astype(np.float32)
    P = len(tp.paths(lmax))
    for p in range(P):
        w = np.zeros(P, np.float32)
        w[p] = 1.0
        got = to_host(e2f.eaas_couple(T(r, dev), T(h, dev), path_w=w))
        ref = tp.tp_dense(h, r, lmax, w)
        err = block_rel_err(got, ref, lmax)
        assert err <= TOL_F32, (tp.paths(lmax)[p], err)
    w = rng.standard_normal(P).astype(np.float32)
    got = to_host(e2f.eaas_couple(T(r, dev), T(h, dev), path_w=w))
    assert block_rel_err(got, tp.tp_dense(h, r, lmax, w), lmax) <= TOL_F32


def test_eaas_in_place_and_bf16(e2f, dev):
    say("eaas in place (fp32) and bf16 storage")
    rng = np.random.default_rng(5)
    n, C, lmax = 1000, 128, 2
    r = (rng.standard_normal((n, 3)) * 30).astype(np.float32)
    h = rng.standard_normal((n, 9, C)).astype(np.float32)
    ref = tp.tp_dense(h, r, lmax)
    ht = T(h, dev)
    out = e2f.eaas_couple(T(r, dev), ht, out=ht)
    assert out.data_ptr() == ht.data_ptr()
    assert block_rel_err(to_host(out), ref, lmax) <= TOL_F32
    hb = bf16_bits_to_f32(f32_to_bf16_bits(h))
    got = e2f.eaas_couple(T(r, dev), T(hb, dev, torch.bfloat16))
    assert got.dtype == torch.bfloat16
    assert block_rel_err(to_host(got), tp.tp_dense(hb, r, lmax), lmax) <= TOL_BF16


def test_eaas_micro_workload_sampled(e2f, dev):
    """2^20 unit vectors, C = 128, all 15 paths: sampled rows against the oracle."""
    say("eaas micro workload: B=2^20, C=128, lmax=2, fp32 (sampled rows)")
    r, h, _ = make_micro()
    out = e2f.eaas_couple(T(r, dev), T(h, dev))
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = np.concatenate([rng.choice(r.shape[0], 512, replace=False), [0, r.shape[0] - 1]])
    got = out[torch.from_numpy(rows).to(dev)].cpu().numpy()
    ref = tp.tp_dense(h[rows], r[rows], 2)
    assert block_rel_err(got, ref, 2) <= TOL_F32


# --------------------------------------------------------------- attention

def run_attn(e2f, dev, cfg, h=None, idx=None, mask=None, dtype=None, return_msg=False, **kw):
    s = cfg.spec
    h = cfg.h if h is None else h
    idx = cfg.idx if idx is None else idx
    mask = cfg.mask if mask is None else mask
    dt = dtype or (torch.bfloat16 if s.dtype == "bf16" else torch.float32)
    return e2f.attn_forward(T(cfg.pos, dev), T(h, dev, dt), T(idx, dev), T(mask, dev), s.H,
                            return_msg=return_msg, **kw)


# shared: the kernels in which several targets of a wave share rows, forced at these sizes
# (by default they run above 4,096 atoms only)
@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("name", ["tiny", "water"])
def test_attention_small_configs_full(e2f, dev, name, shared):
    cfg = make_config(name)
    s = cfg.spec
    say(f"attention {name}: N={cfg.N} K={s.K} lmax={s.lmax} C={s.C} H={s.H} E={cfg.nl.n_edges} "
        f"shared rows {shared}")
    out, msg = run_attn(e2f, dev, cfg, return_msg=True, shared_rows=shared)
    ref, ref_msg = oracle_attn(cfg.pos, cfg.h, cfg.idx, cfg.mask, s.H, s.lmax, return_msg=True,
                               chunk_edges=4096)
    assert block_rel_err(to_host(msg), ref_msg, s.lmax) <= TOL_F32
    assert block_rel_err(to_host(out), ref, s.lmax) <= TOL_F32
    # the stricter per-head metric: the message's heads are independent softmaxes
    assert head_rel_err(to_host(msg), ref_msg, s.lmax, s.H) <= TOL_F32


def _sample_targets(cfg, n, seed):
    rng = np.random.default_rng(seed)
    nv = cfg.mask.sum(1)
    pick = set(rng.choice(cfg.N, n, replace=False).tolist())
    pick |= {int(nv.argmin()), int(nv.argmax()), 0, cfg.N - 1}
    return np.array(sorted(pick))


@pytest.mark.parametrize("name", ["large", "scaleout"])
def test_attention_big_configs_sampled(e2f, dev, name):
    cfg = make_config(name)
    s = cfg.spec
    say(f"attention {name}: N={cfg.N} K={s.K} lmax={s.lmax} C={s.C} H={s.H} dtype={s.dtype} "
        f"E={cfg.nl.n_edges} (sampled targets)")
    out, msg = run_attn(e2f, dev, cfg, return_msg=True)
    torch.cuda.synchronize()
    tg = _sample_targets(cfg, 96, 7)
    tgt = torch.from_numpy(tg).to(dev)
    got, got_msg = to_host(out[tgt]), to_host(msg[tgt])
    ref, ref_msg = oracle_attn(cfg.pos, cfg.h, cfg.idx, cfg.mask, s.H, s.lmax, targets=tg,
                               return_msg=True, chunk_edges=4096)
    tol = TOL_BF16 if s.dtype == "bf16" else TOL_F32
    assert block_rel_err(got_msg, ref_msg, s.lmax) <= tol
    assert block_rel_err(got, ref, s.lmax) <= tol
    assert head_rel_err(got_msg, ref_msg, s.lmax, s.H) <= tol
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("lmax,C,H,K", [(0, 32, 4, 10), (1, 16, 2, 32), (2, 64, 4, 300),
                                        (2, 128, 16, 64), (1, 8, 8, 7), (2, 256, 8, 40),
                                        (2, 128, 16, 300), (2, 96, 12, 300)])
@pytest.mark.parametrize("shared", [False, True])
def test_attention_shapes_vs_oracle(e2f, dev, lmax, C, H, K, shared):
    """Ragged sizes: K not a multiple of 64, K above one LDS tile, d = 1, 16, 32."""
    say(f"attention shapes: lmax={lmax} C={C} H={H} K={K} shared rows {shared}")
    rng = np.random.default_rng(lmax * 1000 + C + K)
    N = 150
    S = (lmax + 1) ** 2
    pos = (rng.standard_normal((N, 3)) * 4).astype(np.float32)
    h = rng.standard_normal((N, S, C)).astype(np.float32)
    idx = rng.integers(0, N, size=(N, K)).astype(np.int32)
    mask = (rng.random((N, K)) < 0.7).astype(np.uint8)
    mask[5] = 0                                    # a target with no valid slot
    out, msg = e2f.attn_forward(T(pos, dev), T(h, dev), T(idx, dev), T(mask, dev), H,
                                return_msg=True, shared_rows=shared)
    ref, ref_msg = oracle_attn(pos, h, idx, mask, H, lmax, return_msg=True)
    assert block_rel_err(to_host(msg), ref_msg, lmax) <= TOL_F32
    assert block_rel_err(to_host(out), ref, lmax) <= TOL_F32
    assert (out[5] == 0).all() and (msg[5] == 0).all()


def test_attention_bf16_small_vs_oracle(e2f, dev):
    cfg = make_config("scaleout", n_atoms=3000)
    s = cfg.spec
    say(f"attention bf16 small: N={cfg.N} K={s.K} E={cfg.nl.n_edges}")
    out, msg = run_attn(e2f, dev, cfg, return_msg=True)
    assert out.dtype == torch.bfloat16
    ref, ref_msg = oracle_attn(cfg.pos, cfg.h, cfg.idx, cfg.mask, s.H, s.lmax, return_msg=True,
                               chunk_edges=4096)
    assert block_rel_err(to_host(msg), ref_msg, s.lmax) <= TOL_BF16
    assert block_rel_err(to_host(out), ref, s.lmax) <= TOL_BF16


def test_aggregate_with_given_values(e2f, dev):
    """Stream only: a hand-filled workspace (k rows and v = 1) gives m = 1 for every target."""
    cfg = make_config("tiny")
    s = cfg.spec
    say("aggregate with v = 1")
    N, S, C = cfg.N, 4, s.C
    ws_np = np.ones((N, S + 1, C), np.float32)
    ws_np[:, 0, :] = cfg.h[:, 0, :]
    ws = torch.zeros(e2f.attn_workspace_bytes(N, s.lmax, C), dtype=torch.uint8, device=dev)
    ws[: ws_np.nbytes].copy_(T(ws_np.view(np.uint8).reshape(-1), dev))
    q_np = np.ascontiguousarray(cfg.h[:, 0, :], dtype=np.float32)   # query rows after the k/v rows
    qoff = (ws_np.nbytes + 255) // 256 * 256
    ws[qoff: qoff + q_np.nbytes].copy_(T(q_np.view(np.uint8).reshape(-1), dev))
    out, msg = e2f.attn_aggregate(T(cfg.pos, dev), T(cfg.idx, dev), T(cfg.mask, dev), ws, s.H,
                                  s.lmax, C, torch.float32, return_msg=True)
    m = msg.cpu().numpy()
    np.testing.assert_allclose(m, 1.0, atol=1e-6)
    ref = tp.tp_dense(np.ones((N, S, C)), cfg.pos, s.lmax)
    assert block_rel_err(to_host(out), ref, s.lmax) <= TOL_F32


# ----------------------------------------------- integer path, bit-exact

@pytest.mark.parametrize("shared", [False, True])
def test_mask_semantics_bit_exact(e2f, dev, shared):
    """Masked slots are never read; out-of-range indices at valid slots are skipped."""
    cfg = make_config("water")
    s = cfg.spec
    say(f"mask semantics on water, shared rows {shared}")
    kw = {"shared_rows": shared}
    base = run_attn(e2f, dev, cfg, **kw).cpu()
    rng = np.random.default_rng(3)
    # poison every masked slot with garbage / out-of-range indices
    idx_p = np.where(cfg.mask != 0, cfg.idx, rng.integers(-2**31, 2**31 - 1, size=cfg.idx.shape)
                     ).astype(np.int32)
    poisoned = run_attn(e2f, dev, cfg, idx=idx_p, **kw).cpu()
    assert torch.equal(base, poisoned)
    # a NaN atom that only appears behind masked slots changes nothing
    N = cfg.N
    extra_h = np.concatenate([cfg.h, np.full((1,) + cfg.h.shape[1:], np.nan, np.float32)])
    extra_pos = np.concatenate([cfg.pos, np.zeros((1, 3), np.float32)])
    extra_idx = np.concatenate([np.where(cfg.mask != 0, cfg.idx, N), np.zeros((1, s.K), np.int32)])
    extra_mask = np.concatenate([cfg.mask, np.zeros((1, s.K), np.uint8)])
    out = e2f.attn_forward(T(extra_pos, dev), T(extra_h, dev), T(extra_idx.astype(np.int32), dev),
                           T(extra_mask, dev), s.H, **kw).cpu()
    assert torch.equal(out[:N], base)
    assert (out[N] == 0).all()
    # all-masked targets give exact zeros
    m2 = cfg.mask.copy()
    m2[::7] = 0
    out2 = run_attn(e2f, dev, cfg, mask=m2, **kw).cpu()
    assert (out2[::7] == 0).all()
    # an out-of-range index at a valid slot is skipped, or reported under validation
    idx_bad = cfg.idx.copy()
    row = int(np.argmax(cfg.mask.sum(1)))
    idx_bad[row, 0] = N + 5
    m3 = cfg.mask.copy()
    m3[row, 0] = 0
    skipped = run_attn(e2f, dev, cfg, idx=idx_bad, **kw).cpu()
    masked = run_attn(e2f, dev, cfg, mask=m3, **kw).cpu()
    assert torch.equal(skipped, masked)
    with pytest.raises(e2f.E2FError) as ei:
        run_attn(e2f, dev, cfg, idx=idx_bad, validate=True, **kw)
    assert ei.value.name == "E2F_ERR_INDEX"
    ok = run_attn(e2f, dev, cfg, validate=True, **kw).cpu()
    assert torch.equal(ok, base)


@pytest.mark.parametrize("shared", [False, True])
def test_slot_order_and_layout_invariance(e2f, dev, shared):
    cfg = make_config("water")
    s = cfg.spec
    say(f"slot shuffle, atom permutation, run twice, shared rows {shared}")
    kw = {"shared_rows": shared}
    base = run_attn(e2f, dev, cfg, **kw).cpu()
    again = run_attn(e2f, dev, cfg, **kw).cpu()
    assert torch.equal(base, again)                   # deterministic: no atomics
    rng = np.random.default_rng(11)
    # shuffled slots (valid slots scattered through the row): the kernel visits a
    # target's neighbours in atom-index order, so the result is bit-identical
    perm_slots = np.argsort(rng.random(cfg.idx.shape), axis=1)
    idx_s = np.take_along_axis(cfg.idx, perm_slots, 1)
    mask_s = np.take_along_axis(cfg.mask, perm_slots, 1)
    shuf = run_attn(e2f, dev, cfg, idx=idx_s, mask=mask_s, **kw).cpu()
    assert torch.equal(shuf, base)
    # atom relabelling with remapped indices: same neighbour sets, visited in
    # another order, so equal up to rounding (a wrong neighbour would be O(1))
    perm = rng.permutation(cfg.N)
    inv = np.argsort(perm)
    idx_p = np.where(cfg.mask[perm] != 0, inv[np.maximum(cfg.idx[perm], 0)], -1).astype(np.int32)
    out_p = e2f.attn_forward(T(cfg.pos[perm], dev), T(cfg.h[perm], dev), T(idx_p, dev),
                             T(cfg.mask[perm], dev), s.H, **kw).cpu()
    assert block_rel_err(to_host(out_p), to_host(base[torch.from_numpy(perm)]), s.lmax) <= 1e-5


def test_rotation_equivariance_on_gpu(e2f, dev):
    cfg = make_config("water")
    s = cfg.spec
    say("rotation equivariance on water")
    R = owig.random_rotation(np.random.default_rng(42))
    D = owig.wigner_d_full(s.lmax, R)
    out = to_host(run_attn(e2f, dev, cfg))
    h_r = np.einsum("ab,nbc->nac", D, cfg.h).astype(np.float32)
    pos_r = (cfg.pos.astype(np.float64) @ R.T).astype(np.float32)
    out_r = to_host(e2f.attn_forward(T(pos_r, dev), T(h_r, dev), T(cfg.idx, dev),
                                     T(cfg.mask, dev), s.H))
    assert block_rel_err(out_r, np.einsum("ab,nbc->nac", D, out), s.lmax) <= 1e-5


def test_empty_and_single_atom(e2f, dev):
    say("N = 0 and N = 1")
    z = torch.zeros((0, 9, 128), device=dev)
    out = e2f.attn_forward(torch.zeros((0, 3), device=dev), z,
                           torch.zeros((0, 8), dtype=torch.int32, device=dev),
                           torch.zeros((0, 8), dtype=torch.uint8, device=dev), 16)
    assert out.shape == (0, 9, 128)
    h = torch.randn((1, 9, 128), device=dev)
    out = e2f.attn_forward(torch.ones((1, 3), device=dev), h,
                           torch.full((1, 8), -1, dtype=torch.int32, device=dev),
                           torch.zeros((1, 8), dtype=torch.uint8, device=dev), 16)
    assert (out == 0).all()


@pytest.mark.parametrize("name", ["water", "large", "scaleout"])
def test_schedule_covers_every_target_bit_exact(e2f, dev, name):
    """The spatial schedule only reorders work: same bits as index order, every target written."""
    cfg = make_config(name)
    s = cfg.spec
    say(f"schedule vs index order on {name}")
    dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    pos, h = T(cfg.pos, dev), T(cfg.h, dev, dt)
    idx, mask = T(cfg.idx, dev), T(cfg.mask, dev)
    a = torch.full_like(h, float("nan"))
    b = torch.full_like(h, float("nan"))
    e2f.attn_forward(pos, h, idx, mask, s.H, out=a)
    e2f.attn_forward(pos, h, idx, mask, s.H, out=b, targets_in_order=True)
    assert torch.isfinite(a).all() and torch.isfinite(b).all()
    assert torch.equal(a, b)


@pytest.mark.parametrize("lmax,C,H,K", [(2, 128, 16, 64), (2, 128, 8, 40), (1, 64, 16, 30),
                                        (2, 8, 8, 20), (2, 512, 64, 16), (0, 16, 2, 300),
                                        (1, 128, 8, 300), (2, 128, 16, 200), (2, 96, 12, 100),
                                        (2, 64, 4, 64)])
def test_attention_bf16_shapes_vs_oracle(e2f, dev, lmax, C, H, K):
    """bf16 storage over every lane mapping: several targets a wave sharing rows (rows of up
    to 64 and up to 256 slots, 1, 2 or 4 lanes per head, idle lanes at C = 96), and one
    target a wave at 8, 4 and 1 channels per lane."""
    say(f"attention bf16 shapes: lmax={lmax} C={C} H={H} K={K}")
    rng = np.random.default_rng(7000 + lmax * 100 + C + K)
    N = 120
    S = (lmax + 1) ** 2
    pos = (rng.standard_normal((N, 3)) * 4).astype(np.float32)
    h = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal((N, S, C)).astype(np.float32)))
    idx = rng.integers(0, N, size=(N, K)).astype(np.int32)
    mask = (rng.random((N, K)) < 0.6).astype(np.uint8)
    mask[3] = 0
    out, msg = e2f.attn_forward(T(pos, dev), T(h, dev, torch.bfloat16), T(idx, dev), T(mask, dev),
                                H, return_msg=True)
    ref, ref_msg = oracle_attn(pos, h, idx, mask, H, lmax, return_msg=True)
    assert block_rel_err(to_host(msg), ref_msg, lmax) <= TOL_BF16
    assert block_rel_err(to_host(out), ref, lmax) <= TOL_BF16
    assert (out[3].float() == 0).all()


def test_unsupported_row_width_is_reported(e2f, dev):
    """Rows wider than 512 channels: a clear error, nothing launched."""
    h = torch.zeros((4, 9, 1024), device=dev)
    with pytest.raises(e2f.E2FError) as ei:
        e2f.attn_forward(torch.zeros((4, 3), device=dev), h,
                         torch.zeros((4, 2), dtype=torch.int32, device=dev),
                         torch.zeros((4, 2), dtype=torch.uint8, device=dev), 8)
    assert ei.value.name == "E2F_ERR_UNSUPPORTED"


def test_targets_sharing_a_wave_stay_independent(e2f, dev):
    """Several targets share each row they read; a row only changes the targets that list it.

    Visiting targets in index order groups consecutive atoms; a non-finite source listed by
    one target must leave its neighbours in the group bit-identical to a run without it.
    """
    cfg = make_config("water")
    s = cfg.spec
    say("shared rows: a NaN source listed by one target only")
    N = cfg.N
    h = np.concatenate([cfg.h, np.full((1,) + cfg.h.shape[1:], np.nan, np.float32)])
    pos = np.concatenate([cfg.pos, cfg.pos[1:2] + 0.5])
    idx = np.concatenate([cfg.idx, np.zeros((1, s.K), np.int32)])
    mask = np.concatenate([cfg.mask, np.zeros((1, s.K), np.uint8)])
    free = int(np.argmin(mask[1]))
    assert mask[1, free] == 0
    idx_nan, mask_nan = idx.copy(), mask.copy()
    idx_nan[1, free] = N                             # only target 1 lists the NaN atom
    mask_nan[1, free] = 1
    run = lambda i, m: e2f.attn_forward(T(pos, dev), T(h, dev), T(i, dev), T(m, dev), s.H,
                                        targets_in_order=True,
                                        shared_rows=True).cpu()  # noqa: E731
    with_nan = run(idx_nan, mask_nan)
    without = run(idx, mask)
    others = np.setdiff1d(np.arange(N + 1), [1])
    assert torch.isnan(with_nan[1]).any()
    assert torch.equal(with_nan[others], without[others])


@pytest.mark.parametrize("C,H", [(128, 16), (24, 8)])
def test_message_in_fp32_with_bf16_storage(e2f, dev, C, H):
    """E2F_MSG_F32: the message m leaves the kernel in fp32; rounded to bf16 it equals the
    bf16-stored message bit for bit (the same value, rounded once), and out is unchanged."""
    say(f"bf16 storage, message in fp32: C={C} H={H}")
    rng = np.random.default_rng(31 + C)
    N, K, lmax = 90, 48, 2
    pos = (rng.standard_normal((N, 3)) * 3).astype(np.float32)
    h = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal((N, 9, C)).astype(np.float32)))
    idx = rng.integers(0, N, size=(N, K)).astype(np.int32)
    mask = (rng.random((N, K)) < 0.6).astype(np.uint8)
    args = (T(pos, dev), T(h, dev, torch.bfloat16), T(idx, dev), T(mask, dev), H)
    p, hh, ii, mm = args[:4]
    ws = e2f.attn_precouple(p, hh)
    out_a, msg_b = e2f.attn_aggregate(p, ii, mm, ws, H, lmax, C, torch.bfloat16, return_msg=True)
    out_b, msg_f = e2f.attn_aggregate(p, ii, mm, ws, H, lmax, C, torch.bfloat16, return_msg=True,
                                      msg_f32=True)
    assert msg_f.dtype == torch.float32 and msg_b.dtype == torch.bfloat16
    assert torch.equal(out_a, out_b)
    got = f32_to_bf16_bits(msg_f.cpu().numpy())
    assert np.array_equal(got, msg_b.cpu().view(torch.int16).numpy().view(np.uint16))
    _, ref_msg = oracle_attn(pos, h, idx, mask, H, lmax, return_msg=True)
    assert block_rel_err(to_host(msg_f), ref_msg, lmax) <= TOL_BF16
