"""GPU parity of the 16-target matrix-core aggregate (E2F_MATRIX_TILES) against the oracle.

The kernel serves fp32 storage with C = 128, H = 16 and rows of at most 256 slots.  Values
are checked at the forward's tolerance (1e-4 block-relative, and per head); which slots are
used, masking, slot order, the schedule and non-finite sources are checked bit for bit:
each target's result is its own chain of fused multiply-adds over its sources in index
order, whatever other targets share its tile.
"""

import sys

import numpy as np
import pytest

from gen import make_config
from oracle.attn import attn_forward as oracle_attn
from oracle.grad import attn_backward as oracle_backward
from tests.helpers import TOL_F32, block_rel_err, head_rel_err, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

C, H = 128, 16


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def e2f():
    import interatomic_potentials_amd as m
    return m


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def T(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def ref_lse(h, idx, mask, heads):
    """natural log-sum-exp of each target's head logits over its valid slots (float64)"""
    hh = np.asarray(h, np.float64)
    N = hh.shape[0]
    d = hh.shape[2] // heads
    q = hh[:, 0, :].reshape(N, heads, d)
    out = np.full((N, heads), -np.inf)
    for i in range(N):
        js = idx[i][mask[i] != 0]
        js = js[(js >= 0) & (js < N)]
        if js.size:
            lg = (q[i][None] * q[js]).sum(-1) / np.sqrt(d)
            mx = lg.max(0)
            out[i] = mx + np.log(np.exp(lg - mx).sum(0))
    return out


def tile_forward(e2f, dev, pos, h, idx, mask, **kw):
    return e2f.attn_forward(T(pos, dev), T(h, dev), T(idx, dev), T(mask, dev), H,
                            matrix_tiles=True, **kw)


def random_graph(lmax, N, K, p, seed):
    rng = np.random.default_rng(seed)
    S = (lmax + 1) ** 2
    pos = (rng.standard_normal((N, 3)) * 4).astype(np.float32)
    h = rng.standard_normal((N, S, C)).astype(np.float32)
    idx = rng.integers(0, N, size=(N, K)).astype(np.int32)     # repeated sources included
    mask = (rng.random((N, K)) < p).astype(np.uint8)
    return pos, h, idx, mask


@pytest.mark.parametrize("lmax", [0, 1, 2])
@pytest.mark.parametrize("K", [7, 37, 64, 256])
def test_tile_random_graphs_vs_oracle(e2f, dev, lmax, K):
    """Random sources (repeats in a row weigh once per slot), K on both key-loading paths."""
    N = 150
    say(f"matrix tiles, random graph: lmax={lmax} K={K} N={N}")
    pos, h, idx, mask = random_graph(lmax, N, K, 0.7, 900 + 10 * lmax + K)
    mask[5] = 0                                                 # a target with no valid slot
    out, msg, lse = tile_forward(e2f, dev, pos, h, idx, mask, return_msg=True, return_lse=True)
    ref, ref_msg = oracle_attn(pos, h, idx, mask, H, lmax, return_msg=True)
    assert block_rel_err(to_host(msg), ref_msg, lmax) <= TOL_F32
    assert head_rel_err(to_host(msg), ref_msg, lmax, H) <= TOL_F32
    assert block_rel_err(to_host(out), ref, lmax) <= TOL_F32
    assert (out[5] == 0).all() and (msg[5] == 0).all()
    rl = ref_lse(h, idx, mask, H)
    got = lse.cpu().numpy()
    assert np.isneginf(got[5]).all()
    ok = np.isfinite(rl)
    np.testing.assert_allclose(got[ok], rl[ok], rtol=1e-5, atol=1e-5)


def test_tile_every_slot_valid(e2f, dev):
    """16 rows of 256 valid slots: 4,096 keys a tile, the most the kernel takes."""
    N, K = 64, 256
    say("matrix tiles, every slot valid (4,096 keys a tile)")
    pos, h, idx, mask = random_graph(2, N, K, 1.1, 77)
    out, msg = tile_forward(e2f, dev, pos, h, idx, mask, return_msg=True)
    ref, ref_msg = oracle_attn(pos, h, idx, mask, H, 2, return_msg=True)
    assert block_rel_err(to_host(msg), ref_msg, 2) <= TOL_F32
    assert block_rel_err(to_host(out), ref, 2) <= TOL_F32


@pytest.mark.parametrize("N", [1, 15, 17, 33, 100])
def test_tile_ragged_atom_counts(e2f, dev, N):
    """N not a multiple of the tile: absent targets add no key and store nothing."""
    say(f"matrix tiles, N={N}")
    pos, h, idx, mask = random_graph(2, N, 24, 0.6, 300 + N)
    out = tile_forward(e2f, dev, pos, h, idx, mask)
    ref = oracle_attn(pos, h, idx, mask, H, 2)
    assert block_rel_err(to_host(out), ref, 2) <= TOL_F32


def test_tile_water_full(e2f, dev):
    cfg = make_config("water")
    s = cfg.spec
    say(f"matrix tiles on water: N={cfg.N} K={s.K}")
    out, msg = tile_forward(e2f, dev, cfg.pos, cfg.h, cfg.idx, cfg.mask, return_msg=True)
    ref, ref_msg = oracle_attn(cfg.pos, cfg.h, cfg.idx, cfg.mask, s.H, s.lmax, return_msg=True,
                               chunk_edges=4096)
    assert block_rel_err(to_host(msg), ref_msg, s.lmax) <= TOL_F32
    assert head_rel_err(to_host(msg), ref_msg, s.lmax, s.H) <= TOL_F32
    assert block_rel_err(to_host(out), ref, s.lmax) <= TOL_F32
    # the same function as the other kernels, rounded in another order
    for kw in ({}, {"shared_rows": True}):
        other = e2f.attn_forward(T(cfg.pos, dev), T(cfg.h, dev), T(cfg.idx, dev),
                                 T(cfg.mask, dev), s.H, **kw)
        assert block_rel_err(to_host(out), to_host(other), s.lmax) <= 1e-5


def test_tile_bit_exact_invariances(e2f, dev):
    """Schedule, slot order, poisoned masked slots and a repeated run change no bit."""
    cfg = make_config("water")
    s = cfg.spec
    say("matrix tiles: schedule / slot order / masked-slot poison, bit for bit")
    base = tile_forward(e2f, dev, cfg.pos, cfg.h, cfg.idx, cfg.mask).cpu()
    assert torch.isfinite(base).all()
    assert torch.equal(base, tile_forward(e2f, dev, cfg.pos, cfg.h, cfg.idx, cfg.mask).cpu())
    in_order = tile_forward(e2f, dev, cfg.pos, cfg.h, cfg.idx, cfg.mask,
                            targets_in_order=True).cpu()
    assert torch.equal(base, in_order)
    rng = np.random.default_rng(11)
    perm = np.argsort(rng.random(cfg.idx.shape), axis=1)
    shuf = tile_forward(e2f, dev, cfg.pos, cfg.h, np.take_along_axis(cfg.idx, perm, 1),
                        np.take_along_axis(cfg.mask, perm, 1)).cpu()
    assert torch.equal(base, shuf)
    idx_p = np.where(cfg.mask != 0, cfg.idx,
                     rng.integers(-2**31, 2**31 - 1, size=cfg.idx.shape)).astype(np.int32)
    assert torch.equal(base, tile_forward(e2f, dev, cfg.pos, cfg.h, idx_p, cfg.mask).cpu())
    # an atom relabelling regroups the tiles: same neighbour sets, so equal up to rounding
    pa = rng.permutation(cfg.N)
    inv = np.argsort(pa)
    idx_r = np.where(cfg.mask[pa] != 0, inv[np.maximum(cfg.idx[pa], 0)], -1).astype(np.int32)
    out_r = tile_forward(e2f, dev, cfg.pos[pa], cfg.h[pa], idx_r, cfg.mask[pa]).cpu()
    assert block_rel_err(to_host(out_r), to_host(base[torch.from_numpy(pa)]), s.lmax) <= 1e-5


def test_tile_non_finite_source_reaches_its_targets_only(e2f, dev):
    """A NaN source listed by one target: every other target of its tile keeps its bits."""
    cfg = make_config("water")
    s = cfg.spec
    say("matrix tiles: a NaN source listed by one target only")
    N = cfg.N
    h = np.concatenate([cfg.h, np.full((1,) + cfg.h.shape[1:], np.nan, np.float32)])
    pos = np.concatenate([cfg.pos, cfg.pos[1:2] + 0.5])
    idx = np.concatenate([cfg.idx, np.zeros((1, s.K), np.int32)])
    mask = np.concatenate([cfg.mask, np.zeros((1, s.K), np.uint8)])
    free = int(np.argmin(mask[1]))
    assert mask[1, free] == 0
    idx_nan, mask_nan = idx.copy(), mask.copy()
    idx_nan[1, free] = N
    mask_nan[1, free] = 1
    with_nan = tile_forward(e2f, dev, pos, h, idx_nan, mask_nan, targets_in_order=True).cpu()
    without = tile_forward(e2f, dev, pos, h, idx, mask, targets_in_order=True).cpu()
    others = np.setdiff1d(np.arange(N + 1), [1])
    assert torch.isnan(with_nan[1]).any()
    assert torch.equal(with_nan[others], without[others])
    # an infinite value in a source's row behaves the same
    h_inf = h.copy()
    h_inf[N] = cfg.h[3]
    h_inf[N, 4, 17] = np.inf
    with_inf = tile_forward(e2f, dev, pos, h_inf, idx_nan, mask_nan, targets_in_order=True).cpu()
    assert not torch.isfinite(with_inf[1]).all()
    assert torch.equal(with_inf[others], without[others])


def test_tile_large_sampled(e2f, dev):
    cfg = make_config("large")
    s = cfg.spec
    say(f"matrix tiles on large: N={cfg.N} E={cfg.nl.n_edges} (sampled targets)")
    pos, h, idx, mask = T(cfg.pos, dev), T(cfg.h, dev), T(cfg.idx, dev), T(cfg.mask, dev)
    out = torch.full_like(h, float("nan"))
    msg = torch.full_like(h, float("nan"))
    lse = torch.full((cfg.N, s.H), float("nan"), device=dev)
    e2f.attn_aggregate(pos, idx, mask, e2f.attn_precouple(pos, h), s.H, s.lmax, s.C,
                       torch.float32, out=out, matrix_tiles=True)
    o2, m2, l2 = e2f.attn_forward(pos, h, idx, mask, s.H, return_msg=True, return_lse=True,
                                  matrix_tiles=True, targets_in_order=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.equal(out, o2)                        # schedule vs index order, every target
    rng = np.random.default_rng(7)
    tg = np.array(sorted(set(rng.choice(cfg.N, 96, replace=False).tolist())
                         | {0, cfg.N - 1, int(cfg.mask.sum(1).argmin())}))
    tgt = torch.from_numpy(tg).to(dev)
    ref, ref_msg = oracle_attn(cfg.pos, cfg.h, cfg.idx, cfg.mask, s.H, s.lmax, targets=tg,
                               return_msg=True, chunk_edges=4096)
    assert block_rel_err(to_host(o2[tgt]), ref, s.lmax) <= TOL_F32
    assert block_rel_err(to_host(m2[tgt]), ref_msg, s.lmax) <= TOL_F32
    assert head_rel_err(to_host(m2[tgt]), ref_msg, s.lmax, s.H) <= TOL_F32
    # log-sum-exp of the sampled targets from their own rows
    hh = cfg.h.astype(np.float64)
    d = s.C // s.H
    q = hh[:, 0, :].reshape(cfg.N, s.H, d)
    got = l2.cpu().numpy()
    for i in tg:
        js = cfg.idx[i][cfg.mask[i] != 0]
        lg = (q[i][None] * q[js]).sum(-1) / np.sqrt(d)
        mx = lg.max(0)
        np.testing.assert_allclose(got[i], mx + np.log(np.exp(lg - mx).sum(0)), rtol=1e-5,
                                   atol=1e-5)


def test_tile_forward_feeds_the_backward(e2f, dev):
    """The backward recomputes weights from the forward's log-sum-exp and message."""
    N, K, lmax = 80, 64, 2
    say("matrix tiles: forward outputs into attn_backward")
    pos, h, idx, mask = random_graph(lmax, N, K, 0.6, 55)
    mask[7] = 0
    g = np.random.default_rng(56).standard_normal(h.shape).astype(np.float32)
    p, hh, ii, mm = T(pos, dev), T(h, dev), T(idx, dev), T(mask, dev)
    ws = e2f.attn_precouple(p, hh)
    _, msg, lse = e2f.attn_aggregate(p, ii, mm, ws, H, lmax, C, torch.float32, return_msg=True,
                                     return_lse=True, matrix_tiles=True)
    gh, gp = e2f.attn_backward(p, hh, ii, mm, H, ws, msg, lse, T(g, dev))
    torch.cuda.synchronize()
    rh, rp = oracle_backward(pos, h, idx, mask, H, lmax, g)
    assert block_rel_err(gh.cpu().numpy(), rh, lmax) <= TOL_F32
    rp = np.asarray(rp, np.float64)
    nr = np.linalg.norm(rp, axis=1)
    err = np.linalg.norm(gp.cpu().numpy() - rp, axis=1) / np.maximum(nr, 1e-3 * nr.max())
    assert float(err.max()) <= TOL_F32


def test_tile_flag_ignored_where_not_served(e2f, dev):
    """Other layouts (here C = 64) run the other kernels under the flag, with the same result."""
    rng = np.random.default_rng(3)
    N, K, lmax, c, hd = 60, 20, 1, 64, 4
    pos = (rng.standard_normal((N, 3)) * 3).astype(np.float32)
    h = rng.standard_normal((N, 4, c)).astype(np.float32)
    idx = rng.integers(0, N, size=(N, K)).astype(np.int32)
    mask = (rng.random((N, K)) < 0.7).astype(np.uint8)
    a = e2f.attn_forward(T(pos, dev), T(h, dev), T(idx, dev), T(mask, dev), hd,
                         matrix_tiles=True).cpu()
    b = e2f.attn_forward(T(pos, dev), T(h, dev), T(idx, dev), T(mask, dev), hd).cpu()
    assert torch.equal(a, b)


def test_tile_allocation_free_entry_point(e2f, dev):
    """The static-workspace entry point runs the same kernel: the same bits, twice in a row."""
    cfg = make_config("water")
    s = cfg.spec
    say("matrix tiles through the allocation-free entry point")
    args = (T(cfg.pos, dev), T(cfg.h, dev), T(cfg.idx, dev), T(cfg.mask, dev), s.H)
    ref = e2f.attn_forward(*args, matrix_tiles=True)
    for _ in range(2):
        got = e2f.attn_forward_noalloc(*args, matrix_tiles=True)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)


def test_tile_graph_replay(e2f, dev):
    """The forward with matrix tiles captured in a HIP graph, replayed on new values."""
    cfg = make_config("water")
    s = cfg.spec
    say("matrix tiles: graph capture and replay")
    pos, h, idx, mask = T(cfg.pos, dev), T(cfg.h, dev), T(cfg.idx, dev), T(cfg.mask, dev)

    def step():
        return e2f.attn_forward(pos, h, idx, mask, s.H, matrix_tiles=True)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()
    rng = np.random.default_rng(4)
    for _ in range(3):
        h.copy_(T(rng.standard_normal(cfg.h.shape).astype(np.float32), dev))
        g.replay()
        torch.cuda.synchronize()
        eager = step()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
