"""Workspace rows past 4 GiB: the forward and backward kernels with 64-bit offsets.

At N = 850,000 atoms (lmax 2, C 128, fp32) the pre-coupled rows take 4.35e9 bytes,
more than the 32-bit byte offsets of the buffer-load kernels reach, so the general
kernels run.  The last M atoms form a closed subsystem: they list only each other and
no other atom lists them, so their outputs and gradients are those of an M-atom
problem that the oracle computes directly, while every one of their rows lies beyond
the first 4 GiB.  The other atoms list random atoms of the rest, so the whole grid
does work; a few of them are checked through their own small problems as well.
"""

import sys

import numpy as np
import pytest

from oracle.attn import attn_forward as oracle_attn
from oracle.grad import attn_backward as oracle_backward
from tests.helpers import TOL_F32, block_rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_BIG = 850_000
M = 160                      # closed subsystem at the end
LMAX, C, H, K = 2, 128, 16, 8
S = (LMAX + 1) ** 2


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def e2f():
    import interatomic_potentials_amd as m
    return m


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def big():
    rng = np.random.default_rng(850)
    base = N_BIG - M
    assert base * (S + 1) * C * 4 > 2**32     # every subsystem row starts past 4 GiB
    pos = rng.random((N_BIG, 3), dtype=np.float32) * 200.0
    h = rng.standard_normal((N_BIG, S, C), dtype=np.float32)
    idx = rng.integers(0, base, size=(N_BIG, K), dtype=np.int32)
    mask = (rng.random((N_BIG, K)) < 0.7).astype(np.uint8)
    idx[base:] = rng.integers(base, N_BIG, size=(M, K), dtype=np.int32)
    mask[base + 3] = 0                         # a subsystem target with no valid slot
    return pos, h, idx, mask, base


def on(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def test_forward_rows_beyond_4_gib(e2f, dev, big):
    pos, h, idx, mask, base = big
    say(f"forward with 64-bit offsets: N={N_BIG} K={K} lmax={LMAX} C={C} H={H}")
    out, msg = e2f.attn_forward(on(pos, dev), on(h, dev), on(idx, dev), on(mask, dev), H,
                                return_msg=True)
    torch.cuda.synchronize()
    sub_out, sub_msg = out[base:].cpu().numpy(), msg[base:].cpu().numpy()
    ref, ref_msg = oracle_attn(pos[base:], h[base:], idx[base:] - base, mask[base:], H, LMAX,
                               return_msg=True)
    assert block_rel_err(sub_msg, ref_msg, LMAX) <= TOL_F32
    assert block_rel_err(sub_out, ref, LMAX) <= TOL_F32
    assert (sub_out[3] == 0).all()
    # targets of the rest, each with its valid sources as a small problem of its own
    for i in np.random.default_rng(1).choice(base, 6, replace=False).tolist() + [base - 1]:
        src = np.unique(idx[i][mask[i] != 0])
        atoms = np.concatenate([[i], src]).astype(np.int64)
        where = {int(a): n for n, a in enumerate(atoms)}
        cidx = np.zeros((len(atoms), K), np.int32)
        cmask = np.zeros((len(atoms), K), np.uint8)
        cidx[0] = [where.get(int(j), 0) for j in idx[i]]
        cmask[0] = mask[i]
        r = oracle_attn(pos[atoms], h[atoms], cidx, cmask, H, LMAX, targets=np.array([0]))
        assert block_rel_err(out[i:i + 1].cpu().numpy(), r, LMAX) <= TOL_F32


def test_backward_rows_beyond_4_gib(e2f, dev, big):
    pos, h, idx, mask, base = big
    say(f"backward with 64-bit offsets: N={N_BIG} K={K} lmax={LMAX} C={C} H={H}")
    g_sub = np.random.default_rng(2).standard_normal((M, S, C), dtype=np.float32)
    p, hh, ii, mm = on(pos, dev), on(h, dev), on(idx, dev), on(mask, dev)
    ws = e2f.attn_precouple(p, hh)
    _, msg, lse = e2f.attn_aggregate(p, ii, mm, ws, H, LMAX, C, torch.float32,
                                     return_msg=True, return_lse=True)
    g = torch.zeros_like(hh)
    g[base:] = on(g_sub, dev)
    gh, gp = e2f.attn_backward(p, hh, ii, mm, H, ws, msg, lse, g)
    torch.cuda.synchronize()
    rh, rp = oracle_backward(pos[base:], h[base:], idx[base:] - base, mask[base:], H, LMAX, g_sub)
    got_h = gh[base:].cpu().numpy()
    got_p = gp[base:].cpu().numpy().astype(np.float64)
    assert block_rel_err(got_h, rh, LMAX) <= TOL_F32
    nr = np.linalg.norm(rp, axis=1)
    den = np.maximum(nr, 1e-3 * nr.max() + 1e-300)
    assert float((np.linalg.norm(got_p - rp, axis=1) / den).max()) <= TOL_F32
    # no gradient reaches the rest from the subsystem's loss
    assert torch.isfinite(gh).all() and torch.isfinite(gp).all()
    assert (gh[:base].abs().max() == 0).item() and (gp[:base].abs().max() == 0).item()
