"""Every channel / head layout with C % H == 0 (up to 512 channels) against the oracle.

Head widths that are not a power of two (d = 3, 5, 6, 12) and rows wider than the
vectorised kernels take (fp32 C = 256 and 512 with wide heads) run on the general
kernel (one channel a lane, per-head sums through LDS); the others on the vectorised
kernels.  Tolerances: 1e-4 (fp32), 2e-2 (bf16 storage, fp32 arithmetic); empty rows
give exact zeros; slot order does not change a bit.
"""

import sys

import numpy as np
import pytest

from gen import bf16_bits_to_f32, f32_to_bf16_bits
from oracle.attn import attn_forward as oracle_attn
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


SHAPES = [(2, 24, 8), (2, 15, 3), (2, 96, 16), (1, 48, 4), (2, 60, 5), (2, 256, 4),
          (2, 512, 64), (0, 36, 12), (2, 512, 8), (1, 256, 2), (2, 48, 16)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("lmax,C,H", SHAPES)
def test_any_head_layout_vs_oracle(e2f, dev, lmax, C, H, dt):
    d = C // H
    say(f"layout lmax={lmax} C={C} H={H} (d={d}) {dt}")
    rng = np.random.default_rng(9000 + lmax * 1000 + C + H)
    N, K = 70, 40
    S = (lmax + 1) ** 2
    pos = (rng.standard_normal((N, 3)) * 4).astype(np.float32)
    h = rng.standard_normal((N, S, C)).astype(np.float32)
    tdt = torch.float32
    if dt == "bf16":
        h = bf16_bits_to_f32(f32_to_bf16_bits(h))
        tdt = torch.bfloat16
    idx = rng.integers(0, N, size=(N, K)).astype(np.int32)
    mask = (rng.random((N, K)) < 0.6).astype(np.uint8)
    mask[5] = 0                                         # a target with no valid slot
    out, msg, lse = e2f.attn_forward(T(pos, dev), T(h, dev, tdt), T(idx, dev), T(mask, dev), H,
                                     return_msg=True, return_lse=True)
    ref, ref_msg = oracle_attn(pos, h, idx, mask, H, lmax, return_msg=True)
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert block_rel_err(to_host(msg), ref_msg, lmax) <= tol
    assert block_rel_err(to_host(out), ref, lmax) <= tol
    assert (out[5].float() == 0).all()
    assert torch.isinf(lse[5]).all() and torch.isfinite(lse[:5]).all()
    # slot order changes nothing, bit for bit
    perm = np.argsort(rng.random(idx.shape), axis=1)
    out2 = e2f.attn_forward(T(pos, dev), T(h, dev, tdt), T(np.take_along_axis(idx, perm, 1), dev),
                            T(np.take_along_axis(mask, perm, 1), dev), H)
    assert torch.equal(out, out2)


@pytest.mark.parametrize("lmax,C,H", [(2, 24, 8), (2, 512, 8)])
def test_any_head_layout_envelope(e2f, dev, lmax, C, H):
    say(f"layout with the envelope: lmax={lmax} C={C} H={H}")
    rng = np.random.default_rng(77 + C)
    N, K = 60, 30
    S = (lmax + 1) ** 2
    pos = (rng.standard_normal((N, 3)) * 2).astype(np.float32)
    h = rng.standard_normal((N, S, C)).astype(np.float32)
    idx = rng.integers(0, N, size=(N, K)).astype(np.int32)
    mask = (rng.random((N, K)) < 0.6).astype(np.uint8)
    r_env = 3.0
    out = e2f.attn_forward(T(pos, dev), T(h, dev), T(idx, dev), T(mask, dev), H, env_cutoff=r_env)
    ref = oracle_attn(pos, h, idx, mask, H, lmax, env_cutoff=r_env)
    assert block_rel_err(to_host(out), ref, lmax) <= TOL_F32


def test_backward_layout_without_a_lane_width_is_reported(e2f, dev):
    """The backward keeps the vectorised lane mapping: d = 3 is reported, nothing launched."""
    N, C, H = 8, 24, 8
    pos = torch.zeros((N, 3), device=dev)
    h = torch.zeros((N, 9, C), device=dev)
    idx = torch.zeros((N, 4), dtype=torch.int32, device=dev)
    mask = torch.zeros((N, 4), dtype=torch.uint8, device=dev)
    ws = e2f.attn_precouple(pos, h)
    out, msg, lse = e2f.attn_aggregate(pos, idx, mask, ws, H, 2, C, torch.float32,
                                       return_msg=True, return_lse=True)
    with pytest.raises(e2f.E2FError) as ei:
        e2f.attn_backward(pos, h, idx, mask, H, ws, msg, lse, torch.zeros_like(h),
                          bwd_ws=torch.empty(256, dtype=torch.uint8, device=dev))
    assert ei.value.name == "E2F_ERR_UNSUPPORTED"
