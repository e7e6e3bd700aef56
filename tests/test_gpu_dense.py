"""GPU parity of the dense Clebsch-Gordan product (e2f_dense_couple) against the oracle.

The dense kernel is the baseline that EAAS replaces (write-up section 2.2, Fig. 3): every
path's full real coupling tensor, 615 multiply-adds per channel at lmax = 2.  It must
equal the oracle's dense contraction path by path (one-hot weights), and, by Proposition
4.3, the EAAS kernel's result up to rounding.
"""

import sys

import numpy as np
import pytest

from gen import bf16_bits_to_f32, f32_to_bf16_bits, make_micro
from oracle import tp
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


@pytest.mark.parametrize("lmax,C,n", [(0, 16, 37), (1, 16, 37), (2, 128, 37), (2, 5, 9),
                                      (2, 6, 300), (1, 128, 1), (2, 300, 17)])
def test_dense_each_path_fp32(e2f, dev, lmax, C, n):
    say(f"dense per path: lmax={lmax} C={C} n={n}")
    rng = np.random.default_rng(200 + lmax * 7 + C + n)
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
        got = to_host(e2f.dense_couple(T(r, dev), T(h, dev), path_w=w))
        ref = tp.tp_dense(h, r, lmax, w)
        err = block_rel_err(got, ref, lmax)
        assert err <= TOL_F32, (tp.paths(lmax)[p], err)
    w = rng.standard_normal(P).astype(np.float32)
    got = to_host(e2f.dense_couple(T(r, dev), T(h, dev), path_w=w))
    assert block_rel_err(got, tp.tp_dense(h, r, lmax, w), lmax) <= TOL_F32


def test_dense_in_place_and_bf16(e2f, dev):
    say("dense in place (fp32) and bf16 storage")
    rng = np.random.default_rng(6)
    n, C, lmax = 1000, 128, 2
    r = (rng.standard_normal((n, 3)) * 30).astype(np.float32)
    h = rng.standard_normal((n, 9, C)).astype(np.float32)
    ref = tp.tp_dense(h, r, lmax)
    ht = T(h, dev)
    out = e2f.dense_couple(T(r, dev), ht, out=ht)
    assert out.data_ptr() == ht.data_ptr()
    assert block_rel_err(to_host(out), ref, lmax) <= TOL_F32
    hb = bf16_bits_to_f32(f32_to_bf16_bits(h))
    got = e2f.dense_couple(T(r, dev), T(hb, dev, torch.bfloat16))
    assert got.dtype == torch.bfloat16
    assert block_rel_err(to_host(got), tp.tp_dense(hb, r, lmax), lmax) <= TOL_BF16


def test_dense_micro_workload_equals_eaas(e2f, dev):
    """2^20 unit vectors, C = 128, all 15 paths: sampled rows against the oracle, and the
    whole output against the EAAS kernel (Proposition 4.3 on the GPU)."""
    say("dense micro workload: B=2^20, C=128, lmax=2, fp32")
    r, h, _ = make_micro()
    rt, ht = T(r, dev), T(h, dev)
    dense = e2f.dense_couple(rt, ht)
    eaas = e2f.eaas_couple(rt, ht)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    rows = np.concatenate([rng.choice(r.shape[0], 512, replace=False), [0, r.shape[0] - 1]])
    sel = torch.from_numpy(rows).to(dev)
    assert block_rel_err(dense[sel].cpu().numpy(), tp.tp_dense(h[rows], r[rows], 2), 2) <= TOL_F32
    # unit vectors: every block is O(1), so an absolute bound covers every row
    diff = (dense - eaas).abs().max().item()
    scale = eaas.abs().max().item()
    assert diff <= 1e-5 * scale, (diff, scale)
