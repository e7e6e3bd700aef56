"""The allocation-free forward (e2f_attn_forward_noalloc) against e2f_attn_forward.

The entry point is for callers that cannot allocate device memory: its workspace is the
library's static per-GPU array.  It runs the same kernels as e2f_attn_forward, so its
outputs must equal the caller-workspace entry point's bit for bit.  Two calls in a row,
the second smaller, check that nothing of the first call's contents leaks into the second.
"""

import ctypes
import sys

import numpy as np
import pytest

from gen import make_config
from oracle.attn import attn_forward as oracle_forward
from tests.helpers import TOL_F32, block_rel_err, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def e2f():
    import interatomic_potentials_amd as m
    return m


def T(x, dev, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    return t if dtype is None else t.to(dtype)


def _inputs(cfg, dev):
    return (T(cfg.pos, dev), T(cfg.h, dev), T(cfg.idx, dev), T(cfg.mask, dev))


def test_noalloc_matches_workspace_entry_point(e2f):
    dev = torch.device("cuda:0")
    assert e2f.attn_noalloc_max_bytes() == 64 << 20
    big = make_config("large", n_atoms=6000)          # 6000 atoms, K = 256: 36 MB of workspace
    small = make_config("water")                       # 648 atoms, K = 64
    for name, cfg in (("6000-atom large-shaped", big), ("water", small)):
        s = cfg.spec
        say(f"noalloc vs workspace forward: {name} N={cfg.N} K={s.K} C={s.C} H={s.H}")
        pos, h, idx, mask = _inputs(cfg, dev)
        ref, ref_msg, ref_lse = e2f.attn_forward(pos, h, idx, mask, s.H, return_msg=True,
                                                 return_lse=True)
        got, msg, lse = e2f.attn_forward_noalloc(pos, h, idx, mask, s.H, return_msg=True,
                                                 return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        assert torch.equal(msg, ref_msg)
        assert torch.equal(lse, ref_lse)
        rows = np.random.default_rng(7).choice(cfg.N, 64, replace=False)
        want = oracle_forward(cfg.pos, cfg.h, cfg.idx, cfg.mask, s.H, s.lmax, targets=rows)
        assert block_rel_err(to_host(got)[rows], want, s.lmax) <= TOL_F32


def test_noalloc_rejects_sizes_above_its_array(e2f):
    cap = e2f.attn_noalloc_max_bytes()
    N = cap // ((9 + 1) * 128 * 4) + 1     # rows alone exceed the array
    fake = ctypes.c_void_p(0x7F0000000000)
    rc = e2f.lib.e2f_attn_forward_noalloc(None, N, 64, 2, 128, 16, 0, fake, fake, fake, fake,
                                          0.0, 0.0, None, fake, None, None, 0)
    assert rc == e2f.STATUS_CODES["E2F_ERR_WORKSPACE"]
