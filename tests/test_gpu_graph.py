"""The forward captured in a HIP graph (through torch.cuda.graph) and replayed.

The library launches only kernels on the caller's stream for a forward without index
validation (no memset, copy or synchronisation), so a captured step replays the same
kernels.  Each replay follows new input values copied into the captured buffers, with
eager work on the same stream between replays, and must equal an eager forward on the
same inputs bit for bit.
"""

import sys

import numpy as np
import pytest

from gen import make_config

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.mark.parametrize("name,proj", [("water", False), ("water", True), ("tiny", False),
                                       ("large", False)])
def test_forward_graph_replays(name, proj):
    import interatomic_potentials_amd as e2f
    from gen import proj_weights

    dev = torch.device("cuda:0")
    cfg = make_config(name)
    s = cfg.spec
    say(f"graph capture: {name} N={cfg.N} proj={proj}")
    pos = torch.from_numpy(cfg.pos).to(dev)
    h = torch.from_numpy(cfg.h).to(dev)
    idx = torch.from_numpy(cfg.idx).to(dev)
    mask = torch.from_numpy(cfg.mask).to(dev)
    w = (tuple(torch.from_numpy(x).to(dev) for x in proj_weights(s.lmax, s.C, seed=13))
         if proj else None)

    def step():
        return e2f.attn_forward(pos, h, idx, mask, s.H, proj=w)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):   # warm-up on the capture stream's side, as torch asks
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()
    rng = np.random.default_rng(3)
    for rep in range(4):
        h.copy_(torch.from_numpy(rng.standard_normal(cfg.h.shape).astype(np.float32)).to(dev))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        _ = (h * 2.0).sum()        # eager work between replays
        ref = step()
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay {rep} differs from the eager forward"
