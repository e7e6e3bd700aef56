"""Pins for the brute-force neighbour-list oracle (oracle/neighbours.py).

Sources of truth: scipy's k-d tree as used by the input generator (an
independent construction), hand-made geometries whose distances are exact in
binary floating point (strict cutoff, index tie-breaks, coincident atoms,
truncation), and a pure-Python double loop.
"""

import numpy as np
import pytest

from gen import make_config
from oracle.neighbours import neighbour_list, pair_d2


@pytest.mark.parametrize("name", ["tiny", "water"])
def test_matches_kdtree_lists_in_full(name):
    cfg = make_config(name)
    idx, mask, nw = neighbour_list(cfg.pos, cfg.spec.cutoff, cfg.spec.K)
    assert np.array_equal(idx, cfg.idx) and np.array_equal(mask, cfg.mask)
    assert np.array_equal(nw, cfg.nl.n_within)


@pytest.mark.parametrize("name,n", [("large", 300), ("scaleout", 300)])
def test_matches_kdtree_lists_sampled(name, n):
    cfg = make_config(name)
    tg = np.random.default_rng(1).choice(cfg.N, n, replace=False)
    idx, mask, nw = neighbour_list(cfg.pos, cfg.spec.cutoff, cfg.spec.K, targets=tg)
    assert np.array_equal(idx, cfg.idx[tg]) and np.array_equal(mask, cfg.mask[tg])
    assert np.array_equal(nw, cfg.nl.n_within[tg])


def test_strict_cutoff_and_index_ties_on_a_line():
    # atoms at x = 0, 1, 2, 3, 4 (exact in binary): distance exactly 2 is outside rc = 2
    pos = np.zeros((5, 3), np.float32)
    pos[:, 0] = np.arange(5)
    idx, mask, nw = neighbour_list(pos, 2.0, 4)
    assert idx[2].tolist() == [1, 3, -1, -1]          # equal distances: smaller index first
    assert mask[2].tolist() == [1, 1, 0, 0] and nw[2] == 2
    assert idx[0].tolist() == [1, -1, -1, -1]
    idx, _, nw = neighbour_list(pos, np.nextafter(2.0, 3.0), 4)
    assert idx[2].tolist() == [1, 3, 0, 4] and nw[2] == 4   # just above 2: both at 2 join


def test_coincident_atoms_and_truncation():
    pos = np.array([[1, 1, 1], [1, 1, 1], [1, 1, 1], [1.5, 1, 1], [9, 9, 9]], np.float32)
    idx, mask, nw = neighbour_list(pos, 1.0, 2)
    assert idx[0].tolist() == [1, 2] and nw[0] == 3     # d = 0 twice, then 0.5: truncated to 2
    assert idx[3].tolist() == [0, 1] and nw[3] == 3
    assert idx[4].tolist() == [-1, -1] and nw[4] == 0 and mask[4].sum() == 0


def test_matches_a_pure_python_double_loop():
    rng = np.random.default_rng(7)
    pos = (rng.random((23, 3)) * 6).astype(np.float32)
    pos[5] = pos[9]                                     # a coincident pair
    rc, K = 2.5, 6
    idx, mask, nw = neighbour_list(pos, rc, K)
    for i in range(len(pos)):
        xi = [float(v) for v in pos[i]]
        cand = []
        for j in range(len(pos)):
            if j == i:
                continue
            xj = [float(v) for v in pos[j]]
            d2 = (xi[0] - xj[0]) ** 2 + (xi[1] - xj[1]) ** 2
            d2 = d2 + (xi[2] - xj[2]) ** 2
            if d2 < rc * rc:
                cand.append((d2, j))
        cand.sort()
        want = [j for _, j in cand[:K]] + [-1] * max(0, K - len(cand))
        assert idx[i].tolist() == want and nw[i] == len(cand)
        assert mask[i].tolist() == [1] * min(K, len(cand)) + [0] * max(0, K - len(cand))


def test_pair_d2_rounds_like_the_definition():
    p = np.array([[0.1, 0.2, 0.3]], np.float32)
    q = np.array([[-0.7, 1.9, 2.5]], np.float32)
    a = p.astype(np.float64)[0] - q.astype(np.float64)[0]
    assert pair_d2(p, q)[0, 0] == (a[0] * a[0] + a[1] * a[1]) + a[2] * a[2]
