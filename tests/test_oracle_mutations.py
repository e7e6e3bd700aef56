"""Planted mistakes in the oracle: each one must make some pin fail.

Every case rewrites one expression in the source of one oracle module: a sign, an
index, a dropped factor, a transposed operand, an operand order, a wrong atom.  The
rewritten module stands in for the original for the duration of the case (its
functions are swapped in wherever the oracle and the pin modules hold the
originals), and the CPU pins run until one fails.  A case passes when one does, so
a mistake of that kind in the oracle could not go unnoticed.  CPU only.
"""

import inspect
import types

import pytest

import oracle
from oracle import attn, cg, grad, neighbours, sh, tp, wigner
from tests import test_oracle_envelope, test_oracle_grad, test_oracle_neighbours, test_oracle_pins

PIN_MODULES = [test_oracle_pins, test_oracle_envelope, test_oracle_grad, test_oracle_neighbours]
ORACLE_MODULES = [oracle, attn, cg, grad, neighbours, sh, tp, wigner]
SLOW_PINS = ("test_matches_kdtree_lists_sampled",)


def _pins():
    """Every pin of the pin modules as (name, function, kwargs), the slow ones last."""
    out = []
    for m in PIN_MODULES:
        for name, fn in vars(m).items():
            if not name.startswith("test_") or not inspect.isfunction(fn):
                continue
            marks = [mk for mk in getattr(fn, "pytestmark", []) if mk.name == "parametrize"]
            if not marks:
                out.append((f"{m.__name__}.{name}", fn, {}))
                continue
            argnames, argvalues = marks[0].args[0], marks[0].args[1]
            names = [a.strip() for a in argnames.split(",")]
            for v in argvalues:
                vals = tuple(v) if len(names) > 1 else (v,)
                out.append((f"{m.__name__}.{name}{list(vals)}", fn, dict(zip(names, vals))))
    return sorted(out, key=lambda p: any(s in p[0] for s in SLOW_PINS))


PINS = _pins()


def _mutant(mod, old, new):
    """The module rebuilt from its source with `old` (found exactly once) replaced by `new`."""
    src = inspect.getsource(mod)
    assert src.count(old) == 1, f"{mod.__name__}: the planted text must occur once: {old!r}"
    m = types.ModuleType(mod.__name__)
    m.__dict__.update(__package__=mod.__package__, __file__=mod.__file__)
    exec(compile(src.replace(old, new), mod.__file__, "exec"), m.__dict__)
    return m


def _swap_in(monkeypatch, mod, mutant):
    """Bind the mutant's functions wherever the originals are bound."""
    for name, new in vars(mutant).items():
        orig = getattr(mod, name, None)
        if orig is None or orig is new or not callable(orig) or isinstance(orig, type):
            continue
        if getattr(orig, "__module__", None) != mod.__name__:
            continue                                   # names the module imported stay
        for holder in ORACLE_MODULES + PIN_MODULES:
            for key, val in list(vars(holder).items()):
                if val is orig:
                    monkeypatch.setattr(holder, key, new)


def _first_failing_pin():
    for name, fn, kw in PINS:
        try:
            fn(**kw)
        except Exception:                              # an assertion, or arithmetic that broke
            return name
    return None


# (oracle module, text, replacement, the mistake it plants)
MUTATIONS = [
    (cg, "total += (-1) ** k / den", "total += (-1) ** (k + 1) / den",
     "Racah sum with the opposite overall sign"),
    (cg, "pre = sqrt((2 * J + 1) *", "pre = sqrt((2 * J + 2) *",
     "wrong normalisation of the Clebsch-Gordan coefficients"),
    (cg, "U[l + m, l - m] = 1j * sign * s", "U[l + m, l - m] = -1j * sign * s",
     "wrong phase in the real-to-complex basis change"),
    (cg, "        T = -1j * T\n    return np.ascontiguousarray(T.real)",
     "        T = 1j * T\n    return np.ascontiguousarray(T.real)",
     "opposite phase for paths with odd l_i + l_f + l_o"),
    (sh, "return np.stack([y, z, x], axis=-1)", "return np.stack([x, y, z], axis=-1)",
     "l = 1 harmonics in the Cartesian instead of the real-m order"),
    (sh, "0.5 * SQRT3 * (x * x - y * y)", "0.5 * SQRT3 * (y * y - x * x)",
     "sign of the m = 2 harmonic"),
    (sh, "0.5 * (3.0 * z * z - rr)", "(3.0 * z * z - rr)",
     "normalisation of the m = 0, l = 2 harmonic"),
    (wigner, "return Dt.T", "return Dt", "transposed Wigner-D blocks"),
    (wigner, "return rot_y(-theta) @ rot_z(-phi)", "return rot_z(-phi) @ rot_y(-theta)",
     "alignment rotations composed in the wrong order"),
    (wigner, "theta = np.arctan2(rho, r[2])", "theta = np.arctan2(r[2], rho)",
     "polar angle measured from the wrong axis"),
    (tp, "if abs(li - lf) <= lo <= li + lf:", "if abs(li - lf) < lo <= li + lf:",
     "a triangle-allowed path dropped"),
    (tp, "Y = solid_harmonic(lf, r)", "Y = solid_harmonic(lf, -r)",
     "dense product with the reversed direction"),
    (tp, "T = real_cg(li, lf, lo)  ",
     "T = real_cg(li, lf, lo).transpose(2, 1, 0) if li == lo else real_cg(li, lf, lo)  ",
     "dense product with a transposed coupling"),
    (tp, "entries.append((p, lo, -m, li, m, -c))", "entries.append((p, lo, -m, li, m, c))",
     "sign factor of the odd reindex dropped"),
    (tp, "entries.append((p, lo, m, li, -m, c))", "entries.append((p, lo, m, li, m, c))",
     "odd paths keeping m_i = m_o"),
    (tp, "w[p] * c * rn ** lf * xt", "w[p] * c * xt", "|r|^l_f factor dropped"),
    (tp, "out[a] = D.T @ yt", "out[a] = D @ yt", "rotated back with D instead of its inverse"),
    (attn, "scale = 1.0 / np.sqrt(d)", "scale = 1.0 / np.sqrt(C)",
     "logits scaled by the channel count instead of the head width"),
    (attn, "a = np.repeat(alpha[e0:e1], d, axis=1)", "a = np.tile(alpha[e0:e1], (1, d))",
     "channels assigned to heads round-robin"),
    (attn, "np.add.at(z, e_row, p)", "np.add.at(z, e_row, np.exp(logits - mx[e_row]))",
     "envelope in the numerator only"),
    (attn, "out = tp_dense(msg, pos[tgt], lmax, path_w)",
     "out = tp_dense(msg, pos[::-1][tgt], lmax, path_w)",
     "step 3 with another atom's harmonics"),
    (attn, "hp_src = tp_dense(v[src], pos[src], lmax, path_w)",
     "hp_src = tp_dense(v[src], -pos[src], lmax, path_w)",
     "step 1 with the reversed source direction"),
    (attn, "(10.0 + 15.0 * x)", "(10.0 + 14.0 * x)", "a wrong envelope coefficient"),
    (attn, "u = y ** 3 * (", "u = y ** 2 * (", "the envelope's zero at the cutoff one order short"),
    (attn, "u = y ** 3 * (1.0 + x * (3.0 + x * (6.0 + x * (10.0 + 15.0 * x))))",
     "u = 1.0 - 21.0 * x ** 5 + 35.0 * x ** 6 - 15.0 * x ** 7",
     "the envelope summed expanded, cancelling near the cutoff"),
    (attn, "e_src = idx[e_row, e_slot].astype(np.int64)",
     "e_src = idx[e_row, np.maximum(e_slot - 1, 0)].astype(np.int64)",
     "slot index off by one"),
    (grad, "p = p * envelope_torch(dist / float(env_cutoff))[:, None]",
     "p = p * envelope_torch(dist.detach() / float(env_cutoff))[:, None]",
     "no gradient through the envelope's distance"),
    (grad, "return torch.stack([y, z, x], dim=-1)", "return torch.stack([x, y, z], dim=-1)",
     "gradient oracle with l = 1 harmonics in the wrong order"),
    (neighbours, "ok = d2 < rc2", "ok = d2 <= rc2", "cutoff taken as inclusive"),
    (neighbours, "np.lexsort((js[sel], d2[r, sel]))", "np.lexsort((-js[sel], d2[r, sel]))",
     "equal distances ordered by decreasing index"),
    (neighbours, "ok[np.arange(rows.size), rows] = False",
     "ok[np.arange(rows.size), rows] = ok[np.arange(rows.size), rows]",
     "an atom listed as its own neighbour"),
]


def test_an_equivalent_rewrite_fails_no_pin(monkeypatch):
    """The harness itself: a rewrite that changes nothing, swapped in the same way, passes
    every pin (so a planted mistake is caught for what it changes, not for the swap)."""
    _swap_in(monkeypatch, tp, _mutant(tp, "out[a] = D.T @ yt", "out[a] = (D.T @ yt) * 1.0"))
    assert _first_failing_pin() is None


@pytest.mark.parametrize("mod,old,new,what", MUTATIONS, ids=[m[3] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(monkeypatch, mod, old, new, what):
    _swap_in(monkeypatch, mod, _mutant(mod, old, new))
    assert _first_failing_pin() is not None, f"no pin notices: {what}"
