"""Plant plausible mistakes in copies of the oracle (on the CPU) and require that
the pins catch every one of them: a dropped term, a wrong sign, a wrong index,
a transposed or swapped operand, a wrong log base, a wrong default, a wrong
split rule."""
import os
import types

import pytest

from oracle_pins import ALL_PINS

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

# (file, text to find, replacement)
MUTANTS = [
    ("attention.py", "ds = p * (dp - delta[:, None])", "ds = p * dp"),
    ("attention.py", "(dp - delta[:, None])", "(dp + delta[:, None])"),
    ("attention.py", "dq[b, rows, h, :] = scale * (ds @ kg)", "dq[b, rows, h, :] = (ds @ kg)"),
    ("attention.py", "dk[b, kb, g, :] += scale * (ds.T @ qr)", "dk[b, kb, g, :] += scale * (ds.T @ dor)"),
    ("attention.py", "dv[b, kb, g, :] += p.T @ dor", "dv[b, kb, g, :] += p.T @ qr"),
    ("attention.py", "dv[b, kb, g, :] += p.T @ dor", "dv[b, kb, g, :] = p.T @ dor"),
    ("attention.py", "return [np.flatnonzero(kmask[b]) for b in range(B)]", "return [np.flatnonzero(kmask[0]) for b in range(B)]"),
    ("attention.py", "kg, vg = k[b, keys[b], g, :], v[b, keys[b], g, :]", "kg, vg = k[b, keys[b], g, :], v[b, :keys[b].size, g, :]"),
    ("attention.py", "dv[b, kb, g, :] += p.T @ dor", "dv[b, :kb.size, g, :] += p.T @ dor"),
    ("attention.py", "kg, vg = k[b, kb, g, :], v[b, kb, g, :]", "kg, vg = k[b, :, g, :][kb], v[b, :, g, :][kb[::-1]]"),
    ("attention.py", "delta = (p * dp).sum(axis=1)", "delta = (p * dp).sum(axis=0).mean()"),
    ("attention.py", "g = h // G", "g = h % Hkv"),
    ("attention.py", "l_row = m + np.log(", "l_row = m + np.log2("),
    ("attention.py", "p = np.exp(s - l_row[:, None])", "p = np.exp(s - m[:, None])"),
    ("attention.py", "scale = 1.0 / np.sqrt(D)", "scale = 1.0 / D"),
    ("attention.py", "s = scale * (q[b, rows, h, :] @ kg.T)", "s = (q[b, rows, h, :] @ kg.T)"),
    ("attention.py", "out[b, rows, h, :] = p @ vg", "out[b, rows, h, :] = p @ kg"),
    ("attention.py", "wa * out_a + wb * out_b", "wa * out_a + wa * out_b"),
    ("attention.py", "np.logaddexp(lse_a, lse_b)", "np.maximum(lse_a, lse_b)"),
    ("attention.py", "wa = np.transpose(wa, (0, 2, 1))[..., None]", "wa = np.transpose(wb, (0, 2, 1))[..., None]"),
    ("attention.py", "(out * dout).sum(axis=3), (0, 2, 1)", "(out * dout).sum(axis=3), (0, 1, 2)"),
    ("permute.py", "(1 if i < extra else 0)", "(1 if i >= parts - extra else 0)"),
    ("permute.py", "x[:, :, hoff[r]:hoff[r + 1], :]", "x[:, :, hoff[R - 1 - r]:hoff[R - r], :]"),
    ("permute.py", "y[soff[i]:soff[i + 1]]", "y[soff[i]:soff[i] + seq_lens[0]]"),
    ("permute.py", "np.concatenate(pieces, axis=0)", "np.concatenate(pieces[::-1], axis=0)"),
]


def _load(mutated_file, find, repl):
    ns = {}
    for fname in ("attention.py", "permute.py"):
        with open(os.path.join(ORACLE_DIR, fname)) as f:
            src = f.read()
        if fname == mutated_file:
            assert find in src, f"mutant no longer applies: {find!r} not in {fname}"
            src = src.replace(find, repl)
        code = compile(src, f"<mutant {fname}>", "exec")
        mod = {"__name__": f"oracle_mutant_{fname[:-3]}"}
        exec(code, mod)
        ns.update({k: v for k, v in mod.items() if not k.startswith("_") or k in ("_offsets",)})
    return types.SimpleNamespace(**ns)


@pytest.mark.parametrize("mutant", MUTANTS, ids=[f"{m[0]}:{m[1][:40]}" for m in MUTANTS])
def test_pins_catch_mutant(mutant):
    o = _load(*mutant)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, IndexError, FloatingPointError) as e:
            caught.append(pin.__name__)
            break
    assert caught, f"no pin catches mutant {mutant}"


def test_unmutated_copy_passes():
    o = _load("attention.py", "g = h // G", "g = h // G")
    for pin in ALL_PINS:
        pin(o)
