"""Mutation test: plant plausible mistakes in copies of the oracle and check the pins catch each.

A mutant is the oracle's own source with one edit (a flipped sign, a dropped term, a swapped or
transposed operand, an off-by-one index, a wrong group map). Each mutant must fail at least one
pin in tests/pins.py; a mutant that passes every pin would mean the pins leave that part of the
oracle unchecked. Everything runs on the CPU on copies; the oracle files are not modified.
"""

import importlib.util
import os
import types

import pytest

import oracle
from oracle import ssd_quadratic, ssd_recurrence

from pins import all_pins

ORACLE_DIR = os.path.dirname(oracle.__file__)


def _mutant(module_file, old, new, fn_name):
    path = os.path.join(ORACLE_DIR, module_file)
    src = open(path).read()
    assert src.count(old) >= 1, f"mutation site not found in {module_file}: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType(f"mutant_{fn_name}")
    mod.__dict__["__name__"] = f"oracle_mutant_{module_file[:-3]}"
    exec(compile(src, path, "exec"), mod.__dict__)
    return getattr(mod, fn_name)


REC = [
    ("decay sign", "np.exp(dt[:, t, :] * A[None, :])", "np.exp(-dt[:, t, :] * A[None, :])"),
    ("decay uses previous dt", "np.exp(dt[:, t, :] * A[None, :])",
     "np.exp(dt[:, t - 1, :] * A[None, :])"),
    ("input not scaled by dt", "u = dt[:, t, :, None] * x[:, t]", "u = x[:, t]"),
    ("skip term dropped", " + D[None, :, None] * x[:, t]", ""),
    ("B and C swapped in update", "u[:, :, :, None] * Bh[:, :, None, :]",
     "u[:, :, :, None] * Ch[:, :, None, :]"),
    ("B used for readout", "(S @ Ch[:, :, :, None])", "(S @ Bh[:, :, :, None])"),
    ("input decayed too", "S = decay[:, :, None, None] * S + u[:, :, :, None] * Bh[:, :, None, :]",
     "S = decay[:, :, None, None] * (S + u[:, :, :, None] * Bh[:, :, None, :])"),
    ("wrong group map", "return np.arange(nheads) // (nheads // ngroups)",
     "return np.arange(nheads) % ngroups"),
    ("initial state ignored", "S = np.zeros((Bt, H, P, N)) if initial_state is None else",
     "S = np.zeros((Bt, H, P, N)) if True else"),
    ("readout before update",
     "        S = decay[:, :, None, None] * S + u[:, :, :, None] * Bh[:, :, None, :]\n"
     "        y[:, t] = (S @ Ch[:, :, :, None])[..., 0] + D[None, :, None] * x[:, t]",
     "        y[:, t] = (S @ Ch[:, :, :, None])[..., 0] + D[None, :, None] * x[:, t]\n"
     "        S = decay[:, :, None, None] * S + u[:, :, :, None] * Bh[:, :, None, :]"),
]

QUAD = [
    ("mask diagonal not 1", "row = np.append(row * a[t], 1.0)", "row = np.append(row * a[t], a[t])"),
    ("mask transposed", "scores = C[b, :, g, :] @ B[b, :, g, :].T",
     "scores = B[b, :, g, :] @ C[b, :, g, :].T"),
    ("final uses first row", "final[b, h] = (lam[L - 1, :, None] * u).T",
     "final[b, h] = (lam[0, :, None] * u).T"),
    ("h0 decay off by one step", "run *= a[t]\n                    from_start[t] = run",
     "from_start[t] = run\n                    run *= a[t]"),
    ("h0 readout uses B", "(C[b, :, g, :] @ h0.T)", "(B[b, :, g, :] @ h0.T)"),
]

CHUNKED = [
    ("exclusive cumsum", "Acs = np.cumsum(dtc * A[None, None, None, :], axis=2)",
     "Acs = np.cumsum(dtc * A[None, None, None, :], axis=2) - dtc * A[None, None, None, :]"),
    ("state decay from chunk start", "w = np.exp(last[None, :] - acs.T)", "w = np.exp(acs.T)"),
    ("passing without decay", "h_in[b, c + 1] = np.exp(last)[:, None, None] * h_in[b, c]",
     "h_in[b, c + 1] = h_in[b, c]"),
    ("inter term uses next state", "np.einsum(\"ihn,hpn->ihp\", Ch, h_in[b, c])",
     "np.einsum(\"ihn,hpn->ihp\", Ch, h_in[b, c + 1])"),
    ("mask includes future", "causal = np.tril(np.ones((Q, Q), dtype=bool))",
     "causal = np.ones((Q, Q), dtype=bool)"),
    ("inter term not decayed", "inter = np.exp(acs.T)[:, :, None] *", "inter = 1.0 *"),
]


def _chunked_wrap(fn, Q=16):
    def f(**kw):
        y, fin, _ = fn(**kw, chunk_size=Q)
        return y, fin
    return f


@pytest.mark.parametrize("label,old,new", REC, ids=[m[0] for m in REC])
def test_recurrence_mutants_are_caught(label, old, new):
    fn = _mutant("recurrence.py", old, new, "ssd_recurrence")
    assert all_pins(fn, ssd_quadratic), f"mutant '{label}' passed every pin"


@pytest.mark.parametrize("label,old,new", QUAD, ids=[m[0] for m in QUAD])
def test_quadratic_mutants_are_caught(label, old, new):
    fn = _mutant("quadratic.py", old, new, "ssd_quadratic")
    assert all_pins(fn, ssd_recurrence), f"mutant '{label}' passed every pin"


@pytest.mark.parametrize("label,old,new", CHUNKED, ids=[m[0] for m in CHUNKED])
def test_chunked_mutants_are_caught(label, old, new):
    fn = _chunked_wrap(_mutant("chunked.py", old, new, "ssd_chunked"))
    assert all_pins(fn, ssd_quadratic), f"mutant '{label}' passed every pin"


def test_unmutated_copies_pass():
    """The exec'd copies themselves (no edit) pass, so a caught mutant is caught by its edit."""
    assert not all_pins(_mutant("recurrence.py", "import numpy", "import numpy",
                                "ssd_recurrence"), ssd_quadratic)
    assert not all_pins(_chunked_wrap(_mutant("chunked.py", "import numpy", "import numpy",
                                              "ssd_chunked")), ssd_quadratic)
