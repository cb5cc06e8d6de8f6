"""Pins for an SSD forward implementation: checks against values fixed outside it.

Each pin takes `fn(x, dt, A, B, C, D, initial_state) -> (y, final_state)` and returns None when
it holds or a short failure message. The pins use hand-worked examples (tests/golden), closed
forms of special cases, brute force against an independent formulation, and invariants. They are
applied to every oracle formulation, and to deliberately broken copies of the oracle (mutation
test) to show that a plausible mistake fails at least one of them.
"""

from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rand_inputs(rng, Bt, L, H, P, N, G, h0=False, dt_lo=1e-3, dt_hi=0.3, a_lo=0.5, a_hi=4.0):
    x = rng.standard_normal((Bt, L, H, P))
    dt = rng.uniform(dt_lo, dt_hi, (Bt, L, H))
    A = -rng.uniform(a_lo, a_hi, H)
    B = rng.standard_normal((Bt, L, G, N))
    C = rng.standard_normal((Bt, L, G, N))
    D = rng.uniform(0.5, 1.5, H)
    s0 = rng.standard_normal((Bt, H, P, N)) if h0 else None
    # float32-exact values, so implementations that take float32 inputs see the same numbers
    f32 = lambda a: None if a is None else a.astype(np.float32).astype(np.float64)
    return dict(x=f32(x), dt=f32(dt), A=f32(A), B=f32(B), C=f32(C), D=f32(D), initial_state=f32(s0))


def _close(a, b, rtol):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if a.shape != b.shape:
        return False
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    return bool(np.max(np.abs(a - b)) <= rtol * scale) if b.size else True


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    s = g["shape"]
    Bt, L, H, P, N, G = (s[k] for k in ("batch", "seqlen", "nheads", "headdim", "dstate",
                                        "ngroups"))
    arr = lambda v, shp: None if v is None else np.asarray(v, np.float64).reshape(shp)
    inp = dict(x=arr(g["x"], (Bt, L, H, P)), dt=arr(g["dt"], (Bt, L, H)), A=arr(g["A"], (H,)),
               B=arr(g["B"], (Bt, L, G, N)), C=arr(g["C"], (Bt, L, G, N)), D=arr(g["D"], (H,)),
               initial_state=arr(g["initial_state"], (Bt, H, P, N)))
    return inp, arr(g["y"], (Bt, L, H, P)), arr(g["final_state"], (Bt, H, P, N)), g["rtol"]


def pin_golden(fn, name):
    inp, y_ref, f_ref, rtol = load_golden(name)
    y, f = fn(**inp)
    if not _close(y, y_ref, rtol):
        return f"{name}: y {np.ravel(y)} != {np.ravel(y_ref)}"
    if not _close(f, f_ref, rtol):
        return f"{name}: final {np.ravel(f)} != {np.ravel(f_ref)}"
    return None


def pin_no_decay(fn, rng):
    """A = 0: y = tril(C B^T) (dt * x) + D x, a causal masked matmul; final = sum_t dt x B^T."""
    inp = rand_inputs(rng, 2, 37, 3, 4, 5, 1)
    inp["A"] = np.zeros(3)
    y, f = fn(**inp)
    for b in range(2):
        for h in range(3):
            Cg, Bg = inp["C"][b, :, 0], inp["B"][b, :, 0]
            u = inp["dt"][b, :, h, None] * inp["x"][b, :, h]
            yr = np.tril(Cg @ Bg.T) @ u + inp["D"][h] * inp["x"][b, :, h]
            fr = u.T @ Bg
            if not _close(y[b, :, h], yr, 1e-10):
                return "A=0: y differs from tril(C B^T)(dt x) + D x"
            if not _close(f[b, h], fr, 1e-10):
                return "A=0: final state differs from sum_t dt x B^T"
    return None


def pin_strong_decay(fn, rng):
    """Decay ~ exp(-100): only the token's own term survives."""
    inp = rand_inputs(rng, 1, 29, 2, 3, 4, 1, h0=True, dt_lo=1e-2, dt_hi=1e-1)
    inp["A"] = np.full(2, -1e4)
    y, f = fn(**inp)
    x, dt, B, C, D = inp["x"], inp["dt"], inp["B"][:, :, 0], inp["C"][:, :, 0], inp["D"]
    cb = np.sum(C * B, axis=-1)                                     # [Bt, L]
    yr = dt[..., None] * cb[:, :, None, None] * x + D[None, None, :, None] * x
    fr = dt[:, -1, :, None, None] * x[:, -1, :, :, None] * B[:, -1, None, None, :]
    if not _close(y, yr, 1e-10):
        return "strong decay: y differs from dt (C.B) x + D x"
    if not _close(f, fr, 1e-10):
        return "strong decay: final differs from dt x_last B_last^T"
    return None


def pin_zero_readout(fn, rng):
    """C = 0: y = D x exactly."""
    inp = rand_inputs(rng, 1, 23, 2, 3, 4, 1, h0=True)
    inp["C"] = np.zeros_like(inp["C"])
    y, _ = fn(**inp)
    if not _close(y, inp["D"][None, None, :, None] * inp["x"], 1e-14):
        return "C=0: y != D x"
    return None


def pin_initial_state_only(fn, rng):
    """x = 0: y_t = exp(sum_{k<=t} dt_k A) C_t . h0, final = exp(sum_t dt_t A) h0."""
    inp = rand_inputs(rng, 2, 31, 2, 3, 4, 2, h0=True)
    inp["x"] = np.zeros_like(inp["x"])
    y, f = fn(**inp)
    h0, dt, A, C = inp["initial_state"], inp["dt"], inp["A"], inp["C"]
    for b in range(2):
        for h in range(2):
            g = h  # H = G = 2
            e = np.exp(np.cumsum(dt[b, :, h] * A[h]))               # [L]
            yr = e[:, None] * (C[b, :, g] @ h0[b, h].T)
            if not _close(y[b, :, h], yr, 1e-10):
                return "x=0: y differs from exp(cumsum) C h0"
            if not _close(f[b, h], e[-1] * h0[b, h], 1e-10):
                return "x=0: final differs from exp(sum) h0"
    return None


def pin_single_step(fn, rng):
    """L = 1: y = exp(dt A) C.h0 + dt (C.B) x + D x, final = exp(dt A) h0 + dt x B^T."""
    inp = rand_inputs(rng, 1, 1, 2, 3, 4, 1, h0=True)
    y, f = fn(**inp)
    x, dt, A, B, C, D, h0 = (inp[k] for k in ("x", "dt", "A", "B", "C", "D", "initial_state"))
    for h in range(2):
        a = np.exp(dt[0, 0, h] * A[h])
        fr = a * h0[0, h] + dt[0, 0, h] * np.outer(x[0, 0, h], B[0, 0, 0])
        yr = fr @ C[0, 0, 0] + D[h] * x[0, 0, h]
        if not _close(y[0, 0, h], yr, 1e-12) or not _close(f[0, h], fr, 1e-12):
            return "L=1 closed form fails"
    return None


def pin_brute_force(fn, reference, rng):
    """Random small problems (several heads, 2 groups, with and without h0) vs an independent
    formulation."""
    for (Bt, L, H, P, N, G, h0) in [(1, 50, 4, 3, 5, 2, False), (2, 41, 2, 4, 2, 1, True),
                                    (1, 64, 6, 2, 3, 3, True)]:
        inp = rand_inputs(rng, Bt, L, H, P, N, G, h0=h0)
        y, f = fn(**inp)
        yr, fr = reference(**inp)
        if not _close(y, yr, 1e-10) or not _close(f, fr, 1e-10):
            return f"brute force mismatch at {(Bt, L, H, P, N, G, h0)}"
    return None


def pin_group_replication(fn, rng):
    """G = 1 equals G = H with B and C copied to every head."""
    inp = rand_inputs(rng, 1, 33, 3, 2, 4, 1, h0=True)
    y1, f1 = fn(**inp)
    rep = dict(inp)
    rep["B"] = np.repeat(inp["B"], 3, axis=2)
    rep["C"] = np.repeat(inp["C"], 3, axis=2)
    y2, f2 = fn(**rep)
    if not _close(y1, y2, 1e-12) or not _close(f1, f2, 1e-12):
        return "G=1 differs from G=H with replicated B, C"
    return None


def pin_state_composition(fn, rng):
    """Running [0, L1) then [L1, L) from the carried state equals one run over [0, L)."""
    inp = rand_inputs(rng, 1, 40, 2, 3, 4, 1, h0=True)
    y, f = fn(**inp)
    L1 = 17
    first = {k: (v[:, :L1] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    ya, fa = fn(**first)
    second = {k: (v[:, L1:] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    second["initial_state"] = fa
    yb, fb = fn(**second)
    if not _close(np.concatenate([ya, yb], axis=1), y, 1e-10) or not _close(fb, f, 1e-10):
        return "state composition fails"
    return None


def all_pins(fn, reference, seed=7):
    rng = np.random.default_rng(seed)
    checks = [
        lambda: pin_golden(fn, "hand_scalar.json"),
        lambda: pin_golden(fn, "hand_matrix.json"),
        lambda: pin_no_decay(fn, rng),
        lambda: pin_strong_decay(fn, rng),
        lambda: pin_zero_readout(fn, rng),
        lambda: pin_initial_state_only(fn, rng),
        lambda: pin_single_step(fn, rng),
        lambda: pin_brute_force(fn, reference, rng),
        lambda: pin_group_replication(fn, rng),
        lambda: pin_state_composition(fn, rng),
    ]
    failures = []
    for c in checks:
        try:
            msg = c()
        except Exception as e:  # a broken implementation may also crash
            msg = f"raised {type(e).__name__}: {e}"
        if msg:
            failures.append(msg)
    return failures
