"""Property-based checks of the float64 oracle (CPU): shapes, chunk lengths, cut points and value
ranges drawn by hypothesis, each property fixed by the mathematics of the recurrence rather than
by another call of the same code:

* the three formulations (token recurrence, quadratic masked form with its running-product mask,
  chunked algorithm at any chunk length) give one result;
* composition: running tokens 0..k-1, then k..L-1 from the state the first part left, gives the
  whole run's y and final state (the state passing between chunks or runs);
* gauge: scaling a group's B by s and its C by 1/s leaves y unchanged (only C B^T and the state's
  readout C S enter y), while the final state scales by s;
* dt = 0 everywhere: no decay and no input, so y_t = C_t h0 + D x_t and the final state is h0;
* the C oracle agrees with the numpy recurrence on the same float32-exact inputs.
"""

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

from oracle import native, ssd_chunked, ssd_quadratic, ssd_recurrence
from pins import rand_inputs

SETTINGS = settings(max_examples=25, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def problems(draw, max_len=48):
    G = draw(st.integers(1, 2))
    H = G * draw(st.integers(1, 2))
    shape = dict(Bt=draw(st.integers(1, 2)), L=draw(st.integers(1, max_len)), H=H,
                 P=draw(st.integers(1, 5)), N=draw(st.integers(1, 6)), G=G)
    h0 = draw(st.booleans())
    seed = draw(st.integers(0, 2**31 - 1))
    # decay per token up to |dt A| ~ 2 (strong) or small (slow), from one draw
    dt_hi = draw(st.sampled_from([0.01, 0.3, 0.8]))
    inp = rand_inputs(np.random.default_rng(seed), shape["Bt"], shape["L"], H, shape["P"],
                      shape["N"], G, h0=h0, dt_hi=dt_hi)
    return shape, inp


def _close(a, b, tol):
    scale = max(1.0, float(np.max(np.abs(b))))
    return float(np.max(np.abs(a - b))) <= tol * scale


@SETTINGS
@given(problems(), st.sampled_from([1, 2, 3, 4, 7, 8, 16, 64]))
def test_three_formulations_agree(prob, Q):
    _, inp = prob
    y, f = ssd_recurrence(**inp)
    yq, fq = ssd_quadratic(**inp)
    yc, fc, _ = ssd_chunked(**inp, chunk_size=Q)
    assert _close(yq, y, 1e-10) and _close(fq, f, 1e-10)
    assert _close(yc, y, 1e-10) and _close(fc, f, 1e-10)


@SETTINGS
@given(problems(), st.data())
def test_composition_over_a_cut(prob, data):
    shape, inp = prob
    L = shape["L"]
    if L < 2:
        return
    k = data.draw(st.integers(1, L - 1))
    y, f = ssd_recurrence(**inp)
    first = {n: (v[:, :k] if n in ("x", "dt", "B", "C") else v) for n, v in inp.items()}
    y1, f1 = ssd_recurrence(**first)
    second = {n: (v[:, k:] if n in ("x", "dt", "B", "C") else v) for n, v in inp.items()}
    second["initial_state"] = f1
    y2, f2 = ssd_recurrence(**second)
    assert _close(np.concatenate([y1, y2], axis=1), y, 1e-12)
    assert _close(f2, f, 1e-12)


@SETTINGS
@given(problems(), st.floats(0.25, 4.0))
def test_gauge_of_b_and_c(prob, s):
    shape, inp = prob
    y, f = ssd_recurrence(**inp)
    g = np.ones(shape["G"])
    g[0] = s  # only the first group rescaled
    scaled = dict(inp, B=inp["B"] * g[None, None, :, None], C=inp["C"] / g[None, None, :, None])
    if inp["initial_state"] is not None:  # the initial state lives in the same gauge as B
        heads = np.arange(shape["H"]) // (shape["H"] // shape["G"])
        scaled["initial_state"] = inp["initial_state"] * g[heads][None, :, None, None]
    ys, fs = ssd_recurrence(**scaled)
    assert _close(ys, y, 1e-12)
    heads = np.arange(shape["H"]) // (shape["H"] // shape["G"])
    assert _close(fs, f * g[heads][None, :, None, None], 1e-12)


@SETTINGS
@given(problems())
def test_zero_dt_keeps_the_initial_state(prob):
    shape, inp = prob
    Bt, H, P, N = shape["Bt"], shape["H"], shape["P"], shape["N"]
    h0 = inp["initial_state"] if inp["initial_state"] is not None else np.zeros((Bt, H, P, N))
    z = dict(inp, dt=np.zeros_like(inp["dt"]), initial_state=h0)
    y, f = ssd_recurrence(**z)
    heads = np.arange(H) // (H // shape["G"])
    Ch = inp["C"][:, :, heads]                                   # [Bt, L, H, N]
    expect = np.einsum("bhpn,bthn->bthp", h0, Ch) + inp["D"][None, None, :, None] * inp["x"]
    assert _close(y, expect, 1e-13)
    assert np.array_equal(f, h0)


@SETTINGS
@given(problems(max_len=40))
def test_c_oracle_matches_numpy(prob):
    _, inp = prob
    if native.max_threads() < 1:
        pytest.skip("C oracle not built")
    y, f = ssd_recurrence(**inp)
    yn, fn = native.forward(**inp)
    assert _close(yn, y, 1e-12) and _close(fn, f, 1e-12)
