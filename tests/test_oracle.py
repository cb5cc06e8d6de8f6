"""The CPU oracle against its pins (hand-worked examples, closed forms, brute force, invariants).

No GPU needed. Every oracle formulation (numpy recurrence, quadratic masked form, chunked
decomposition at several chunk sizes, the C/OpenMP recurrence) must pass every pin.
"""

import numpy as np
import pytest

from oracle import dt_effective, native, ssd_chunked, ssd_quadratic, ssd_recurrence, ssd_step
from mamba_ssd_chunked_cumsum_amd import synth

from pins import all_pins, rand_inputs


def chunked_fn(Q):
    def fn(**kw):
        y, f, _ = ssd_chunked(**kw, chunk_size=Q)
        return y, f
    return fn


def native_fn(**kw):
    return native.forward(**kw)


@pytest.mark.parametrize("name,fn,ref", [
    ("recurrence", ssd_recurrence, ssd_quadratic),
    ("quadratic", ssd_quadratic, ssd_recurrence),
    ("chunked_Q1", chunked_fn(1), ssd_quadratic),
    ("chunked_Q7", chunked_fn(7), ssd_quadratic),
    ("chunked_Q16", chunked_fn(16), ssd_quadratic),
    ("chunked_Q64", chunked_fn(64), ssd_quadratic),
    ("chunked_Q256", chunked_fn(256), ssd_quadratic),
    ("native_c", native_fn, ssd_quadratic),
])
def test_pins(name, fn, ref):
    failures = all_pins(fn, ref)
    assert not failures, f"{name}: {failures}"


@pytest.mark.parametrize("Q", [1, 16, 32, 64, 100, 128, 256, 300])
def test_chunked_independent_of_chunk_size(Q):
    """y and final_state do not depend on Q, including a ragged last chunk and Q > L."""
    rng = np.random.default_rng(11)
    inp = rand_inputs(rng, 2, 270, 4, 8, 16, 2, h0=True)
    y, f = ssd_recurrence(**inp)
    yc, fc, it = ssd_chunked(**inp, chunk_size=Q)
    scale = np.abs(y).max()
    assert np.abs(yc - y).max() <= 1e-12 * scale
    assert np.abs(fc - f).max() <= 1e-12 * np.abs(f).max()
    assert np.array_equal(it["h_in"][:, -1], fc)


def test_chunked_intermediates_definitions():
    """Acs is the per-chunk inclusive cumsum of dt*A; CB is C.B; states chain to final."""
    rng = np.random.default_rng(5)
    Q = 16
    inp = rand_inputs(rng, 1, 40, 2, 3, 4, 1, h0=True)
    y, f, it = ssd_chunked(**inp, chunk_size=Q)
    dt, A, B, C = inp["dt"], inp["A"], inp["B"], inp["C"]
    # chunk 1 of head 1, computed element by element
    acs = [sum(dt[0, 16 + k, 1] * A[1] for k in range(i + 1)) for i in range(16)]
    assert np.allclose(it["Acs"][0, 1, 1], acs, rtol=1e-13, atol=0)
    # the ragged last chunk (tokens 32..39) repeats its last value past the end
    assert np.allclose(it["Acs"][0, 0, 2, 8:], it["Acs"][0, 0, 2, 7])
    assert np.isclose(it["CB"][0, 2, 0, 3, 5], np.dot(C[0, 35, 0], B[0, 37, 0]))
    assert np.all(it["CB"][0, 2, 0, 8:, :] == 0)
    # the state entering chunk 1 equals the recurrence's state after token 15
    _, f16 = ssd_recurrence(**{k: (v[:, :16] if k in "x dt B C".split() else v)
                               for k, v in inp.items()})
    assert np.allclose(it["h_in"][:, 1], f16, rtol=1e-12, atol=1e-12)


def test_step_matches_recurrence():
    """One decode step from a state equals one more token of the recurrence."""
    rng = np.random.default_rng(3)
    inp = rand_inputs(rng, 2, 9, 4, 3, 5, 2, h0=True)
    y, f = ssd_recurrence(**inp)
    first = {k: (v[:, :8] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    _, f8 = ssd_recurrence(**first)
    ys, fs = ssd_step(f8, inp["x"][:, 8], inp["dt"][:, 8], inp["A"], inp["B"][:, 8],
                      inp["C"][:, 8], inp["D"])
    assert np.allclose(ys, y[:, 8], rtol=1e-13, atol=1e-13)
    assert np.allclose(fs, f, rtol=1e-13, atol=1e-13)


def test_step_hand_worked_scalar():
    """P = N = H = 1: a = exp(0.5 * -2 ln 2) = 1/2; s' = a * 2 + 0.5 * 3 * 4 = 7;
    y = -1 * 7 + 0.25 * 3 = -6.25."""
    st = np.array([[[[2.0]]]])
    y, s = ssd_step(st, np.array([[[3.0]]]), np.array([[0.5]]), np.array([-2.0 * np.log(2.0)]),
                    np.array([[[4.0]]]), np.array([[[-1.0]]]), np.array([0.25]))
    assert abs(s[0, 0, 0, 0] - 7.0) < 1e-14 and abs(y[0, 0, 0] + 6.25) < 1e-14


def test_step_closed_forms():
    """dt = 0: the state is unchanged and y = S C + D x. A = 0: S + dt x B^T (no decay). A
    group's B and C reach exactly its heads."""
    rng = np.random.default_rng(21)
    Bt, H, P, N, G = 2, 4, 3, 5, 2
    S = rng.standard_normal((Bt, H, P, N))
    x = rng.standard_normal((Bt, H, P))
    B, C = rng.standard_normal((Bt, G, N)), rng.standard_normal((Bt, G, N))
    A, D = -rng.uniform(0.5, 2, H), rng.uniform(0.5, 1.5, H)
    grp = np.arange(H) // (H // G)
    y, s = ssd_step(S, x, np.zeros((Bt, H)), A, B, C, D)
    assert np.array_equal(s, S)
    want = np.einsum("bhpn,bhn->bhp", S, C[:, grp]) + D[None, :, None] * x
    assert np.allclose(y, want, rtol=1e-14, atol=1e-14)
    dt = rng.uniform(0.1, 1, (Bt, H))
    _, s = ssd_step(S, x, dt, np.zeros(H), B, C, D)
    want = S + dt[:, :, None, None] * x[:, :, :, None] * B[:, grp][:, :, None, :]
    assert np.allclose(s, want, rtol=1e-14, atol=1e-14)
    B2 = B.copy()
    B2[:, 1] = 0.0  # group 1 (heads 2, 3) gets no input term: pure decay
    _, s = ssd_step(S, x, dt, A, B2, C, D)
    assert np.allclose(s[:, 2:], np.exp(dt[:, 2:] * A[2:])[:, :, None, None] * S[:, 2:],
                       rtol=1e-14, atol=1e-14)


def test_linearity_and_causality():
    """With h0 = 0, y - D x is linear in x; perturbing x at t0 leaves y[:t0] unchanged."""
    rng = np.random.default_rng(9)
    inp = rand_inputs(rng, 1, 60, 2, 3, 4, 1)
    x2 = rng.standard_normal(inp["x"].shape)
    ya, _ = ssd_recurrence(**inp)
    yb, _ = ssd_recurrence(**{**inp, "x": x2})
    yab, _ = ssd_recurrence(**{**inp, "x": 2.0 * inp["x"] + 3.0 * x2})
    assert np.allclose(yab, 2.0 * ya + 3.0 * yb, rtol=1e-12, atol=1e-12)
    xp = inp["x"].copy()
    xp[:, 37] += 5.0
    yp, _ = ssd_recurrence(**{**inp, "x": xp})
    assert np.array_equal(yp[:, :37], ya[:, :37])
    assert not np.allclose(yp[:, 37:], ya[:, 37:])


def test_head_permutation_equivariance():
    rng = np.random.default_rng(13)
    inp = rand_inputs(rng, 1, 30, 4, 2, 3, 1, h0=True)
    perm = np.array([2, 0, 3, 1])
    y, f = ssd_recurrence(**inp)
    pin = dict(inp)
    pin["x"] = inp["x"][:, :, perm]
    pin["dt"] = inp["dt"][:, :, perm]
    pin["A"], pin["D"] = inp["A"][perm], inp["D"][perm]
    pin["initial_state"] = inp["initial_state"][:, perm]
    yp, fp = ssd_recurrence(**pin)
    assert np.allclose(yp, y[:, :, perm], rtol=1e-14, atol=1e-14)
    assert np.allclose(fp, f[:, perm], rtol=1e-14, atol=1e-14)


def _rel(a, r):
    return np.max(np.abs(a - r)) / max(np.max(np.abs(r)), 1e-300)


@pytest.mark.parametrize("cfg", [0])
def test_native_matches_numpy_on_workload(cfg):
    inp = synth.make_inputs(synth.CONFIGS[cfg])
    y, f = ssd_recurrence(**inp)
    yc, fc = native.forward(**inp)
    assert _rel(yc, y) <= 1e-12 and _rel(fc, f) <= 1e-12


def test_native_matches_numpy_mamba_shaped():
    """A shortened Mamba-2-130M-shaped layer (L = 256), bf16 inputs, nonzero initial state."""
    shape = synth.config("mamba2_130m_layer").replace(seqlen=256, batch=2, init_state=True)
    inp = synth.make_inputs(shape, seed=21)
    y, f = ssd_recurrence(**inp)
    yc, fc = native.forward(**inp)
    assert _rel(yc, y) <= 1e-12 and _rel(fc, f) <= 1e-12


def test_native_unit_subset():
    rng = np.random.default_rng(17)
    inp = rand_inputs(rng, 2, 20, 3, 2, 4, 1, h0=True)
    y, f = native.forward(**inp)
    ys, fs = native.forward(**inp, units=[4, 1])
    for u in (4, 1):
        b, h = divmod(u, 3)
        assert np.array_equal(ys[b, :, h], y[b, :, h]) and np.array_equal(fs[b, h], f[b, h])
    assert np.isnan(ys[0, :, 0]).all()
    with pytest.raises(ValueError):
        native.forward(**inp, units=[6])


def test_dt_effective_closed_forms():
    """softplus(0) = ln 2; softplus(v) -> v for large v and -> exp(v) for very negative v; the bias
    is added per head before softplus; the clamp bounds the result; nothing set = identity."""
    dt = np.array([[[0.0, -30.0, 50.0, 0.5]]])
    assert np.array_equal(dt_effective(dt), dt)
    v = dt_effective(dt, softplus=True)
    assert abs(v[0, 0, 0] - np.log(2.0)) < 1e-15
    assert abs(v[0, 0, 1] / np.exp(-30.0) - 1.0) < 1e-12
    assert abs(v[0, 0, 2] - 50.0) < 1e-15
    assert abs(v[0, 0, 3] - np.log1p(np.exp(0.5))) < 1e-15
    bias = np.array([1.0, 2.0, -3.0, 0.0])
    assert np.allclose(dt_effective(dt, bias), dt + bias, rtol=0, atol=0)
    w = dt_effective(dt, bias, softplus=True)
    assert abs(w[0, 0, 0] - np.log1p(np.e)) < 1e-15   # softplus(0 + 1)
    c = dt_effective(dt, bias, softplus=True, dt_min=0.1, dt_max=1.0)
    assert c.min() >= 0.1 and c.max() <= 1.0
    assert c[0, 0, 2] == 1.0 and abs(c[0, 0, 3] - np.log1p(np.exp(0.5))) < 1e-15
