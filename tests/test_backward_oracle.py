"""Pins of the float64 backward oracle (no GPU): central finite differences of the forward
recurrence, which fix every gradient independently of how the oracle derives it."""

import numpy as np
import pytest

from oracle.backward import ssd_backward
from oracle.recurrence import ssd_recurrence

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _inputs(rng, Bt, L, H, P, N, G, h0):
    return dict(
        x=rng.standard_normal((Bt, L, H, P)),
        dt=rng.uniform(0.05, 0.6, (Bt, L, H)),
        A=-rng.uniform(0.3, 3.0, H),
        B=rng.standard_normal((Bt, L, G, N)),
        C=rng.standard_normal((Bt, L, G, N)),
        D=rng.uniform(0.5, 1.5, H),
        initial_state=rng.standard_normal((Bt, H, P, N)) if h0 else None,
    )


def _loss(inp, dy, dfinal):
    y, f = ssd_recurrence(**inp)
    out = float(np.sum(dy * y))
    if dfinal is not None:
        out += float(np.sum(dfinal * f))
    return out


CASES = [
    # Bt, L, H, P, N, G, h0, dfinal
    (1, 5, 2, 3, 2, 1, False, False),
    (2, 6, 4, 2, 3, 2, True, True),
    (1, 7, 3, 2, 2, 3, True, False),
    (1, 1, 2, 2, 2, 1, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:6])) + ("_h0" if c[6] else "") + ("_df" if c[7] else ""))
def test_backward_matches_finite_differences(case):
    Bt, L, H, P, N, G, h0, df = case
    rng = np.random.default_rng(7 + L * 11 + H)
    inp = _inputs(rng, Bt, L, H, P, N, G, h0)
    dy = rng.standard_normal((Bt, L, H, P))
    dfinal = rng.standard_normal((Bt, H, P, N)) if df else None
    g = ssd_backward(**inp, dy=dy, dfinal=dfinal)
    names = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
             "initial_state": "dinitial_state"}
    eps = 1e-6
    for k, gk in names.items():
        if inp[k] is None:
            continue
        arr = inp[k]
        num = np.empty_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + eps
            lp = _loss(inp, dy, dfinal)
            arr[idx] = keep - eps
            lm = _loss(inp, dy, dfinal)
            arr[idx] = keep
            num[idx] = (lp - lm) / (2 * eps)
        scale = max(1.0, float(np.max(np.abs(num))))
        err = float(np.max(np.abs(g[gk] - num)))
        assert err <= 1e-6 * scale, f"{gk}: max |analytic - finite difference| = {err:.3e}"


def test_backward_without_initial_state_still_returns_its_gradient():
    # the gradient with respect to a zero initial state is the same as with an explicit zero one
    rng = np.random.default_rng(3)
    inp = _inputs(rng, 1, 6, 2, 3, 2, 1, False)
    dy = rng.standard_normal((1, 6, 2, 3))
    g0 = ssd_backward(**inp, dy=dy)
    inp["initial_state"] = np.zeros((1, 2, 3, 2))
    g1 = ssd_backward(**inp, dy=dy)
    for k in g0:
        np.testing.assert_allclose(g0[k], g1[k], rtol=0, atol=0)


def test_backward_closed_form_no_decay():
    # A = 0: y_t = sum_{s<=t} dt_s (C_t . B_s) x_s + D x_t (causal linear attention), so
    # dx_s = D dy_s + dt_s sum_{t>=s} (C_t . B_s) dy_t  (written out with a causal mask)
    rng = np.random.default_rng(11)
    L, P, N = 6, 3, 4
    inp = _inputs(rng, 1, L, 1, P, N, 1, False)
    inp["A"] = np.zeros(1)
    dy = rng.standard_normal((1, L, 1, P))
    g = ssd_backward(**inp, dy=dy)
    Bm, Cm, dt = inp["B"][0, :, 0], inp["C"][0, :, 0], inp["dt"][0, :, 0]
    K = np.tril(Cm @ Bm.T)                              # K[t, s] = C_t . B_s for s <= t
    dx = inp["D"][0] * dy[0, :, 0] + dt[:, None] * (K.T @ dy[0, :, 0])
    np.testing.assert_allclose(g["dx"][0, :, 0], dx, rtol=1e-12, atol=1e-12)


def test_dlog_decay_abs_bounds_the_decay_gradient():
    """dlog_decay_abs_t = sum |G_t a_t S_{t-1}| bounds |dlog_t| = |<G_t, a_t S_{t-1}>|, and equals it
    when every product is >= 0 (nonnegative inputs and initial state)."""
    rng = np.random.default_rng(11)
    Bt, L, H, P, N, G = 1, 12, 2, 3, 4, 1
    inp = dict(x=rng.standard_normal((Bt, L, H, P)), dt=rng.uniform(0.1, 0.5, (Bt, L, H)),
               A=-rng.uniform(0.5, 2.0, H), B=rng.standard_normal((Bt, L, G, N)),
               C=rng.standard_normal((Bt, L, G, N)), D=np.ones(H),
               initial_state=rng.standard_normal((Bt, H, P, N)))
    dy = rng.standard_normal((Bt, L, H, P))
    g = ssd_backward(**inp, dy=dy)
    assert np.all(g["dlog_decay_abs"] >= np.abs(g["dlog_decay"]) * (1 - 1e-12))
    assert np.any(g["dlog_decay_abs"] > 1.01 * np.abs(g["dlog_decay"]))  # cancellation occurs
    pos = {k: (np.abs(v) if k in ("x", "B", "C", "initial_state") else v) for k, v in inp.items()}
    gp = ssd_backward(**pos, dy=np.abs(dy))
    assert np.allclose(gp["dlog_decay_abs"], gp["dlog_decay"], rtol=1e-12)
