"""The parity measures behave as defined (no GPU needed)."""

import numpy as np
import torch

from oracle import metrics


def _rng_heavy(n, seed=0):
    rng = np.random.default_rng(seed)
    r = rng.standard_normal(n) * np.exp(rng.uniform(-6, 3, n))   # heavy-tailed, mixed scales
    r[:5] = [0.0, 2.0 ** -130, -2.0 ** -127, 1.0, -255.9]
    return r


def test_half_ulp_bf16_values():
    h = metrics.half_ulp_bf16(np.array([1.0, 1.5, 2.0, 3.999, 2.0 ** -126, 2.0 ** -127, 0.0]))
    assert list(h) == [2.0 ** -8, 2.0 ** -8, 2.0 ** -7, 2.0 ** -7, 2.0 ** -134, 2.0 ** -134,
                       2.0 ** -134]


def test_bf16_round_matches_torch_rne():
    r = _rng_heavy(20000)
    ours = metrics.bf16_round_f64(r)
    # torch rounds float32 -> bf16 with RNE; compare on float32-exact inputs (no double rounding)
    r32 = r.astype(np.float32)
    ref = torch.from_numpy(r32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(metrics.bf16_round_f64(r32.astype(np.float64)), ref)
    assert np.all(np.abs(ours - r) <= metrics.half_ulp_bf16(r))


def test_r1_floor_is_zero_for_rounded_exact_answer():
    r = _rng_heavy(50000, seed=1)
    assert metrics.rms_r1(metrics.bf16_round_f64(r), r) == 0.0
    # the literal measure of the same rounded answer is its (positive) floor
    assert metrics.rms_literal(metrics.bf16_round_f64(r), r) > 0.0


def test_r1_counts_only_excess_beyond_half_ulp():
    r = np.array([1.0, -3.0, 10.0, 0.5])
    s = metrics.rms(r)
    g = r.copy()
    g[2] += 2.0 ** -4 + 0.01        # half ulp at 10 is 2^-5; excess = 2^-4 + 0.01 - 2^-5
    assert np.isclose(metrics.rms_r1(g, r), (2.0 ** -4 + 0.01 - 2.0 ** -5) / s)


def test_rel_floored_and_strict():
    r = np.array([1e-9, 2.0, -2.0, 0.0])
    g = r + np.array([1e-9, 2e-4, 0.0, 0.0])
    s = metrics.rms(r)
    assert np.isclose(metrics.rel_floored(g, r), max(1e-9 / s, 2e-4 / 2.0))
    assert np.isclose(metrics.rel_strict(g, r), 1.0)           # the tiny entry is off by 100%
    assert metrics.rel_floored(r, r) == 0.0


def test_parity_report_thresholds():
    r = np.linspace(-3, 3, 101)
    f = np.linspace(-1, 1, 50)
    rep = metrics.parity_report(r, r, f, f, "f32")
    assert rep["pass"]
    rep = metrics.parity_report(r + 0.5, r, f, f, "bf16")
    assert not rep["pass"]
