"""Error measures for GPU-vs-oracle parity -- test infrastructure.

All measures compare a result g with the float64 oracle r and are computed in float64.
RMS(r) = sqrt(mean(r^2)) over the whole oracle tensor.

* ``rel_floored``  max |g - r| / max(|r|, RMS(r))           -- fp32 workloads, bound 1e-4
* ``rel_strict``   max |g - r| / |r|                         -- diagnostic only
* ``rms_literal``  max |g - r| / RMS(r)                      -- bf16 workloads' final_state, 2e-2
* ``rms_r1``       max max(0, |g - r| - half_ulp_bf16(r)) / RMS(r)
                                                             -- bf16 workloads' y, bound 2e-2

rms_r1 removes exactly the error that rounding the exact answer once to bf16 can make, so the
exact answer rounded to nearest bf16 scores 0; rms_literal applied to that rounded answer is the
floor that no bf16 output can beat.
"""

from __future__ import annotations

import numpy as np


def rms(r) -> float:
    r = np.asarray(r, dtype=np.float64)
    return float(np.sqrt(np.mean(r * r))) if r.size else 0.0


def half_ulp_bf16(r) -> np.ndarray:
    """Half the spacing of bf16 numbers at |r|: 2^(floor(log2|r|) - 8); 2^-134 below 2^-126."""
    r = np.abs(np.asarray(r, dtype=np.float64))
    out = np.full(r.shape, 2.0 ** -134)
    normal = r >= 2.0 ** -126
    _, e = np.frexp(r[normal])          # r = m * 2^e with m in [0.5, 1): floor(log2 r) = e - 1
    out[normal] = np.ldexp(1.0, e - 1 - 8)
    return out


def rel_floored(g, r) -> float:
    g, r = np.asarray(g, np.float64), np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    den = np.maximum(np.abs(r), rms(r))
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(g - r) / den))


def rel_strict(g, r) -> float:
    g, r = np.asarray(g, np.float64), np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    d = np.abs(g - r)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(d == 0, 0.0, d / np.abs(r))
    return float(np.max(q))


def rms_literal(g, r) -> float:
    g, r = np.asarray(g, np.float64), np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    s = rms(r)
    return float(np.max(np.abs(g - r)) / (s if s > 0 else 1.0))


def rms_r1(g, r) -> float:
    g, r = np.asarray(g, np.float64), np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    s = rms(r)
    excess = np.maximum(0.0, np.abs(g - r) - half_ulp_bf16(r))
    return float(np.max(excess) / (s if s > 0 else 1.0))


def bf16_round_f64(r) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as float64.

    Used only to report the floor of the literal measure; done in float64 so no double rounding
    through float32 occurs.
    """
    r = np.asarray(r, dtype=np.float64)
    out = np.zeros_like(r)
    nz = r != 0
    m, e = np.frexp(r[nz])                       # |m| in [0.5, 1)
    e = np.maximum(e, -125)                      # subnormal bf16 share the 2^-133 spacing
    scale = np.ldexp(1.0, 8 - e)                 # 8 significant bits in [2^(e-1), 2^e)
    out[nz] = np.round(r[nz] * scale) / scale    # np.round is ties-to-even
    return out


TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def parity_report(y, y_ref, final, final_ref, io: str) -> dict:
    """All measures for one run, and whether it passes the workload's bound."""
    rep = {
        "y_rel_floored": rel_floored(y, y_ref),
        "y_rel_strict": rel_strict(y, y_ref),
        "y_rms_literal": rms_literal(y, y_ref),
        "y_rms_r1": rms_r1(y, y_ref),
        "final_rel_floored": rel_floored(final, final_ref),
        "final_rms_literal": rms_literal(final, final_ref),
    }
    if io == "f32":
        rep["pass"] = rep["y_rel_floored"] <= TOL_F32 and rep["final_rel_floored"] <= TOL_F32
    else:
        rep["y_literal_floor"] = rms_literal(bf16_round_f64(y_ref), y_ref)
        rep["pass"] = rep["y_rms_r1"] <= TOL_BF16 and rep["final_rms_literal"] <= TOL_BF16
    return rep
