"""dt pre-processing in float64 -- test infrastructure, see the package header.

Mamba-2 layers do not feed the recurrence the projected dt directly: a per-head bias is added, the
result goes through softplus (so dt > 0) and may be clamped to a range. The pages do not describe
this step (it precedes the path); it is written out here from its definition, in the order the
library documents:

    v = dt + dt_bias[h];   v = softplus(v) = log(1 + exp(v));   v = clip(v, dt_min, dt_max)

softplus is evaluated exactly as log(exp(0) + exp(v)) (numpy's logaddexp, no overflow); the clamp
applies when dt_max > 0.
"""

from __future__ import annotations

import numpy as np


def dt_effective(dt, dt_bias=None, softplus=False, dt_min=0.0, dt_max=0.0):
    """dt [..., H] -> the effective dt the recurrence runs on, float64."""
    v = np.asarray(dt, dtype=np.float64)
    if dt_bias is not None:
        v = v + np.asarray(dt_bias, dtype=np.float64)
    if softplus:
        v = np.logaddexp(0.0, v)
    if dt_max > 0:
        v = np.clip(v, dt_min, dt_max)
    return v
