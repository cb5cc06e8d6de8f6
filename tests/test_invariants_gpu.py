"""Invariants of the method checked on the GPU path against the oracle (the oracle's own
invariants are pinned in test_oracle.py):

  - linearity: y is linear in (x, initial state) for fixed dt, A, B, C, D, so the GPU outputs of
    two inputs add up to the oracle's output of their sum (inputs on a grid coarse enough that
    the sums are exact in bf16);
  - head permutation: heads do not interact (B and C are shared within a group), so permuting
    the heads' x, dt, A, D and initial states permutes the outputs; on the fused path, whose
    per-head arithmetic does not depend on where a head sits, the result is bitwise the
    permutation of the unpermuted run.
"""

import numpy as np
import pytest
import torch

import mamba_ssd_chunked_cumsum_amd as ssd
from mamba_ssd_chunked_cumsum_amd import synth
from oracle import native

from gpu_util import as64, note, score, to_device

pytestmark = pytest.mark.gpu


def _grid(rng, shape, step=1 / 16, lim=4.0):
    """Values k * step in [-lim, lim]: sums of two stay exact in bf16 (at most 8 significant
    bits)."""
    return (np.round(rng.uniform(-lim, lim, shape) / step) * step).astype(np.float32)


def _gpu(inp, variant, chunk):
    d = to_device(inp, "bf16")
    y, f = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk,
                       d["initial_state"], variant=variant)
    torch.cuda.synchronize()
    return as64(y), as64(f)


@pytest.mark.parametrize("variant", ["fused", "unfused"])
def test_linearity_in_x_and_initial_state(variant):
    shape = synth.SSDShape("linear", 2, 700, 8, 64, 128, 1, 64, init_state=True)
    base = synth.make_inputs(shape, seed=31)
    rng = np.random.default_rng(32)
    parts = []
    for _ in range(2):
        p = dict(base)
        p["x"] = _grid(rng, base["x"].shape)
        p["initial_state"] = rng.standard_normal(base["initial_state"].shape).astype(np.float32)
        parts.append(p)
    total = dict(base)
    total["x"] = parts[0]["x"] + parts[1]["x"]
    total["initial_state"] = parts[0]["initial_state"] + parts[1]["initial_state"]
    note(f"linearity {variant}")
    (y1, f1), (y2, f2) = (_gpu(p, variant, shape.chunk_size) for p in parts)
    y_ref, f_ref = native.forward(**total)
    # each GPU result carries its own rounding; their sum is held to twice the parity bar
    rep = score(y1 + y2, f1 + f2, y_ref, f_ref, "bf16")
    assert rep["y_rms_r1"] <= 4e-2 and rep["final_rms_literal"] <= 4e-2, rep


@pytest.mark.parametrize("variant", ["fused", "unfused"])
def test_head_permutation(variant):
    shape = synth.SSDShape("perm", 1, 500, 16, 64, 128, 1, 64, init_state=True, random_d=True)
    inp = synth.make_inputs(shape, seed=33)
    perm = np.random.default_rng(34).permutation(shape.nheads)
    pinp = dict(inp)
    pinp["x"] = np.ascontiguousarray(inp["x"][:, :, perm])
    pinp["dt"] = np.ascontiguousarray(inp["dt"][:, :, perm])
    pinp["A"], pinp["D"] = inp["A"][perm], inp["D"][perm]
    pinp["initial_state"] = np.ascontiguousarray(inp["initial_state"][:, perm])
    note(f"head permutation {variant}")
    y, f = _gpu(inp, variant, shape.chunk_size)
    yp, fp = _gpu(pinp, variant, shape.chunk_size)
    if variant == "fused":
        assert np.array_equal(yp, y[:, :, perm]) and np.array_equal(fp, f[:, perm])
    y_ref, f_ref = native.forward(**pinp)
    assert score(yp, fp, y_ref, f_ref, "bf16")["pass"]
    assert score(yp, fp, y[:, :, perm], f[:, perm], "bf16")["pass"]
