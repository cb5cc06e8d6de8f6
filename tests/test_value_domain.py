"""Inputs outside the kernels' domain (the binding's forward() documents the behaviour these tests
check): a NaN reaches only its head's outputs from its sub-chunk or chunk onwards (its group's
heads, for B); a bf16 value beyond fp16's range becomes infinite in the fused path's operands
with the same reach (the fp32 precision option has no such limit); the opt-in check rejects NaN, A > 0, dt < 0 and fp16 overflow before
anything is launched. Every other head, and the earlier tokens of the affected head, still match
the oracle."""

import numpy as np
import pytest
import torch

import mamba_ssd_chunked_cumsum_amd as ssd
from mamba_ssd_chunked_cumsum_amd import libssd, synth
from oracle import native

from gpu_util import as64, note, score, to_device

pytestmark = pytest.mark.gpu

SHAPE = synth.SSDShape("domain", 2, 300, 4, 64, 128, 1, 64)
T_BAD, H_BAD, B_BAD = 150, 2, 1   # the token, head and batch entry that get the bad value


def _run(inp, variant, **kw):
    d = to_device(inp, SHAPE.io)
    y, f = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], SHAPE.chunk_size,
                       d["initial_state"], variant=variant, **kw)
    torch.cuda.synchronize()
    return as64(y), as64(f)


def _clean_units_match(y, f, inp, bad_units):
    """Every (batch, head) unit but bad_units matches the oracle."""
    units = [u for u in range(SHAPE.batch * SHAPE.nheads) if u not in bad_units]
    y_ref, f_ref = native.forward(**inp, units=units)
    rep = score(y, f, y_ref, f_ref, SHAPE.io, units, SHAPE.nheads)
    assert rep["pass"], rep


def _bad_head_reach(y, f, inp, start, final_too=True):
    """The bad unit: finite (and matching the oracle) before `start`, not finite at the bad token
    (and, for a NaN, in its final state)."""
    yb = y[B_BAD, :, H_BAD]
    assert np.all(np.isfinite(yb[:start])), "earlier tokens must stay finite"
    assert not np.all(np.isfinite(yb[T_BAD])), "the bad token's output"
    if final_too:
        assert not np.all(np.isfinite(f[B_BAD, H_BAD])), "the final state"
    clean = {k: (None if v is None else v.copy()) for k, v in inp.items()}
    clean["x"] = clean["x"][:, :start]
    clean["dt"] = clean["dt"][:, :start]
    clean["B"], clean["C"] = clean["B"][:, :start], clean["C"][:, :start]
    u = B_BAD * SHAPE.nheads + H_BAD
    y_ref, _ = native.forward(**clean, units=[u])
    err = np.max(np.abs(yb[:start] - y_ref[B_BAD, :, H_BAD]))
    assert err <= 2e-2 * np.sqrt(np.mean(y_ref[B_BAD, :, H_BAD] ** 2)) + 1e-2, err


@pytest.mark.parametrize("variant,grain", [("fused", 32), ("unfused", SHAPE.chunk_size)])
def test_nan_in_x_reaches_its_head_only(variant, grain):
    inp = synth.make_inputs(SHAPE, seed=21)
    inp["x"][B_BAD, T_BAD, H_BAD, 5] = np.nan
    note(f"domain nan x {variant}")
    y, f = _run(inp, variant)
    _clean_units_match(y, f, inp, {B_BAD * SHAPE.nheads + H_BAD})
    _bad_head_reach(y, f, inp, (T_BAD // grain) * grain)


def test_nan_in_B_reaches_its_group():
    inp = synth.make_inputs(SHAPE, seed=22)
    inp["B"][B_BAD, T_BAD, 0, 7] = np.nan
    note("domain nan B")
    y, f = _run(inp, "fused")
    # one group: every head of batch entry B_BAD; the other batch entry is untouched
    bad = {B_BAD * SHAPE.nheads + h for h in range(SHAPE.nheads)}
    _clean_units_match(y, f, inp, bad)
    assert np.all(np.isfinite(y[B_BAD, :(T_BAD // 32) * 32]))
    assert not np.all(np.isfinite(y[B_BAD, T_BAD:]))


def test_fp16_overflow_in_the_fused_path():
    # the value itself is infinite in the fused scan's fp16 x operand; the run states take x
    # multiplied by its decay weight (below 1) before rounding, so whether the final state stays
    # finite depends on the weight: only the outputs from the value's sub-chunk on are undefined
    inp = synth.make_inputs(SHAPE, seed=23)
    inp["x"][B_BAD, T_BAD, H_BAD, 3] = 99840.0   # exact in bf16, beyond fp16
    note("domain fp16 overflow")
    y, f = _run(inp, "fused")
    _clean_units_match(y, f, inp, {B_BAD * SHAPE.nheads + H_BAD})
    _bad_head_reach(y, f, inp, (T_BAD // 32) * 32, final_too=False)


def test_fp32_precision_has_no_fp16_limit():
    inp = synth.make_inputs(SHAPE, seed=23)
    inp["x"][B_BAD, T_BAD, H_BAD, 3] = 99840.0
    note("domain fp16-range value, fp32 precision")
    y, f = _run(inp, "unfused", precision="fp32")
    y_ref, f_ref = native.forward(**inp)
    rep = score(y, f, y_ref, f_ref, SHAPE.io)
    # relative to each value's own size: one output near 1e5 has a bf16 spacing of 512, which
    # the RMS-normalised bar of the ordinary workloads cannot absorb
    assert rep["y_rel_floored"] <= 2e-2 and rep["final_rel_floored"] <= 2e-2, rep


@pytest.mark.parametrize("what", ["nan_x", "A_positive", "dt_negative", "fp16_range"])
def test_opt_in_check_rejects(what):
    inp = synth.make_inputs(SHAPE, seed=24)
    if what == "nan_x":
        inp["x"][0, 0, 0, 0] = np.nan
    elif what == "A_positive":
        inp["A"][1] = 0.5
    elif what == "dt_negative":
        inp["dt"][0, 3, 1] = -0.01
    else:
        inp["C"][1, 2, 0, 0] = 70144.0
    d = to_device(inp, SHAPE.io)
    y = torch.full_like(d["x"], 5.0)
    note(f"domain check {what}")
    with pytest.raises(ValueError, match="outside the kernels' domain"):
        ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], SHAPE.chunk_size,
                    d["initial_state"], out=y, check=True)
    torch.cuda.synchronize()
    assert torch.all(y == 5.0), "nothing may be launched"


def test_opt_in_check_accepts_the_workloads_inputs():
    inp = synth.make_inputs(SHAPE, seed=25)
    d = to_device(inp, SHAPE.io)
    note("domain check clean")
    libssd.check_domain(d["x"], d["dt"], d["A"], d["B"], d["C"])
    y, f = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], SHAPE.chunk_size,
                       d["initial_state"], check=True)
    torch.cuda.synchronize()
    y_ref, f_ref = native.forward(**inp)
    assert score(as64(y), as64(f), y_ref, f_ref, SHAPE.io)["pass"]
