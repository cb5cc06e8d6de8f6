"""ssd_forward_noalloc, the forward that allocates nothing (workspace from the library's static
per-device scratch), against ssd_forward_ex through the C ABI: two calls in a row, the second on a
smaller input, each compared with ssd_forward_ex's output on the same inputs; a plan fitted to the
scratch (runs lengthened) held to the parity bar against the oracle, as ssd_forward_ex is; the
unfused path within the scratch; and an unfused request beyond it rejected with nothing written."""

import numpy as np
import pytest
import torch

import mamba_ssd_chunked_cumsum_amd as ssd
from mamba_ssd_chunked_cumsum_amd import libssd, synth
from oracle import native

from gpu_util import as64, note, score, to_device

pytestmark = pytest.mark.gpu


def _run(shape, seed, noalloc, variant="auto", run_chunks=0):
    d = to_device(synth.make_inputs(shape, seed=seed), shape.io)
    y = torch.full_like(d["x"], 3.0)
    fin = torch.full((shape.batch, shape.nheads, shape.headdim, shape.dstate), 3.0,
                     dtype=torch.float32, device=d["x"].device)
    tm = libssd.KernelTimer()
    ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], shape.chunk_size,
                d["initial_state"], variant=variant, out=y, final_out=fin, noalloc=noalloc,
                timer=tm, run_chunks=run_chunks)
    torch.cuda.synchronize()
    return y, fin, tm.kernels()


CHAINED = [
    # several runs per sequence, workspace within the scratch: the same plan, bitwise equal
    synth.SSDShape("noalloc_big", 2, 2048, 16, 64, 128, 1, 64, init_state=True),
    synth.SSDShape("noalloc_small", 1, 500, 8, 64, 128, 2, 64),
]


def test_two_calls_in_a_row_match_the_allocating_forward():
    for shape in CHAINED:  # the second call is smaller, on the scratch the first one left
        note(f"noalloc {shape}")
        y0, f0, k0 = _run(shape, 5, noalloc=False)
        y1, f1, k1 = _run(shape, 5, noalloc=True)
        assert k0 == k1 == ("run_states", "chain", "fused_scan"), (k0, k1)
        assert torch.equal(y0, y1) and torch.equal(f0, f1), shape.name


def test_plan_fitted_to_the_scratch():
    # headdim 128, dstate 256, runs of one 128-token chunk: 32 runs per sequence, two sequences,
    # would need 2 x 31 x 2 MiB of fp16 run states (all but the last run's) plus the decays; the
    # no-allocation plan doubles the run length, so the numbers differ from the allocating
    # forward's only by rounding
    shape = synth.SSDShape("noalloc_fitted", 2, 4096, 32, 128, 256, 1, 128, init_state=True)
    note(f"noalloc fitted {shape}")
    y0, f0, _ = _run(shape, 9, noalloc=False, run_chunks=1)
    y1, f1, _ = _run(shape, 9, noalloc=True, run_chunks=1)
    assert not torch.equal(y0, y1)  # a different cut of the sequence
    # both held to the parity bar against the oracle (two bf16 outputs of different plans may
    # differ by a rounding of each, which the bar's half-ulp allowance covers only once)
    inp = synth.make_inputs(shape, seed=9)
    units = [0, 13, 31, 50, 63]
    y_ref, f_ref = native.forward(**inp, units=units)
    for y, f in ((y0, f0), (y1, f1)):
        rep = score(as64(y), as64(f), y_ref, f_ref, "bf16", units, shape.nheads)
        assert rep["pass"], rep


def test_unfused_within_and_beyond_the_scratch():
    shape = synth.SSDShape("noalloc_f32", 2, 300, 3, 32, 16, 3, 32, io="f32", init_state=True)
    note(f"noalloc unfused {shape}")
    y0, f0, _ = _run(shape, 4, noalloc=False, variant="unfused")
    y1, f1, k1 = _run(shape, 4, noalloc=True, variant="unfused")
    assert len(k1) == 5 and torch.equal(y0, y1) and torch.equal(f0, f1)
    # 64 chunks x 32 heads x 64 x 128 fp32 states alone are 64 MiB
    big = synth.SSDShape("noalloc_f32_big", 1, 4096, 32, 64, 128, 1, 64, io="f32")
    d = to_device(synth.make_inputs(big, seed=4), "f32")
    y = torch.full_like(d["x"], 3.0)
    with pytest.raises(libssd.SSDError) as e:
        ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 64, variant="unfused",
                    out=y, noalloc=True)
    assert e.value.status == libssd.SSD_ERR_WORKSPACE_LIMIT
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)
