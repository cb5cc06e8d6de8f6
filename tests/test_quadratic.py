"""The quadratic variant (one kernel, the whole sequence as one masked block) on the GPU against
the float64 oracle on identical seeded inputs.

It computes in fp32 whatever the io type, so beyond the workloads' bars (fp32 io: 1e-4 relative;
bf16 io: y within 2e-2 of RMS beyond bf16 output rounding, final state 2e-2) it is held to fp32
accuracy: for bf16 io the y error left after the output's own rounding, and the final state's
error, both at most 1e-4 of RMS (fp32 rounding accumulated over a few hundred terms is ~1e-6).
"""

import numpy as np
import pytest
import torch

import mamba_ssd_chunked_cumsum_amd as ssd
from mamba_ssd_chunked_cumsum_amd import synth
from oracle import native

from gpu_util import DEV, as64, check_shape, note, run_gpu, score, to_device

pytestmark = pytest.mark.gpu

FP32_BAR = 1e-4

QUAD_SHAPES = [
    synth.config("tiny_fp32"),                                                        # tiny fp32 workload
    synth.SSDShape("len1", 1, 1, 2, 16, 16, 1, 64, init_state=True),
    synth.SSDShape("len256_p64n128", 2, 256, 4, 64, 128, 1, 64, init_state=True),
    synth.SSDShape("ragged_p48n48_g2", 2, 130, 4, 48, 48, 2, 32, io="f32", init_state=True),
    synth.SSDShape("p80_two_tiles", 1, 200, 3, 80, 64, 3, 64, random_d=True),
    synth.SSDShape("n256_tile32", 1, 150, 2, 64, 256, 1, 128, init_state=True),
    synth.SSDShape("n144_p256_f32", 1, 97, 2, 256, 144, 1, 16, io="f32", init_state=True),
    synth.SSDShape("len64_p32n16", 3, 64, 6, 32, 16, 2, 64, io="f32"),
    synth.SSDShape("len255_f32", 1, 255, 2, 16, 32, 1, 256, io="f32", init_state=True),
]


def _check(rep, io):
    assert rep["pass"], rep
    if io == "bf16":
        assert rep["y_rms_r1"] <= FP32_BAR and rep["final_rms_literal"] <= FP32_BAR, rep


@pytest.mark.parametrize("shape", QUAD_SHAPES, ids=[s.name for s in QUAD_SHAPES])
def test_quadratic_matches_oracle(shape):
    rep = check_shape(shape, seed=51, variant="quadratic")
    print(shape.name, rep)
    _check(rep, shape.io)


def _strong_decay(inp):
    """Decay far beyond fp32's exponent range between distant tokens (head 0), in bursts (head
    1), and tokens with no decay at all (head 2)."""
    dt, A = inp["dt"], inp["A"]
    A[:3] = -16.0
    dt[:, :, 0] = 0.5 + dt[:, :, 0]
    dt[:, 40:80, 1] = 2.0
    dt[:, ::7, 2] = 0.0


def test_quadratic_strong_decay():
    shape = synth.SSDShape("strong", 1, 200, 3, 64, 64, 1, 64, init_state=True)
    rep = check_shape(shape, seed=52, variant="quadratic", mutate=_strong_decay)
    _check(rep, shape.io)


@pytest.mark.parametrize("clamp", [False, True])
def test_quadratic_dt_preprocessing(clamp):
    from oracle import dt_effective
    shape = synth.SSDShape("dt_quad", 2, 180, 4, 64, 128, 2, 64, init_state=True)
    inp = synth.make_inputs(shape, seed=53)
    rng = np.random.default_rng(54)
    raw = rng.normal(-2.5, 1.0, inp["dt"].shape).astype(np.float32)
    bias = rng.uniform(-1.0, 1.0, shape.nheads).astype(np.float32)
    lim = (0.02, 0.2) if clamp else None
    eff = dt_effective(raw, bias, True, *(lim or (0.0, 0.0)))
    note(f"quadratic dt pre-processing clamp={clamp}")
    d = to_device(inp, shape.io)
    y, f = ssd.forward(d["x"], torch.from_numpy(raw).to(DEV), d["A"], d["B"], d["C"], d["D"],
                       shape.chunk_size, d["initial_state"], variant="quadratic",
                       dt_bias=torch.from_numpy(bias).to(DEV), dt_softplus=True, dt_limit=lim)
    torch.cuda.synchronize()
    y_ref, f_ref = native.forward(**dict(inp, dt=eff.astype(np.float32)))
    _check(score(as64(y), as64(f), y_ref, f_ref, shape.io), shape.io)


def test_quadratic_no_final_and_null_state():
    shape = synth.SSDShape("nf", 2, 120, 4, 64, 64, 1, 64)
    d = to_device(synth.make_inputs(shape, seed=55), shape.io)
    note("quadratic: null initial state, no final state")
    y0, f0 = run_gpu(d, 64, "quadratic")
    d["initial_state"] = torch.zeros_like(f0)
    y1, f1 = run_gpu(d, 64, "quadratic")
    assert torch.equal(y0, y1) and torch.equal(f0, f1)
    y2, f2 = run_gpu(d, 64, "quadratic", want_final=False)
    assert f2 is None and torch.equal(y2, y1)


def test_quadratic_rejects_long_sequences():
    shape = synth.SSDShape("long", 1, 257, 2, 16, 16, 1, 64, io="f32")
    d = to_device(synth.make_inputs(shape, seed=56), shape.io)
    note("quadratic: seqlen 257 rejected")
    with pytest.raises(ssd.SSDError):
        run_gpu(d, 64, "quadratic")
