"""Full forward on the GPU against the float64 oracle (C recurrence) on identical seeded inputs.

Bars: fp32 workloads max |g - r| / max(|r|, RMS(r)) <= 1e-4 for y and final_state; bf16 workloads
y within 2e-2 of RMS beyond the half-ulp of bf16 output rounding, final_state max |g - r| / RMS
<= 2e-2. Full-size workloads are compared on a spread sample of (batch, head) units, every token
of each (RMS over the sampled units), and, on the fused path, the three large bf16 workloads on
every unit.
"""

import numpy as np
import pytest
import torch

import mamba_ssd_chunked_cumsum_amd as ssd
from mamba_ssd_chunked_cumsum_amd import synth
from oracle import metrics, native

from gpu_util import DEV, as64, check_shape, note, run_gpu, score, to_device

pytestmark = pytest.mark.gpu

VARIANTS = ["unfused", "fused"]
FUSED_SHAPES = {(p, n) for p in (64, 128) for n in (64, 128, 256)}   # (headdim, dstate)


def skip_unfusable(shape, variant, precision="auto"):
    if variant != "fused":
        return
    if shape.io != "bf16" or precision == "fp32" or \
            (shape.headdim, shape.dstate) not in FUSED_SHAPES:
        pytest.skip("the fused kernels cover bf16 io with (headdim, dstate) in "
                    f"{sorted(FUSED_SHAPES)}")


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_workloads(cfg, variant):
    shape = synth.CONFIGS[cfg]
    skip_unfusable(shape, variant)
    rep = check_shape(shape, cfg_index=cfg, variant=variant, max_units=8)
    print(cfg, variant, rep)
    assert rep["pass"], rep


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_fused_workloads_every_unit(cfg):
    """The fused path (auto's choice for every bf16 workload) on every (batch, head) unit of the
    three large bf16 workloads; the float64 C oracle takes a few seconds for each."""
    shape = synth.CONFIGS[cfg]
    rep = check_shape(shape, cfg_index=cfg, variant="fused")
    print(cfg, "fused, every unit", rep)
    assert rep["pass"], rep


EDGE = [
    synth.SSDShape("len1", 1, 1, 2, 16, 16, 1, 64),
    synth.SSDShape("shorter_than_chunk", 2, 37, 3, 32, 64, 1, 128, init_state=True),
    synth.SSDShape("ragged_q16", 1, 50, 2, 16, 32, 2, 16),
    synth.SSDShape("ragged_q256", 1, 513, 2, 64, 128, 1, 256, init_state=True),
    synth.SSDShape("n48_p48", 2, 130, 4, 48, 48, 4, 32),
    synth.SSDShape("max_dims", 1, 96, 2, 256, 256, 1, 32, init_state=True),
    synth.SSDShape("f32_ragged", 2, 100, 3, 32, 16, 3, 32, io="f32", init_state=True),
    synth.SSDShape("f32_q256", 1, 600, 2, 64, 64, 1, 256, io="f32"),
    # shapes the fused kernels cover: ragged chunk and run ends, several chunks per run
    synth.SSDShape("p64n128_ragged_q64", 2, 1000, 3, 64, 128, 1, 64, init_state=True),
    synth.SSDShape("p64n64_q32", 1, 777, 4, 64, 64, 2, 32),
    synth.SSDShape("p64n128_q16", 1, 300, 2, 64, 128, 1, 16, init_state=True),
    synth.SSDShape("p64n128_q256_ragged", 1, 1100, 2, 64, 128, 1, 256),
    synth.SSDShape("p128n128_q128", 1, 640, 4, 128, 128, 2, 128, init_state=True),
    synth.SSDShape("p128n256_q128_ragged", 2, 500, 2, 128, 256, 2, 128, random_d=True),
    synth.SSDShape("p128n256_q32", 1, 333, 2, 128, 256, 1, 32),
    synth.SSDShape("p64n256_heads5", 1, 300, 5, 64, 256, 1, 64, init_state=True),
    synth.SSDShape("p128n64_g3", 2, 200, 6, 128, 64, 3, 32, random_d=True),
    # head counts that leave part of a fused block idle, and groups of one head
    synth.SSDShape("p64n128_heads7", 1, 390, 7, 64, 128, 1, 64),
    synth.SSDShape("p64n128_g6", 1, 150, 6, 64, 128, 6, 128, init_state=True),
]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("shape", EDGE, ids=[s.name for s in EDGE])
def test_edge_shapes(shape, variant):
    skip_unfusable(shape, variant)
    rep = check_shape(shape, seed=77, variant=variant)
    assert rep["pass"], rep


RUN_SHAPES = [
    synth.SSDShape("runs_q64", 2, 1000, 3, 64, 128, 1, 64, init_state=True),
    synth.SSDShape("runs_q16_n64", 1, 300, 2, 64, 64, 2, 16),
    synth.SSDShape("runs_q256", 1, 1500, 2, 64, 128, 1, 256, init_state=True),
    synth.SSDShape("runs_p128_n256", 1, 700, 2, 128, 256, 1, 64, random_d=True),
    synth.SSDShape("runs_p128_n128", 1, 512, 2, 128, 128, 2, 32, init_state=True),
]


@pytest.mark.parametrize("run_chunks", [1, 2, 3, 7, 1000])
@pytest.mark.parametrize("shape", RUN_SHAPES, ids=[s.name for s in RUN_SHAPES])
def test_fused_run_lengths(shape, run_chunks):
    """The fused variant with the state carried through runs of 1, 2, 3, 7 and all chunks
    (ragged last runs and chunks included)."""
    rep = check_shape(shape, seed=12, variant="fused", run_chunks=run_chunks)
    assert rep["pass"], rep


# One run per sequence. The plan gives it when the (batch, head block) units alone fill at least
# half the device (16 batch entries x 10 blocks of 8 heads = 160 blocks in the first shape), or
# when asked for runs longer than the sequence; the forward is then the run-state kernel
# completing the final state and the scan kernel starting from the initial state, with no chain
# between runs.
SINGLE_RUN = [
    synth.SSDShape("batched_prefill", 16, 300, 80, 64, 128, 1, 256, init_state=True),
    synth.SSDShape("batched_prefill_q64", 24, 130, 48, 64, 128, 1, 64),
    synth.SSDShape("batched_p128n256", 20, 200, 32, 128, 256, 4, 128, init_state=True),
    synth.SSDShape("batched_p64n64_len40", 40, 40, 64, 64, 64, 2, 32, init_state=True),
]


@pytest.mark.parametrize("precision", ["auto", "fp16"])
@pytest.mark.parametrize("shape", SINGLE_RUN, ids=[s.name for s in SINGLE_RUN])
def test_single_run_plan(shape, precision):
    rep = check_shape(shape, seed=21, variant="fused", precision=precision, max_units=8)
    assert rep["pass"], rep
    if precision == "auto":   # the final state keeps the run-state kernel's hi + lo accuracy
        assert rep["final_rms_literal"] <= 1e-3, rep


def test_single_run_null_state_and_no_final():
    shape = synth.config("mamba2_130m_layer").replace(seqlen=200, batch=2)
    d = to_device(synth.make_inputs(shape, seed=13), "bf16")
    note("single run: null initial state, no final state")
    y0, f0 = run_gpu(d, 64, "fused", run_chunks=1000)
    d["initial_state"] = torch.zeros_like(f0)
    y1, f1 = run_gpu(d, 64, "fused", run_chunks=1000)
    assert torch.equal(y0, y1) and torch.equal(f0, f1)
    y2, f2 = run_gpu(d, 64, "fused", run_chunks=1000, want_final=False)
    assert f2 is None and torch.equal(y2, y1)


def _strong_decay(inp):
    """Decay far beyond fp32's exponent range inside one 16-token block: head 0 everywhere,
    head 1 in bursts of 40 tokens, head 2 left as drawn (the fused kernel's factored decay
    mask must hand such blocks to its direct form)."""
    dt, A = inp["dt"], inp["A"]
    A[:3] = -16.0
    dt[:, :, 0] = 0.5 + dt[:, :, 0]                       # ~8 nats per token
    L = dt.shape[1]
    for t0 in range(17, L, 150):
        dt[:, t0:t0 + 40, 1] = 2.0                        # 32 nats per token
    dt[:, ::37, 2] = 0.0                                  # no decay at some tokens


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("shape", [
    synth.SSDShape("strong_p64n128", 2, 700, 3, 64, 128, 1, 64, init_state=True),
    synth.SSDShape("strong_p128n64_q32", 1, 450, 4, 128, 64, 2, 32),
], ids=lambda s: s.name)
def test_strong_decay(shape, variant):
    skip_unfusable(shape, variant)
    rep = check_shape(shape, seed=31, variant=variant, mutate=_strong_decay)
    assert rep["pass"], rep


@pytest.mark.parametrize("precision", ["fp16", "fp32"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_precision_options(precision, variant):
    shape = synth.config("mamba2_130m_layer").replace(seqlen=512)
    skip_unfusable(shape, variant, precision)
    rep = check_shape(shape, seed=5, variant=variant, precision=precision)
    assert rep["pass"], rep
    if precision == "fp32":
        assert rep["y_rms_r1"] <= 1e-3 and rep["final_rms_literal"] <= 1e-4


@pytest.mark.parametrize("variant", VARIANTS)
def test_null_initial_state_equals_zeros_and_no_final(variant):
    shape = synth.config("mamba2_130m_layer").replace(seqlen=300, batch=1)
    inp = synth.make_inputs(shape, seed=3)
    d = to_device(inp, "bf16")
    note(f"null-vs-zero {variant}")
    y0, f0 = run_gpu(d, 64, variant)
    d["initial_state"] = torch.zeros_like(f0)
    y1, f1 = run_gpu(d, 64, variant)
    assert torch.equal(y0, y1) and torch.equal(f0, f1)
    d["initial_state"] = None
    y2, f2 = run_gpu(d, 64, variant, want_final=False)
    assert f2 is None and torch.equal(y2, y0)


@pytest.mark.parametrize("variant", VARIANTS)
def test_deterministic(variant):
    shape = synth.config("mamba2_130m_layer").replace(seqlen=1024)
    d = to_device(synth.make_inputs(shape, seed=8), "bf16")
    note(f"determinism {variant}")
    ya, fa = run_gpu(d, 64, variant)
    yb, fb = run_gpu(d, 64, variant)
    assert torch.equal(ya, yb) and torch.equal(fa, fb)


@pytest.mark.parametrize("variant", VARIANTS)
def test_zero_readout_gives_skip_exactly(variant):
    shape = synth.config("mamba2_130m_layer").replace(seqlen=256, batch=1)
    inp = synth.make_inputs(shape, seed=4)
    inp["C"] = np.zeros_like(inp["C"])
    d = to_device(inp, "bf16")
    note(f"C=0 {variant}")
    y, _ = run_gpu(d, 64, variant)
    if variant == "unfused":
        assert torch.equal(y, d["x"])      # D = 1, so y = x bit for bit
        return
    # The fused scan carries D x through the fp16 diagonal of the masked C B^T block: bit for bit
    # wherever x is an fp16 normal number, within fp16's subnormal spacing (2^-24) below that.
    yf, xf = y.float(), d["x"].float()
    normal = xf.abs() >= 2.0 ** -14
    assert torch.equal(yf[normal], xf[normal])
    assert float((yf - xf).abs().max()) <= 2.0 ** -24


@pytest.mark.parametrize("variant", VARIANTS)
def test_causality(variant):
    shape = synth.config("mamba2_130m_layer").replace(seqlen=256, batch=1)
    inp = synth.make_inputs(shape, seed=6)
    d = to_device(inp, "bf16")
    note(f"causality {variant}")
    ya, _ = run_gpu(d, 64, variant)
    t0 = 150
    d["x"][:, t0] += 3.0
    yb, _ = run_gpu(d, 64, variant)
    assert torch.equal(ya[:, :t0], yb[:, :t0])
    assert not torch.equal(ya[:, t0:], yb[:, t0:])


@pytest.mark.parametrize("variant", VARIANTS)
def test_chunk_size_invariance_and_state_composition(variant):
    shape = synth.config("mamba2_130m_layer").replace(seqlen=700, batch=2, nheads=6, init_state=True)
    inp = synth.make_inputs(shape, seed=9)
    y_ref, f_ref = native.forward(**inp)
    d = to_device(inp, "bf16")
    note(f"Q invariance {variant}")
    for Q in (16, 64, 256):
        y, f = run_gpu(d, Q, variant)
        rep = score(as64(y), as64(f), y_ref, f_ref, "bf16")
        assert rep["pass"], (Q, rep)
    L1 = 333
    first = {k: (v[:, :L1].contiguous() if k in ("x", "dt", "B", "C") else v)
             for k, v in d.items()}
    second = {k: (v[:, L1:].contiguous() if k in ("x", "dt", "B", "C") else v)
              for k, v in d.items()}
    ya, fa = run_gpu(first, 64, variant)
    second["initial_state"] = fa
    yb, fb = run_gpu(second, 64, variant)
    rep = score(as64(torch.cat([ya, yb], 1)), as64(fb), y_ref, f_ref, "bf16")
    assert rep["pass"], rep


@pytest.mark.parametrize("variant", VARIANTS)
def test_group_replication(variant):
    shape = synth.SSDShape("g", 1, 200, 4, 64, 64, 1, 64)
    inp = synth.make_inputs(shape, seed=10)
    d = to_device(inp, "bf16")
    note(f"group replication {variant}")
    y1, f1 = run_gpu(d, 64, variant)
    d["B"] = d["B"].repeat(1, 1, 4, 1).contiguous()
    d["C"] = d["C"].repeat(1, 1, 4, 1).contiguous()
    y2, f2 = run_gpu(d, 64, variant)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


DT_SHAPES = [
    synth.SSDShape("dt_p64n128_ragged", 2, 700, 4, 64, 128, 1, 64, init_state=True),
    synth.SSDShape("dt_f32", 1, 300, 3, 32, 32, 1, 64, io="f32"),
]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("clamp", [False, True])
@pytest.mark.parametrize("shape", DT_SHAPES, ids=[s.name for s in DT_SHAPES])
def test_dt_preprocessing(shape, clamp, variant):
    """dt passed raw, with a per-head bias, softplus and (optionally) a clamp applied inside the
    kernels, against the oracle run on the effective dt."""
    from oracle import dt_effective
    skip_unfusable(shape, variant)
    inp = synth.make_inputs(shape, seed=41)
    rng = np.random.default_rng(42)
    raw = rng.normal(-2.5, 1.0, inp["dt"].shape).astype(np.float32)
    bias = rng.uniform(-1.0, 1.0, shape.nheads).astype(np.float32)
    lim = (0.02, 0.2) if clamp else None
    eff = dt_effective(raw, bias, True, *(lim or (0.0, 0.0)))
    note(f"{shape} dt pre-processing clamp={clamp} variant={variant}")
    dinp = to_device(inp, shape.io)
    y, f = ssd.forward(dinp["x"], torch.from_numpy(raw).to(DEV), dinp["A"], dinp["B"], dinp["C"],
                       dinp["D"], shape.chunk_size, dinp["initial_state"], variant=variant,
                       dt_bias=torch.from_numpy(bias).to(DEV), dt_softplus=True, dt_limit=lim)
    torch.cuda.synchronize()
    ref = dict(inp, dt=eff.astype(np.float32))
    y_ref, f_ref = native.forward(**ref)
    rep = score(as64(y), as64(f), y_ref, f_ref, shape.io)
    assert rep["pass"], rep
