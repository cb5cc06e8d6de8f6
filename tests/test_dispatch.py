"""Which kernels the auto variant launches, read from the kernel mask the library reports
(ssd_options.kernel_mask; the kernels it names were launched in increasing bit order): the
dispatch rules documented in ssd.h."""

import pytest
import torch

import mamba_ssd_chunked_cumsum_amd as ssd
from mamba_ssd_chunked_cumsum_amd import libssd, synth

from gpu_util import note, to_device

pytestmark = pytest.mark.gpu


def _launch(shape, want_final=True, variant="auto"):
    """Kernel names and per-kernel event intervals of one call."""
    d = to_device(synth.make_inputs(shape, seed=3), shape.io)
    note(f"dispatch {shape} want_final={want_final}")
    timer = libssd.KernelTimer()
    ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], shape.chunk_size,
                d["initial_state"], variant=variant, want_final=want_final, timer=timer)
    torch.cuda.synchronize()
    times = timer.times_ms()
    assert timer.n_kernels.value == len(timer.kernels())
    assert all(t >= 0 for t in times.values())
    return timer.kernels()


def test_tiny_fp32_takes_the_quadratic_kernel():
    assert _launch(synth.config("tiny_fp32")) == ("quadratic",)


def test_fp32_beyond_the_quadratic_bounds_takes_the_unfused_kernels():
    # 300 tokens (more than one quadratic block), then 256 tokens x dstate 64 (> 8192 products)
    for shape in (synth.SSDShape("long", 1, 300, 2, 16, 16, 1, 64, io="f32"),
                  synth.SSDShape("wide", 1, 256, 2, 32, 64, 1, 64, io="f32")):
        assert _launch(shape) == ("chunk_cumsum", "bmm_chunk", "chunk_state", "state_passing",
                                  "chunk_scan"), shape.name


def test_batched_prefill_runs_without_the_chain():
    # 16 x 10 head blocks fill more than half the device: one run per sequence, so no chain; the
    # run-state kernel only for the final state
    shape = synth.SSDShape("prefill", 16, 300, 80, 64, 128, 1, 256, init_state=True)
    assert _launch(shape) == ("run_states", "fused_scan")
    assert _launch(shape, want_final=False) == ("fused_scan",)


def test_long_bf16_sequence_chains_runs():
    shape = synth.config("mamba2_130m_layer")
    assert _launch(shape) == ("run_states", "chain", "fused_scan")
    assert _launch(shape, want_final=False) == ("run_states", "chain", "fused_scan")


def test_unfused_request_on_a_fusable_shape():
    shape = synth.config("mamba2_130m_layer").replace(seqlen=256)
    assert _launch(shape, variant="unfused") == ("chunk_cumsum", "bmm_chunk", "chunk_state",
                                                 "state_passing", "chunk_scan")
