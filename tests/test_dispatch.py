"""Which kernels the auto variant launches, read from the kernel count and the per-kernel events
the library records (ssd_options.n_kernels / events): the dispatch rules documented in ssd.h."""

import pytest
import torch

import mamba_ssd_chunked_cumsum_amd as ssd
from mamba_ssd_chunked_cumsum_amd import libssd, synth

from gpu_util import note, to_device

pytestmark = pytest.mark.gpu


def _launch(shape, want_final=True, variant="auto"):
    d = to_device(synth.make_inputs(shape, seed=3), shape.io)
    timer = libssd.KernelTimer()
    note(f"dispatch {shape} want_final={want_final}")
    ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], shape.chunk_size,
                d["initial_state"], variant=variant, want_final=want_final, timer=timer)
    torch.cuda.synchronize()
    return timer.times_ms()


def test_tiny_fp32_takes_the_quadratic_kernel():
    t = _launch(synth.CONFIGS[0])
    assert list(t) == ["quadratic"], t


def test_fp32_beyond_the_quadratic_bounds_takes_the_unfused_kernels():
    # 300 tokens (more than one quadratic block), then 256 tokens x dstate 64 (> 8192 products)
    for shape in (synth.SSDShape("long", 1, 300, 2, 16, 16, 1, 64, io="f32"),
                  synth.SSDShape("wide", 1, 256, 2, 32, 64, 1, 64, io="f32")):
        t = _launch(shape)
        assert list(t) == ["chunk_cumsum", "bmm_chunk", "chunk_state", "state_passing",
                           "chunk_scan"], (shape.name, t)


def test_batched_prefill_runs_without_the_chain():
    # 16 x 10 head blocks fill more than half the device: one run per sequence, no chain kernel
    shape = synth.SSDShape("prefill", 16, 300, 80, 64, 128, 1, 256, init_state=True)
    t = _launch(shape)
    assert list(t) == ["run_state", "state_passing", "fused_scan"], t
    # an empty interval (two events back to back) against the scan kernel's time
    empty = 0.1 * t["fused_scan"]
    assert t["state_passing"] < empty < t["run_state"], t
    t = _launch(shape, want_final=False)
    empty = 0.1 * t["fused_scan"]
    assert t["run_state"] < empty and t["state_passing"] < empty, t


def test_long_bf16_sequence_chains_runs():
    t = _launch(synth.CONFIGS[1])
    assert list(t) == ["run_state", "state_passing", "fused_scan"], t
    assert t["state_passing"] > 0.1 * t["fused_scan"], t       # the chain kernel ran
