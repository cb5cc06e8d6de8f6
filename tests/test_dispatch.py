"""Which kernels the auto variant launches, read from the kernel count and the per-kernel events
the library records (ssd_options.n_kernels / events): the dispatch rules documented in ssd.h."""

import pytest
import torch

import mamba_ssd_chunked_cumsum_amd as ssd
from mamba_ssd_chunked_cumsum_amd import libssd, synth

from gpu_util import note, to_device

pytestmark = pytest.mark.gpu


def _launch(shape, want_final=True, variant="auto"):
    """Per-kernel event intervals of one call, after an untimed call of the same problem (the
    first calls of a process show event gaps of several microseconds)."""
    d = to_device(synth.make_inputs(shape, seed=3), shape.io)
    note(f"dispatch {shape} want_final={want_final}")
    for timer in (None, libssd.KernelTimer()):
        ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], shape.chunk_size,
                    d["initial_state"], variant=variant, want_final=want_final, timer=timer)
        torch.cuda.synchronize()
    return timer.times_ms()


# An empty interval (two events recorded back to back) against the scan kernel's time, and the
# share a kernel that ran takes at least at these shapes (run states and the chain take 30% or
# more of the scan's time there; an empty interval has measured below 11%).
EMPTY, RAN = 0.25, 0.3


def test_tiny_fp32_takes_the_quadratic_kernel():
    t = _launch(synth.config("tiny_fp32"))
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
    assert t["state_passing"] < EMPTY * t["fused_scan"], t
    assert t["run_state"] > RAN * t["fused_scan"], t
    t = _launch(shape, want_final=False)
    assert max(t["run_state"], t["state_passing"]) < EMPTY * t["fused_scan"], t


def test_long_bf16_sequence_chains_runs():
    t = _launch(synth.config("mamba2_130m_layer"))
    assert list(t) == ["run_state", "state_passing", "fused_scan"], t
    assert t["state_passing"] > RAN * t["fused_scan"], t       # the chain kernel ran
