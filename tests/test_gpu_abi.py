"""Boundary checks with real device tensors: invalid requests fail with the documented status and
write nothing."""

import pytest
import torch

import mamba_ssd_chunked_cumsum_amd as ssd
from mamba_ssd_chunked_cumsum_amd import libssd, synth

from gpu_util import note, to_device

pytestmark = pytest.mark.gpu


def _inputs():
    shape = synth.config("mamba2_130m_layer").replace(seqlen=128, batch=1, nheads=2)
    return to_device(synth.make_inputs(shape, seed=1), "bf16")


def test_misaligned_and_aliasing_rejected():
    d = _inputs()
    note("abi rejects")
    y = torch.full_like(d["x"], 7.0)
    # y aliasing x
    with pytest.raises(libssd.SSDError) as e:
        ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 64, out=d["x"])
    assert e.value.status == libssd.SSD_ERR_INVALID_ARGUMENT
    # misaligned x (a view offset by one element)
    flat = torch.empty(d["x"].numel() + 8, dtype=d["x"].dtype, device=d["x"].device)
    xm = flat[1:1 + d["x"].numel()].view(d["x"].shape)
    with pytest.raises(libssd.SSDError) as e:
        ssd.forward(xm, d["dt"], d["A"], d["B"], d["C"], d["D"], 64, out=y)
    assert e.value.status == libssd.SSD_ERR_INVALID_ARGUMENT
    # unsupported chunk size
    with pytest.raises(libssd.SSDError) as e:
        ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 48, out=y)
    assert e.value.status == libssd.SSD_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)          # nothing was written


def test_binding_rejects_wrong_dtypes():
    d = _inputs()
    with pytest.raises(ValueError):
        ssd.forward(d["x"], d["dt"].double(), d["A"], d["B"], d["C"], d["D"], 64)
    with pytest.raises(ValueError):
        ssd.forward(d["x"], d["dt"], d["A"], d["B"].float(), d["C"], d["D"], 64)
    with pytest.raises(ValueError):
        ssd.forward(d["x"].transpose(1, 2), d["dt"], d["A"], d["B"], d["C"], d["D"], 64)


def test_kernel_timer_events():
    """Per-kernel timing events recorded by the library around each kernel."""
    d = _inputs()
    note("kernel timer")
    for variant, names in (("fused", ("run_states", "chain", "fused_scan")),
                           ("unfused", ("chunk_cumsum", "bmm_chunk", "chunk_state",
                                        "state_passing", "chunk_scan"))):
        tm = libssd.KernelTimer()
        ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 64, variant=variant,
                    timer=tm)
        torch.cuda.synchronize()
        times = tm.times_ms()
        assert tm.kernels() == names, (variant, tm.kernels())
        assert len(times) == len(names) and all(t >= 0 for t in times.values())
