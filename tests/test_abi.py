"""C-ABI boundary without a GPU: the library loads, exports every symbol include/ssd.h declares,
and rejects invalid requests on the host before any HIP call.

Calls here pass placeholder (never dereferenced) addresses, so they run only where no GPU is
visible; on a GPU machine the validation paths are exercised with real tensors by test_gpu_abi.py.
"""

import ctypes
import os
import re

import pytest
import torch

from mamba_ssd_chunked_cumsum_amd import libssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="placeholder-pointer checks run only without a visible GPU")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_0-9]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = libssd.load()
    names = declared_functions()
    assert "ssd_forward" in names and "ssd_status_string" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ssd.h but not exported"
    assert set(names) == set(libssd.EXPORTS)


def test_version_and_status_strings():
    assert libssd.version() == 10500
    assert libssd.status_string(0) == "ok"
    assert libssd.status_string(3) == "no HIP device"
    assert libssd.status_string(99) == "unknown status"


def test_struct_layout_matches_header():
    assert ctypes.sizeof(libssd.SSDProblem) == 6 * 8 + 2 * 4
    assert ctypes.sizeof(libssd.SSDOptions) == 64


# placeholder device addresses: 16-byte aligned, far apart, never dereferenced
BASE = 1 << 40
SPAN = 1 << 34


def addr(i, extra=0):
    return ctypes.c_void_p(BASE + i * SPAN + extra)


def good_problem(**kw):
    p = dict(batch=2, seqlen=100, nheads=4, headdim=16, dstate=32, ngroups=2, io_dtype=1)
    p.update(kw)
    return libssd.problem(p["batch"], p["seqlen"], p["nheads"], p["headdim"], p["dstate"],
                          p["ngroups"], p["io_dtype"])


def call_forward(prob, Q=64, ptrs=None, opts=None):
    a = [addr(i) for i in range(9)] if ptrs is None else ptrs
    x, dt, A, B, C, D, h0, y, fin = a
    lib = libssd.load()
    o = ctypes.byref(opts) if opts is not None else None
    return lib.ssd_forward_ex(ctypes.byref(prob) if prob is not None else None, x, dt, A, B, C,
                              D, Q, h0, y, fin, None, o)


@no_gpu
def test_valid_request_reports_no_device():
    assert call_forward(good_problem()) == libssd.SSD_ERR_NO_DEVICE
    lib = libssd.load()
    assert lib.ssd_forward(ctypes.byref(good_problem()), *[addr(i) for i in range(6)], 64, None,
                           addr(7), None, None) == libssd.SSD_ERR_NO_DEVICE


@no_gpu
@pytest.mark.parametrize("field,value", [("batch", 0), ("seqlen", -1), ("nheads", 0),
                                         ("headdim", 0), ("dstate", -5), ("ngroups", 0),
                                         ("ngroups", 3), ("io_dtype", 7)])
def test_invalid_problem(field, value):
    assert call_forward(good_problem(**{field: value})) == libssd.SSD_ERR_INVALID_ARGUMENT


@no_gpu
def test_null_problem_and_reserved():
    assert call_forward(None) == libssd.SSD_ERR_INVALID_ARGUMENT
    p = good_problem()
    p.reserved = 1
    assert call_forward(p) == libssd.SSD_ERR_INVALID_ARGUMENT


@no_gpu
@pytest.mark.parametrize("Q,status", [(0, 1), (-64, 1), (8, 2), (48, 2), (512, 2), (16, 3),
                                      (32, 3), (256, 3)])
def test_chunk_size(Q, status):
    assert call_forward(good_problem(), Q=Q) == status


@no_gpu
@pytest.mark.parametrize("kw", [dict(headdim=24), dict(headdim=272), dict(dstate=8),
                                dict(dstate=512), dict(batch=1 << 20, seqlen=1 << 12)])
def test_unsupported_shapes(kw):
    assert call_forward(good_problem(**kw)) == libssd.SSD_ERR_UNSUPPORTED


@no_gpu
@pytest.mark.parametrize("which", range(7))
def test_null_required_pointer(which):
    ptrs = [addr(i) for i in range(9)]
    idx = [0, 1, 2, 3, 4, 5, 7][which]   # x, dt, A, B, C, D, y
    ptrs[idx] = None
    assert call_forward(good_problem(), ptrs=ptrs) == libssd.SSD_ERR_INVALID_ARGUMENT


@no_gpu
def test_optional_pointers_may_be_null():
    ptrs = [addr(i) for i in range(9)]
    ptrs[6] = ptrs[8] = None
    assert call_forward(good_problem(), ptrs=ptrs) == libssd.SSD_ERR_NO_DEVICE


@no_gpu
@pytest.mark.parametrize("which", range(9))
def test_misaligned_pointer(which):
    ptrs = [addr(i) for i in range(9)]
    ptrs[which] = addr(which, 4)
    assert call_forward(good_problem(), ptrs=ptrs) == libssd.SSD_ERR_INVALID_ARGUMENT


@no_gpu
@pytest.mark.parametrize("alias_of", [0, 1, 2, 3, 4, 5, 6])
def test_output_aliasing_rejected(alias_of):
    ptrs = [addr(i) for i in range(9)]
    ptrs[7] = ptrs[alias_of]                                   # y overlaps an input
    assert call_forward(good_problem(), ptrs=ptrs) == libssd.SSD_ERR_INVALID_ARGUMENT
    ptrs[7] = ctypes.c_void_p(ptrs[alias_of].value - 16)       # partial overlap from below
    assert call_forward(good_problem(), ptrs=ptrs) == libssd.SSD_ERR_INVALID_ARGUMENT
    ptrs = [addr(i) for i in range(9)]
    ptrs[8] = ptrs[alias_of]                                   # final_state overlaps an input
    assert call_forward(good_problem(), ptrs=ptrs) == libssd.SSD_ERR_INVALID_ARGUMENT


@no_gpu
def test_final_overlapping_y_rejected():
    ptrs = [addr(i) for i in range(9)]
    ptrs[8] = ptrs[7]
    assert call_forward(good_problem(), ptrs=ptrs) == libssd.SSD_ERR_INVALID_ARGUMENT


@no_gpu
def test_adjacent_buffers_are_not_aliasing():
    # y placed exactly after x: x occupies batch*seqlen*nheads*headdim*2 bytes
    p = good_problem()
    xbytes = 2 * 100 * 4 * 16 * 2
    ptrs = [addr(i) for i in range(9)]
    ptrs[7] = ctypes.c_void_p(ptrs[0].value + xbytes)
    assert call_forward(p, ptrs=ptrs) == libssd.SSD_ERR_NO_DEVICE


@no_gpu
@pytest.mark.parametrize("variant,precision,status", [(0, 0, 3), (1, 1, 3), (1, 3, 3), (3, 0, 3),
                                                      (4, 0, 1), (-1, 0, 1), (0, 2, 1), (0, 9, 1)])
def test_options(variant, precision, status):
    assert call_forward(good_problem(),
                        opts=libssd.SSDOptions(variant, precision, 0, 0, None, None)) == status


@no_gpu
def test_negative_run_chunks_rejected():
    assert call_forward(good_problem(), opts=libssd.SSDOptions(2, 0, -1, 0, None, None)) == 1
    assert call_forward(good_problem(), opts=libssd.SSDOptions(2, 0, 3, 0, None, None)) == 3


@no_gpu
def test_event_options_checked():
    ev = (ctypes.c_void_p * 6)()
    evp = ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p))
    assert call_forward(good_problem(), opts=libssd.SSDOptions(0, 0, 0, 6, None, None)) == 1
    assert call_forward(good_problem(), opts=libssd.SSDOptions(0, 0, 0, 5, evp, None)) == 1
    assert call_forward(good_problem(), opts=libssd.SSDOptions(0, 0, 0, -1, evp, None)) == 1
    assert call_forward(good_problem(), opts=libssd.SSDOptions(0, 0, 0, 6, evp, None)) == 3


@no_gpu
def test_stage_entry_points_validate_before_device():
    lib = libssd.load()
    p = good_problem()
    a = [addr(i) for i in range(8)]
    assert lib.ssd_chunk_cumsum(ctypes.byref(p), a[0], a[1], 64, a[2], a[3], None) == 3
    assert lib.ssd_chunk_cumsum(ctypes.byref(p), a[0], a[1], 63, a[2], a[3], None) == 2
    assert lib.ssd_chunk_cumsum(ctypes.byref(p), a[0], a[1], 64, a[2], a[2], None) == 1
    assert lib.ssd_bmm_chunk(ctypes.byref(p), a[0], a[1], 64, None, None) == 1
    assert lib.ssd_bmm_chunk(ctypes.byref(p), a[0], a[1], 64, a[2], None) == 3
    assert lib.ssd_chunk_state(ctypes.byref(p), a[0], a[1], a[2], a[3], 64, a[4], None,
                               None) == 3
    assert lib.ssd_state_passing(ctypes.byref(p), a[0], a[1], 64, None, a[0], None, None) == 1
    assert lib.ssd_state_passing(ctypes.byref(p), a[0], a[1], 64, None, a[2], None, None) == 3
    assert lib.ssd_chunk_scan(ctypes.byref(p), a[0], a[1], a[2], a[3], a[4], a[5], a[6], 64,
                              a[0], None, None) == 1
    assert lib.ssd_chunk_scan(ctypes.byref(p), a[0], a[1], a[2], a[3], a[4], a[5], a[6], 64,
                              a[7], None, None) == 3


def test_workspace_sizes():
    p = good_problem()
    s = libssd.workspace_sizes(p, 64)
    nc = 2
    assert s == [2 * 4 * nc * 64 * 4, 2 * 4 * nc * 64 * 4, 2 * nc * 2 * 64 * 64 * 4,
                 2 * nc * 4 * 16 * 32 * 4, 2 * nc * 4 * 16 * 32 * 4]
    with pytest.raises(libssd.SSDError):
        libssd.workspace_sizes(p, 24)


# ---- ssd_step (single-token decode step) ----------------------------------------------------------

def call_step(prob, ptrs=None):
    a = [addr(i) for i in range(10)] if ptrs is None else ptrs
    x, dt, A, B, C, D, s_in, s_out, y = a[:9]
    lib = libssd.load()
    return lib.ssd_step(ctypes.byref(prob) if prob is not None else None, x, dt, A, B, C, D,
                        s_in, s_out, y, None)


@no_gpu
def test_step_valid_request_reports_no_device():
    assert call_step(good_problem(seqlen=1)) == libssd.SSD_ERR_NO_DEVICE


@no_gpu
def test_step_in_place_state_is_valid():
    ptrs = [addr(i) for i in range(10)]
    ptrs[7] = ptrs[6]
    assert call_step(good_problem(seqlen=1), ptrs=ptrs) == libssd.SSD_ERR_NO_DEVICE


@no_gpu
@pytest.mark.parametrize("kw,status", [(dict(seqlen=2), 1), (dict(seqlen=0), 1),
                                       (dict(nheads=3), 1), (dict(headdim=24), 2),
                                       (dict(dstate=512), 2)])
def test_step_invalid_problem(kw, status):
    kw.setdefault("seqlen", 1)
    assert call_step(good_problem(**kw)) == status


@no_gpu
@pytest.mark.parametrize("which", range(9))
def test_step_null_or_misaligned_pointer(which):
    ptrs = [addr(i) for i in range(10)]
    ptrs[which] = None
    assert call_step(good_problem(seqlen=1), ptrs=ptrs) == libssd.SSD_ERR_INVALID_ARGUMENT
    ptrs = [addr(i) for i in range(10)]
    ptrs[which] = addr(which, 4)
    assert call_step(good_problem(seqlen=1), ptrs=ptrs) == libssd.SSD_ERR_INVALID_ARGUMENT


@no_gpu
@pytest.mark.parametrize("out,alias_of", [(8, i) for i in range(8)] + [(7, i) for i in range(6)])
def test_step_output_aliasing_rejected(out, alias_of):
    """y (8) may overlap nothing; state_out (7) no input (x, dt, A, B, C, D)."""
    ptrs = [addr(i) for i in range(10)]
    ptrs[out] = addr(alias_of)  # starts where the other buffer starts
    assert call_step(good_problem(seqlen=1), ptrs=ptrs) == libssd.SSD_ERR_INVALID_ARGUMENT


@no_gpu
def test_step_partial_state_overlap_rejected():
    ptrs = [addr(i) for i in range(10)]
    ptrs[7] = addr(6, 16)
    assert call_step(good_problem(seqlen=1), ptrs=ptrs) == libssd.SSD_ERR_INVALID_ARGUMENT


# ---- dt pre-processing options -------------------------------------------------------------------

def dt_opts(**kw):
    o = libssd._options("auto", "auto")
    for k, v in kw.items():
        setattr(o, k, v)
    return o


@no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(dt_softplus=1), 3), (dict(dt_min=0.1, dt_max=2.0), 3), (dict(dt_max=0.0, dt_min=5.0), 3),
    (dict(dt_bias=BASE + 20 * SPAN), 3),
    (dict(dt_max=-1.0), 1), (dict(dt_min=3.0, dt_max=2.0), 1), (dict(dt_max=float("nan")), 1),
    (dict(dt_min=float("nan"), dt_max=1.0), 1), (dict(dt_bias=BASE + 20 * SPAN + 4), 1),
])
def test_dt_options_checked(kw, status):
    assert call_forward(good_problem(), opts=dt_opts(**kw)) == status


@no_gpu
def test_dt_bias_may_not_overlap_outputs():
    ptrs = [addr(i) for i in range(9)]
    assert call_forward(good_problem(), ptrs=ptrs, opts=dt_opts(dt_bias=ptrs[7].value)) == 1
    assert call_forward(good_problem(), ptrs=ptrs, opts=dt_opts(dt_bias=ptrs[8].value)) == 1


# ---- ssd_backward -----------------------------------------------------------------------------

def call_backward(prob, Q=64, ptrs=None):
    # x, dt, A, B, C, D, h0, dy, dfinal, dx, ddt, dA, dB, dC, dD, dh0
    a = [addr(i) for i in range(16)] if ptrs is None else ptrs
    lib = libssd.load()
    return lib.ssd_backward(ctypes.byref(prob), a[0], a[1], a[2], a[3], a[4], a[5], Q, a[6],
                            a[7], a[8], a[9], a[10], a[11], a[12], a[13], a[14], a[15], None)


@no_gpu
def test_backward_valid_request_reports_no_device():
    assert call_backward(good_problem()) == libssd.SSD_ERR_NO_DEVICE
    ptrs = [addr(i) for i in range(16)]
    ptrs[6] = ptrs[8] = ptrs[15] = None          # initial state, dfinal, its gradient: optional
    assert call_backward(good_problem(), ptrs=ptrs) == libssd.SSD_ERR_NO_DEVICE


@no_gpu
@pytest.mark.parametrize("which", [0, 1, 2, 3, 4, 5, 7, 9, 10, 11, 12, 13, 14])
def test_backward_null_required_pointer(which):
    ptrs = [addr(i) for i in range(16)]
    ptrs[which] = None
    assert call_backward(good_problem(), ptrs=ptrs) == libssd.SSD_ERR_INVALID_ARGUMENT


@no_gpu
@pytest.mark.parametrize("out,alias_of", [(9, 0), (9, 7), (12, 3), (13, 4), (11, 2), (15, 6),
                                          (10, 9), (13, 12)])
def test_backward_output_aliasing_rejected(out, alias_of):
    ptrs = [addr(i) for i in range(16)]
    ptrs[out] = ptrs[alias_of]
    assert call_backward(good_problem(), ptrs=ptrs) == libssd.SSD_ERR_INVALID_ARGUMENT


@no_gpu
def test_backward_misaligned_and_unsupported():
    ptrs = [addr(i) for i in range(16)]
    ptrs[7] = addr(7, 4)
    assert call_backward(good_problem(), ptrs=ptrs) == libssd.SSD_ERR_INVALID_ARGUMENT
    assert call_backward(good_problem(headdim=24)) == libssd.SSD_ERR_UNSUPPORTED
