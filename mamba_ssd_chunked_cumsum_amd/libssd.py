"""Python binding of libssd (ctypes). Argument marshalling only: every step of the forward runs
in the library's HIP kernels; torch provides device memory and the current stream.

The library must have been built (``python -m mamba_ssd_chunked_cumsum_amd.build``); there is no
fallback: a missing or unloadable library raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB

SSD_OK, SSD_ERR_INVALID_ARGUMENT, SSD_ERR_UNSUPPORTED = 0, 1, 2
SSD_ERR_NO_DEVICE, SSD_ERR_OUT_OF_MEMORY, SSD_ERR_HIP, SSD_ERR_WORKSPACE_LIMIT = 3, 4, 5, 6

VARIANTS = {"auto": 0, "unfused": 1, "fused": 2, "quadratic": 3}
PRECISIONS = {"auto": 0, "fp16": 1, "fp32": 3}
DTYPES = {torch.float32: 0, torch.bfloat16: 1}

# Symbols include/ssd.h declares.
EXPORTS = ("ssd_forward", "ssd_forward_ex", "ssd_forward_noalloc", "ssd_chunk_cumsum",
           "ssd_bmm_chunk",
           "ssd_chunk_state", "ssd_state_passing", "ssd_chunk_scan", "ssd_workspace_sizes",
           "ssd_step", "ssd_backward", "ssd_status_string", "ssd_version")


class SSDProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SSDOptions(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("precision", ctypes.c_int32),
                ("run_chunks", ctypes.c_int32), ("n_events", ctypes.c_int32),
                ("events", ctypes.POINTER(ctypes.c_void_p)),
                ("n_kernels", ctypes.POINTER(ctypes.c_int32)),
                ("dt_bias", ctypes.c_void_p), ("dt_softplus", ctypes.c_int32),
                ("dt_min", ctypes.c_float), ("dt_max", ctypes.c_float),
                ("kernel_mask", ctypes.POINTER(ctypes.c_int32))]


# ssd_kernel bits (include/ssd.h) and the names the timer reports; a call launches its kernels in
# increasing bit order
KERNEL_BITS = ((1, "quadratic"), (2, "chunk_cumsum"), (4, "bmm_chunk"), (8, "chunk_state"),
               (16, "state_passing"), (32, "chunk_scan"), (64, "run_states"),
               (128, "chain"), (256, "fused_scan"))


def kernel_names(mask: int) -> tuple:
    """Names of the kernels a forward launched, in launch order, from its kernel mask."""
    return tuple(name for bit, name in KERNEL_BITS if mask & bit)


class SSDError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def load():
    """Load libssd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        raise RuntimeError(f"libssd is not built ({LIB} missing): run "
                           "`python -m mamba_ssd_chunked_cumsum_amd.build`")
    lib = ctypes.CDLL(LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    P = ctypes.POINTER(SSDProblem)
    O = ctypes.POINTER(SSDOptions)
    sig = {
        "ssd_forward": [P, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp],
        "ssd_forward_ex": [P, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, O],
        "ssd_forward_noalloc": [P, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, O],
        "ssd_chunk_cumsum": [P, vp, vp, i64, vp, vp, vp],
        "ssd_bmm_chunk": [P, vp, vp, i64, vp, vp],
        "ssd_chunk_state": [P, vp, vp, vp, vp, i64, vp, vp, O],
        "ssd_state_passing": [P, vp, vp, i64, vp, vp, vp, vp],
        "ssd_chunk_scan": [P, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, O],
        "ssd_workspace_sizes": [P, i64, ctypes.POINTER(ctypes.c_int64)],
        "ssd_step": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "ssd_backward": [P, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                         vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.ssd_status_string.argtypes = [ctypes.c_int]
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().ssd_status_string(int(status)).decode()


def version() -> int:
    return int(load().ssd_version())


def _check(status: int, where: str):
    if status != SSD_OK:
        raise SSDError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def problem(batch, seqlen, nheads, headdim, dstate, ngroups, io_dtype) -> SSDProblem:
    return SSDProblem(batch, seqlen, nheads, headdim, dstate, ngroups, io_dtype, 0)


def _problem_from(x, B) -> SSDProblem:
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [batch, seqlen, nheads, headdim], B/C [batch, seqlen, "
                         "ngroups, dstate]")
    if x.dtype not in DTYPES:
        raise ValueError(f"unsupported io dtype {x.dtype}")
    Bt, L, H, P = x.shape
    return problem(Bt, L, H, P, B.shape[3], B.shape[2], DTYPES[x.dtype])


def _check_shapes(named) -> None:
    """named: (name, tensor or None, expected shape). The C ABI sees only pointers, so a tensor of
    the wrong shape would be read or written out of bounds: every shape is checked here, before
    anything is launched."""
    for name, t, shp in named:
        if t is not None and tuple(t.shape) != tuple(shp):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shp)}")


def _sequence_shapes(x, B, C, dt, A, D, initial_state):
    """The forward's and backward's shared inputs against x [Bt, L, H, P] and B [Bt, L, G, N]."""
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [batch, seqlen, nheads, headdim], B/C [batch, seqlen, "
                         "ngroups, dstate]")
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _check_shapes((("B", B, (Bt, L, G, N)), ("C", C, (Bt, L, G, N)), ("dt", dt, (Bt, L, H)),
                   ("A", A, (H,)), ("D", D, (H,)), ("initial_state", initial_state,
                                                    (Bt, H, P, N))))
    return Bt, L, H, P, G, N


def _require(t, name, dtype=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _options(variant, precision, run_chunks=0, dt_bias=None, dt_softplus=False, dt_limit=None):
    lo, hi = (0.0, 0.0) if dt_limit is None else (float(dt_limit[0]), float(dt_limit[1]))
    return SSDOptions(VARIANTS[variant], PRECISIONS[precision], int(run_chunks), 0, None, None,
                      _ptr(dt_bias), 1 if dt_softplus else 0, lo, hi, None)


class KernelTimer:
    """Six torch.cuda.Event objects handed to the library, which records them on the call's
    stream around each kernel it launches. After synchronising, `times_ms()` gives each kernel's
    elapsed time."""

    def __init__(self):
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        for e in self.events:       # torch creates the HIP event lazily, at its first record
            e.record()
        handles = [e.cuda_event for e in self.events]
        if not all(handles):
            raise RuntimeError("could not create timing events")
        self._arr = (ctypes.c_void_p * 6)(*[ctypes.c_void_p(h) for h in handles])
        self.n_kernels = ctypes.c_int32(0)
        self.kernel_mask = ctypes.c_int32(0)

    def attach(self, opts: SSDOptions):
        opts.n_events = 6
        opts.events = ctypes.cast(self._arr, ctypes.POINTER(ctypes.c_void_p))
        opts.n_kernels = ctypes.pointer(self.n_kernels)
        opts.kernel_mask = ctypes.pointer(self.kernel_mask)

    def kernels(self) -> tuple:
        """Names of the kernels the last call launched, in launch order."""
        return kernel_names(self.kernel_mask.value)

    def times_ms(self) -> dict:
        names = self.kernels()
        return {names[k]: self.events[k].elapsed_time(self.events[k + 1])
                for k in range(len(names))}


FP16_MAX = 65504.0


def check_domain(x, dt, A, B, C, *, fp16_operands=True, dt_processed=False):
    """Raise ValueError unless the inputs lie in the domain the kernels assume: A <= 0 and dt >= 0
    (every decay at most 1; dt is not checked when the kernels pre-process it), no NaN or
    infinity, and, with bf16 io at a precision with fp16 matrix-core operands, |x|, |B|, |C|
    below fp16's largest finite value 65504. One reduction per tensor and a host
    synchronisation: a check for callers that want it, not done by forward() unless asked."""
    def bad(name, cond):
        if bool(cond):
            raise ValueError(f"{name} is outside the kernels' domain")
    bad("A (positive or not finite)", ~torch.all(torch.isfinite(A) & (A <= 0)))
    if not dt_processed:
        bad("dt (negative or not finite)", ~torch.all(torch.isfinite(dt) & (dt >= 0)))
    for name, t in (("x", x), ("B", B), ("C", C)):
        bad(f"{name} (not finite)", ~torch.all(torch.isfinite(t)))
        if fp16_operands and t.dtype == torch.bfloat16:
            bad(f"{name} (beyond fp16's range, 65504)", torch.amax(torch.abs(t)) >= FP16_MAX)


def forward(x, dt, A, B, C, D, chunk_size, initial_state=None, *, variant="auto",
            precision="auto", run_chunks=0, want_final=True, out=None, final_out=None,
            timer: KernelTimer | None = None, dt_bias=None, dt_softplus=False, dt_limit=None,
            noalloc=False, check=False):
    """SSD chunked forward. Returns (y, final_state) (final_state None if not wanted).

    dt_bias [H], dt_softplus and dt_limit=(lo, hi) pre-process dt inside the kernels:
    dt + dt_bias, softplus, clamp to [lo, hi] (hi > 0), in that order. noalloc: call
    ssd_forward_noalloc (workspace from the library's static scratch; give out and final_out to
    keep torch from allocating too). check: run check_domain() on the inputs first.

    Outside the domain (no check): a NaN or infinity in a head's inputs reaches that head's
    outputs from the sub-chunk (fused: 32 tokens) or chunk (unfused) that holds it onwards and its
    final state (in B or C: every head of the group), leaving the other heads and the earlier
    tokens as they are; a bf16 x, B or C of magnitude 65504 or more is infinite in the fused
    path's fp16 operands: the affected heads' outputs from its sub-chunk onwards are undefined
    (so are the unfused kernels' at the default precision; the fp32 precision option has no such
    limit); A > 0 or dt < 0 (decays above 1) give results the
    kernels do not define."""
    Bt, L, H, P, G, N = _sequence_shapes(x, B, C, dt, A, D, initial_state)
    _check_shapes((("dt_bias", dt_bias, (H,)), ("out", out, x.shape),
                   ("final_out", final_out if want_final else None, (Bt, H, P, N))))
    if check:
        check_domain(x, dt, A, B, C, fp16_operands=precision != "fp32",
                     dt_processed=dt_bias is not None or dt_softplus or dt_limit is not None)
    dev = x.device
    _require(x, "x", device=dev)
    for n, t in (("B", B), ("C", C)):
        _require(t, n, x.dtype, dev)
    for n, t in (("dt", dt), ("A", A), ("D", D), ("initial_state", initial_state),
                 ("dt_bias", dt_bias)):
        _require(t, n, torch.float32, dev)
    prob = _problem_from(x, B)
    y = out if out is not None else torch.empty_like(x)
    _require(y, "out", x.dtype, dev)
    fin = None
    if want_final:
        fin = final_out if final_out is not None else torch.empty(
            (x.shape[0], x.shape[2], x.shape[3], B.shape[3]), dtype=torch.float32, device=dev)
        _require(fin, "final_out", torch.float32, dev)
    opts = _options(variant, precision, run_chunks, dt_bias, dt_softplus, dt_limit)
    if timer is not None:
        timer.attach(opts)
    entry = "ssd_forward_noalloc" if noalloc else "ssd_forward_ex"
    st = getattr(load(), entry)(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                _ptr(D), int(chunk_size), _ptr(initial_state), _ptr(y),
                                _ptr(fin), _stream(x), ctypes.byref(opts))
    _check(st, entry)
    return y, fin


def step(state, x, dt, A, B, C, D, *, out_state=None, out=None):
    """Single-token recurrent step (decode). state [Bt, H, P, N] f32; x [Bt, H, P]; dt [Bt, H];
    B, C [Bt, G, N] (x's dtype); A, D [H]. Returns (y [Bt, H, P], new_state); out_state may be
    `state` itself (updated in place)."""
    dev = x.device
    _require(x, "x", device=dev)
    for n, t in (("B", B), ("C", C)):
        _require(t, n, x.dtype, dev)
    for n, t in (("state", state), ("dt", dt), ("A", A), ("D", D)):
        _require(t, n, torch.float32, dev)
    if x.dim() != 3 or B.dim() != 3 or x.dtype not in DTYPES:
        raise ValueError("x must be [batch, nheads, headdim] and B/C [batch, ngroups, dstate], "
                         "float32 or bfloat16")
    Bt, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    for n, t, shp in (("B", B, (Bt, G, N)), ("C", C, (Bt, G, N)), ("dt", dt, (Bt, H)),
                      ("A", A, (H,)), ("D", D, (H,)), ("state", state, (Bt, H, P, N))):
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {shp}")
    prob = problem(Bt, 1, H, P, N, G, DTYPES[x.dtype])
    y = out if out is not None else torch.empty_like(x)
    _require(y, "out", x.dtype, dev)
    so = out_state if out_state is not None else torch.empty_like(state)
    _require(so, "out_state", torch.float32, dev)
    if tuple(y.shape) != (Bt, H, P) or tuple(so.shape) != (Bt, H, P, N):
        raise ValueError("out / out_state have the wrong shape")
    st = load().ssd_step(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                         _ptr(D), _ptr(state), _ptr(so), _ptr(y), _stream(x))
    _check(st, "ssd_step")
    return y, so


def backward(x, dt, A, B, C, D, dy, chunk_size, initial_state=None, dfinal=None, *,
             want_initial_grad=True):
    """Gradients of the forward for output gradient dy (x's dtype and shape) and final-state
    gradient dfinal ([Bt, H, P, N] f32, or None for zero). Returns a dict of float32 tensors:
    dx, ddt, dA, dB, dC, dD and dinitial_state (None unless want_initial_grad)."""
    Bt, L, H, P, G, N = _sequence_shapes(x, B, C, dt, A, D, initial_state)
    _check_shapes((("dy", dy, x.shape), ("dfinal", dfinal, (Bt, H, P, N))))
    dev = x.device
    _require(x, "x", device=dev)
    for n, t in (("B", B), ("C", C), ("dy", dy)):
        _require(t, n, x.dtype, dev)
    for n, t in (("dt", dt), ("A", A), ("D", D), ("initial_state", initial_state),
                 ("dfinal", dfinal)):
        _require(t, n, torch.float32, dev)
    prob = _problem_from(x, B)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dx=torch.empty((Bt, L, H, P), **f32), ddt=torch.empty((Bt, L, H), **f32),
               dA=torch.empty((H,), **f32), dB=torch.empty((Bt, L, G, N), **f32),
               dC=torch.empty((Bt, L, G, N), **f32), dD=torch.empty((H,), **f32),
               dinitial_state=torch.empty((Bt, H, P, N), **f32) if want_initial_grad else None)
    st = load().ssd_backward(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                             _ptr(D), int(chunk_size), _ptr(initial_state), _ptr(dy),
                             _ptr(dfinal), _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]),
                             _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
                             _ptr(out["dinitial_state"]), _stream(x))
    _check(st, "ssd_backward")
    return out


# ---- stages of the unfused path ------------------------------------------------------------------

def workspace_sizes(prob: SSDProblem, chunk_size: int):
    out = (ctypes.c_int64 * 5)()
    _check(load().ssd_workspace_sizes(ctypes.byref(prob), int(chunk_size), out),
           "ssd_workspace_sizes")
    return list(out)


def _nc(L, Q):
    return -(-L // Q)


def chunk_cumsum(dt, A, chunk_size, *, headdim=16, dstate=16, ngroups=1):
    Bt, L, H = dt.shape
    _require(dt, "dt", torch.float32)
    _require(A, "A", torch.float32, dt.device)
    prob = problem(Bt, L, H, headdim, dstate, ngroups, 0)
    nc = _nc(L, chunk_size)
    Acs = torch.empty((Bt, H, nc, chunk_size), dtype=torch.float32, device=dt.device)
    dtc = torch.empty_like(Acs)
    _check(load().ssd_chunk_cumsum(ctypes.byref(prob), _ptr(dt), _ptr(A), int(chunk_size),
                                   _ptr(Acs), _ptr(dtc), _stream(dt)), "ssd_chunk_cumsum")
    return Acs, dtc


def bmm_chunk(B, C, chunk_size, *, nheads=None, headdim=16):
    Bt, L, G, N = B.shape
    _require(B, "B")
    _require(C, "C", B.dtype, B.device)
    prob = problem(Bt, L, nheads or G, headdim, N, G, DTYPES[B.dtype])
    nc = _nc(L, chunk_size)
    CB = torch.zeros((Bt, nc, G, chunk_size, chunk_size), dtype=torch.float32, device=B.device)
    _check(load().ssd_bmm_chunk(ctypes.byref(prob), _ptr(B), _ptr(C), int(chunk_size), _ptr(CB),
                                _stream(B)), "ssd_bmm_chunk")
    return CB


def chunk_state(x, B, Acs, dtc, chunk_size, *, precision="auto"):
    _require(x, "x")
    _require(B, "B", x.dtype, x.device)
    prob = _problem_from(x, B)
    Bt, L, H, P = x.shape
    N = B.shape[3]
    st = torch.empty((Bt, _nc(L, chunk_size), H, P, N), dtype=torch.float32, device=x.device)
    opts = _options("unfused", precision)
    _check(load().ssd_chunk_state(ctypes.byref(prob), _ptr(x), _ptr(B), _ptr(Acs), _ptr(dtc),
                                  int(chunk_size), _ptr(st), _stream(x), ctypes.byref(opts)),
           "ssd_chunk_state")
    return st


def state_passing(states, Acs, chunk_size, initial_state=None, *, seqlen, ngroups=1,
                  want_final=True):
    Bt, nc, H, P, N = states.shape
    prob = problem(Bt, seqlen, H, P, N, ngroups, 0)
    h_in = torch.empty_like(states)
    fin = torch.empty((Bt, H, P, N), dtype=torch.float32, device=states.device) \
        if want_final else None
    _check(load().ssd_state_passing(ctypes.byref(prob), _ptr(states), _ptr(Acs), int(chunk_size),
                                    _ptr(initial_state), _ptr(h_in), _ptr(fin),
                                    _stream(states)), "ssd_state_passing")
    return h_in, fin


def chunk_scan(x, C, CB, Acs, dtc, h_in, D, chunk_size, *, precision="auto"):
    _require(x, "x")
    _require(C, "C", x.dtype, x.device)
    prob = _problem_from(x, C)
    y = torch.empty_like(x)
    opts = _options("unfused", precision)
    _check(load().ssd_chunk_scan(ctypes.byref(prob), _ptr(x), _ptr(C), _ptr(CB), _ptr(Acs),
                                 _ptr(dtc), _ptr(h_in), _ptr(D), int(chunk_size), _ptr(y),
                                 _stream(x), ctypes.byref(opts)), "ssd_chunk_scan")
    return y
