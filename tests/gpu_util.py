"""Helpers for the GPU tests: move seeded inputs to the device, run libssd, run the oracle on the
same inputs, and score the result."""

from __future__ import annotations

import sys

import numpy as np
import torch

import mamba_ssd_chunked_cumsum_amd as ssd
from mamba_ssd_chunked_cumsum_amd import synth
from oracle import metrics, native

DEV = "cuda:0"


def note(msg):
    """Print (and flush) what a GPU step is about to run, so a fault can be attributed."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_device(inp: dict, io: str) -> dict:
    out = {}
    for k, v in inp.items():
        if v is None:
            out[k] = None
            continue
        t = torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
        if k in ("x", "B", "C") and io == "bf16":
            t = t.to(torch.bfloat16)          # exact: the values are bf16 already
        out[k] = t
    return out


def run_gpu(dinp: dict, chunk_size: int, variant="auto", precision="auto", want_final=True,
            run_chunks=0):
    y, f = ssd.forward(dinp["x"], dinp["dt"], dinp["A"], dinp["B"], dinp["C"], dinp["D"],
                       chunk_size, dinp["initial_state"], variant=variant, precision=precision,
                       want_final=want_final, run_chunks=run_chunks)
    torch.cuda.synchronize()
    return y, f


def as64(t):
    return None if t is None else t.float().cpu().numpy().astype(np.float64)


def sample_units(Bt: int, H: int, k: int) -> list:
    """k (batch, head) units spread over the whole range, as batch * H + head indices."""
    n = Bt * H
    if k >= n:
        return list(range(n))
    return sorted(set(int(round(i * (n - 1) / (k - 1))) for i in range(k)))


def score(y, f, y_ref, f_ref, io, units=None, H=None):
    """Parity report on all entries, or on the given (batch * H + head) units only."""
    if units is not None:
        bs = [u // H for u in units]
        hs = [u % H for u in units]
        y = np.stack([y[b, :, h] for b, h in zip(bs, hs)])
        y_ref = np.stack([y_ref[b, :, h] for b, h in zip(bs, hs)])
        if f is not None:
            f = np.stack([f[b, h] for b, h in zip(bs, hs)])
            f_ref = np.stack([f_ref[b, h] for b, h in zip(bs, hs)])
    if f is None:
        f, f_ref = np.zeros(1), np.zeros(1)
    return metrics.parity_report(y, y_ref, f, f_ref, io)


def check_shape(shape: synth.SSDShape, seed=None, cfg_index=None, variant="auto",
                precision="auto", max_units=None, run_chunks=0, mutate=None):
    """Run one workload on the GPU and the oracle; return the parity report. `mutate`, if
    given, edits the drawn input arrays in place before both sides see them."""
    inp = synth.make_inputs(shape, seed=seed, cfg_index=cfg_index)
    if mutate is not None:
        mutate(inp)
    units = None
    if max_units is not None and shape.batch * shape.nheads > max_units:
        units = sample_units(shape.batch, shape.nheads, max_units)
    note(f"{shape} variant={variant} precision={precision} run_chunks={run_chunks} "
         f"units={units}")
    dinp = to_device(inp, shape.io)
    y, f = run_gpu(dinp, shape.chunk_size, variant, precision, run_chunks=run_chunks)
    y64, f64 = as64(y), as64(f)
    del dinp, y, f
    y_ref, f_ref = native.forward(**inp, units=units)
    return score(y64, f64, y_ref, f_ref, shape.io, units, shape.nheads)
