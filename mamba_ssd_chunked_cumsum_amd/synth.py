"""Seeded synthetic inputs for the SSD chunked forward.

This module draws the inputs of the Mamba-2 SSD layer (x, dt, A, B, C, D and an optional
initial state) with the value distributions of the Mamba-2-shaped workloads: x, B, C standard
normal; dt = softplus(z + dt_bias) with z ~ N(0, 0.5^2) and dt_bias the inverse softplus of a
log-uniform draw in [1e-3, 1e-1] (one per head); A_h = -U[1, 16]; D = 1 (or N(1, 0.1^2) per head);
an optional initial state ~ N(0, 1).

It holds none of the method's arithmetic (no decay, no cumulative sum, no contraction): the
softplus here produces the *input* dt, which the method then consumes as given. Both the CPU
oracle side and the GPU side read the arrays this module returns, so the two see identical values.

Every array is returned as numpy float32. When the io dtype is bf16, x, B and C are rounded to
bf16 (round-to-nearest-even) and stored back in float32, so the float32 array holds exactly the
bf16 values: widening to float64 (oracle) or narrowing the bit pattern to bf16 (GPU) is exact.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "SSDShape",
    "CONFIGS",
    "config",
    "make_inputs",
    "round_to_bf16",
    "bf16_bits",
]


@dataclasses.dataclass(frozen=True)
class SSDShape:
    """Shape and input recipe of one SSD forward workload."""

    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_size: int
    io: str = "bf16"          # dtype of x, B, C and y: "f32" or "bf16"
    init_state: bool = False  # draw a nonzero initial state ~ N(0, 1)
    random_d: bool = False    # D ~ N(1, 0.1^2) per head instead of D = 1

    @property
    def nchunks(self) -> int:
        return -(-self.seqlen // self.chunk_size)

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def replace(self, **kw) -> "SSDShape":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny fp32 case, then Mamba-2-130M-, 2.7B-shaped layers, a long-sequence
# layer with a nonzero initial state, and a wide-head grouped layer.
CONFIGS = (
    SSDShape("tiny_fp32", 1, 256, 2, 16, 16, 1, 64, io="f32"),
    SSDShape("mamba2_130m_layer", 4, 2048, 24, 64, 128, 1, 64),
    SSDShape("mamba2_2p7b_layer", 2, 8192, 80, 64, 128, 1, 256),
    SSDShape("long_seq_layer", 1, 65536, 32, 64, 128, 1, 64, init_state=True),
    SSDShape("wide_grouped_layer", 2, 16384, 64, 128, 256, 8, 128, random_d=True),
)


def config(idx_or_name) -> SSDShape:
    if isinstance(idx_or_name, int):
        return CONFIGS[idx_or_name]
    for c in CONFIGS:
        if c.name == idx_or_name:
            return c
    raise KeyError(idx_or_name)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); result stored as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # finite inputs only: the largest finite pattern plus the rounding bias stays below 2^32
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are exactly bf16 (asserted), as uint16."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("array holds values that are not exactly representable in bf16")
    return (u >> 16).astype(np.uint16)


def _softplus(v: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, v)


def make_inputs(shape: SSDShape, seed: int | None = None, cfg_index: int | None = None) -> dict:
    """Draw one seeded set of inputs for `shape`.

    The generator is numpy's PCG64 seeded with `seed` (default 1000 + the workload's index in
    CONFIGS, or 1000 for shapes outside it). Draw order: u[H], z[Bt,L,H], A[H], x, B, C, then D
    (random_d) and the initial state (init_state).
    """
    if seed is None:
        if cfg_index is None:
            cfg_index = next((i for i, c in enumerate(CONFIGS) if c == shape), 0)
        seed = 1000 + cfg_index
    rng = np.random.default_rng(seed)
    Bt, L, H, P, N, G = (shape.batch, shape.seqlen, shape.nheads, shape.headdim,
                         shape.dstate, shape.ngroups)
    if H % G:
        raise ValueError("nheads must be a multiple of ngroups")

    u = np.exp(rng.uniform(math.log(1e-3), math.log(1e-1), size=H))
    dt_bias = np.log(np.expm1(u))                      # inverse softplus of u
    z = rng.normal(0.0, 0.5, size=(Bt, L, H))
    dt = _softplus(z + dt_bias[None, None, :]).astype(np.float32)
    A = (-rng.uniform(1.0, 16.0, size=H)).astype(np.float32)

    x = rng.standard_normal(size=(Bt, L, H, P), dtype=np.float32)
    B = rng.standard_normal(size=(Bt, L, G, N), dtype=np.float32)
    C = rng.standard_normal(size=(Bt, L, G, N), dtype=np.float32)
    if shape.io == "bf16":
        x, B, C = round_to_bf16(x), round_to_bf16(B), round_to_bf16(C)
    elif shape.io != "f32":
        raise ValueError(f"unknown io dtype {shape.io!r}")

    if shape.random_d:
        D = rng.normal(1.0, 0.1, size=H).astype(np.float32)
    else:
        D = np.ones(H, dtype=np.float32)
    h0 = None
    if shape.init_state:
        h0 = rng.standard_normal(size=(Bt, H, P, N), dtype=np.float32)
    return {"x": x, "dt": dt, "A": A, "B": B, "C": C, "D": D, "initial_state": h0}
