"""ssd_step (one recurrent decode step) on the GPU against the oracle's step, element by element.

Bars: the state is an fp32 output computed in fp32 (a few roundings per element): max |g - r| /
max(|r|, RMS(r)) <= 1e-5. y: fp32 io the same bar; bf16 io at most 1e-5 of RMS beyond half a bf16
ulp of the exact value (the one rounding of the output).
"""

import numpy as np
import pytest
import torch

import mamba_ssd_chunked_cumsum_amd as ssd
from oracle import metrics, ssd_recurrence, ssd_step as oracle_step

from gpu_util import DEV, as64, note

pytestmark = pytest.mark.gpu

TOL = 1e-5


def rand_step(rng, Bt, H, P, N, G, io):
    x = rng.standard_normal((Bt, H, P)).astype(np.float32)
    B = rng.standard_normal((Bt, G, N)).astype(np.float32)
    C = rng.standard_normal((Bt, G, N)).astype(np.float32)
    if io == "bf16":  # bf16-exact values, so both sides see the same numbers
        x, B, C = (torch.from_numpy(v).to(torch.bfloat16).float().numpy() for v in (x, B, C))
    dt = rng.uniform(1e-3, 0.5, (Bt, H)).astype(np.float32)
    A = (-rng.uniform(0.5, 8.0, H)).astype(np.float32)
    D = rng.uniform(0.5, 1.5, H).astype(np.float32)
    S = rng.standard_normal((Bt, H, P, N)).astype(np.float32)
    return dict(state=S, x=x, dt=dt, A=A, B=B, C=C, D=D)


def dev(inp, io):
    out = {}
    for k, v in inp.items():
        t = torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
        if k in ("x", "B", "C") and io == "bf16":
            t = t.to(torch.bfloat16)
        out[k] = t
    return out


def check(y, s, y_ref, s_ref, io):
    assert metrics.rel_floored(s, s_ref) <= TOL, metrics.rel_floored(s, s_ref)
    if io == "bf16":
        assert metrics.rms_r1(y, y_ref) <= TOL, metrics.rms_r1(y, y_ref)
    else:
        assert metrics.rel_floored(y, y_ref) <= TOL, metrics.rel_floored(y, y_ref)


SHAPES = [  # (Bt, H, P, N, G): lanes per state row 4, 8 (N=32), 16 (N=48: 12 used), 32, 64
    (1, 1, 16, 16, 1), (2, 4, 16, 32, 2), (1, 3, 32, 48, 1), (2, 8, 64, 128, 1),
    (1, 4, 128, 256, 2), (1, 2, 256, 64, 1), (3, 6, 48, 80, 3), (2, 80, 64, 128, 1),
]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_step_matches_oracle(shape, io):
    rng = np.random.default_rng(hash(shape) % (1 << 31))
    inp = rand_step(rng, *shape, io)
    note(f"ssd_step {shape} {io}")
    d = dev(inp, io)
    y, s = ssd.step(d["state"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"])
    torch.cuda.synchronize()
    y_ref, s_ref = oracle_step(inp["state"], inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                               inp["D"])
    check(as64(y), as64(s), y_ref, s_ref, io)
    assert torch.equal(d["state"].cpu(), torch.from_numpy(inp["state"]))  # input untouched


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_step_in_place_and_repeated(io):
    """Ten steps updating one state in place (each token with its own draw) against ten oracle
    steps; y every step, the state at the end."""
    rng = np.random.default_rng(5)
    Bt, H, P, N, G, L = 2, 4, 64, 128, 2, 10
    toks = [rand_step(rng, Bt, H, P, N, G, io) for _ in range(L)]
    note(f"ssd_step in place x{L} {io}")
    state = torch.from_numpy(toks[0]["state"]).to(DEV)
    S = toks[0]["state"].astype(np.float64)
    for t in range(L):
        d = dev(toks[t], io)
        y, s = ssd.step(state, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], out_state=state)
        assert s.data_ptr() == state.data_ptr()
        torch.cuda.synchronize()
        k = toks[t]
        y_ref, S = oracle_step(S, k["x"], k["dt"], k["A"], k["B"], k["C"], k["D"])
        ok = metrics.rms_r1 if io == "bf16" else metrics.rel_floored
        assert ok(as64(y), y_ref) <= TOL, (t, ok(as64(y), y_ref))
    assert metrics.rel_floored(as64(state), S) <= TOL


def test_step_continues_forward():
    """forward over L tokens, then one step with token L: equals the oracle over L + 1 tokens."""
    from mamba_ssd_chunked_cumsum_amd import synth
    shape = synth.SSDShape("cont", 1, 257, 4, 64, 128, 1, 64, init_state=True)
    inp = synth.make_inputs(shape, seed=9)
    note("ssd_step after forward")
    d = {k: (None if v is None else torch.from_numpy(v).to(DEV)) for k, v in inp.items()}
    for k in ("x", "B", "C"):
        d[k] = d[k].to(torch.bfloat16)
    L = shape.seqlen - 1
    _, fin = ssd.forward(d["x"][:, :L].contiguous(), d["dt"][:, :L].contiguous(), d["A"],
                         d["B"][:, :L].contiguous(), d["C"][:, :L].contiguous(), d["D"], 64,
                         d["initial_state"])
    y, s = ssd.step(fin, d["x"][:, L].contiguous(), d["dt"][:, L].contiguous(), d["A"],
                    d["B"][:, L].contiguous(), d["C"][:, L].contiguous(), d["D"])
    torch.cuda.synchronize()
    y_ref, s_ref = ssd_recurrence(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                                  initial_state=inp["initial_state"])
    # the forward's final state carries the bf16 path's error (within its 2e-2 bar)
    assert metrics.rms_literal(as64(s), s_ref) <= 2e-2
    assert metrics.rms_r1(as64(y), y_ref[:, L]) <= 2e-2
