"""ssd_backward on the GPU against the float64 backward oracle, element by element.

The GPU backward computes in fp32 throughout (its four chunked recurrences run the fp32 matrix
cores; the inputs are exact in fp32, also for bf16 io), so dx, dB, dC, dD and the initial-state
gradient are held to max |g - r| <= TOL * max|r| over the tensor: fp32 rounding (2^-24 per
operation) accumulated over a few hundred terms of mixed sign leaves a few 1e-6; TOL = 1e-4 keeps
a margin.

The decay gradients are held to a bound derived from how the GPU forms them. dlog_t (the
gradient with respect to dt_t A) is <G_t, exp(dt_t A) S_{t-1}>, and the difference of two
tokens' values is a sum of per-token terms q_s = dy_s . ys_s - dt_s x_s . u_s (ys the state part
of y, u = G B, both outputs of fp32 recurrences, dotted over headdim in fp32). The GPU forms
dlog at the first token t0 of every 256-token tile from the product itself (in double, from the
fp32 states the forward and adjoint recurrences hold there) and within the tile as
dlog_t0 - sum_{t0 <= s < t} q_s (in double). Then ddt_t = A dlog_t + x_t . u_t and
dA = sum over batch and time of dt_t dlog_t. If every fp32 quantity entering those sums carries
a relative error of at most EPS,

    |ddt_t error| <= EPS (|A| R_t + X_t) + 2^-24 |ddt_t|,   |dA error| <= EPS sum_t dt_t R_t,

with R_t = sum_{t0 <= s < t} (sum_p |dy_sp ys_sp| + |dt_s x_sp u_sp|) + dlog_abs_t0 (the
absolute values of the products dlog_t0 sums) and X_t = sum_p |x_tp u_tp| (computed here from
the oracle's y, dx = D dy + dt u and dlog_decay_abs). EPS = 2^-24 (Q + N + P) with Q = 64, the
backward's own chunk length, is the rounding bound of a sum of that many fp32 terms (a
recurrence output sums at most a chunk of Q tokens and a state row of N entries, and the dot
over headdim adds P). The tests print each element's error as a multiple of
2^-24 (|A| R_t + X_t) and each head's dA error relative to its own |dA| (large only on heads
whose dA cancels to a small fraction of its terms).
"""

import numpy as np
import pytest
import torch

import mamba_ssd_chunked_cumsum_amd as ssd
from oracle import ssd_recurrence
from oracle.backward import ssd_backward as oracle_backward

from gpu_util import DEV, note

pytestmark = pytest.mark.gpu

TOL = 1e-4
U32 = 2.0 ** -24
BWD_CHUNK = 64  # the chunk length the backward's recurrences run at, whatever the caller's


def _eps(N, P):
    return U32 * (BWD_CHUNK + N + P)

# Bt, L, H, P, N, G, chunk, io, h0, dfinal
CASES = [
    (1, 64, 2, 16, 16, 1, 16, "f32", False, False),
    (2, 100, 4, 32, 16, 2, 32, "f32", True, True),     # ragged last chunk
    (1, 48, 3, 16, 32, 3, 16, "f32", True, False),     # one group per head
    (1, 96, 2, 64, 128, 1, 64, "bf16", True, True),    # the workloads' head shape
    (2, 130, 8, 64, 64, 2, 64, "bf16", False, True),
    (1, 1, 2, 16, 16, 1, 16, "f32", True, True),       # a single token
    (1, 1024, 4, 64, 128, 1, 256, "bf16", True, True),  # longer runs of chunks
    (1, 600, 2, 32, 64, 1, 64, "f32", True, True),      # several 256-token tiles, ragged end
    (2, 520, 4, 64, 128, 2, 64, "bf16", False, True),   # ... with groups, no initial state
    (1, 300, 2, 128, 256, 1, 128, "bf16", True, True),  # dstate 256: the general C B^T kernel
    (1, 130, 2, 32, 256, 2, 64, "f32", False, True),    # ... with fp32 inputs
]


def _case_id(c):
    return f"{c[0]}x{c[1]}x{c[2]}x{c[3]}x{c[4]}_g{c[5]}_q{c[6]}_{c[7]}" + (
        "_h0" if c[8] else "") + ("_df" if c[9] else "")


def _bf16_exact(a):
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).float().numpy()


def _inputs(rng, Bt, L, H, P, N, G, io, h0, df):
    f32 = lambda a: a.astype(np.float32)
    inp = dict(
        x=f32(rng.standard_normal((Bt, L, H, P))),
        dt=f32(rng.uniform(1e-3, 0.3, (Bt, L, H))),
        A=f32(-rng.uniform(0.5, 4.0, H)),
        B=f32(rng.standard_normal((Bt, L, G, N))),
        C=f32(rng.standard_normal((Bt, L, G, N))),
        D=f32(rng.uniform(0.5, 1.5, H)),
        initial_state=f32(rng.standard_normal((Bt, H, P, N))) if h0 else None,
    )
    dy = f32(rng.standard_normal((Bt, L, H, P)))
    dfinal = f32(rng.standard_normal((Bt, H, P, N))) if df else None
    if io == "bf16":
        for k in ("x", "B", "C"):
            inp[k] = _bf16_exact(inp[k])
        dy = _bf16_exact(dy)
    return inp, dy, dfinal


def _dev(a, io, io_tensor):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t.to(torch.bfloat16) if (io_tensor and io == "bf16") else t


TILE = 256  # the GPU's decay-gradient tiles


def _decay_scales(inp, dy, ref):
    """R [Bt, L, H] and X [Bt, L, H] of the decay-gradient bound, from oracle quantities."""
    y, _ = ssd_recurrence(**inp)
    x = inp["x"].astype(np.float64)
    dt = inp["dt"].astype(np.float64)
    dy64 = dy.astype(np.float64)
    D = inp["D"].astype(np.float64)[None, None, :, None]
    ys = y - D * x
    dtu = ref["dx"] - D * dy64                                   # dt_t u_t
    q_abs = np.sum(np.abs(dy64 * ys), axis=3) + np.sum(np.abs(x * dtu), axis=3)
    X = np.sum(np.abs(x * dtu), axis=3) / dt
    R = np.empty_like(q_abs)
    L = q_abs.shape[1]
    for t0 in range(0, L, TILE):  # exclusive prefix sums within the tile, plus its anchor's scale
        seg = q_abs[:, t0:t0 + TILE]
        R[:, t0:t0 + TILE] = (np.cumsum(seg, axis=1) - seg
                              + ref["dlog_decay_abs"][:, t0][:, None, :])
    return R, X


def _check_decay(got_ddt, got_dA, ref, inp, R, X, eps, label):
    """ddt element by element and dA per head against the derived bound; prints the errors as
    multiples of the bound's fp32 scale and each head's dA error relative to its own |dA|."""
    A = np.abs(inp["A"].astype(np.float64))[None, None, :]
    scale = A * R + X
    err = np.abs(got_ddt - ref["ddt"])
    bound = eps * scale + U32 * np.abs(ref["ddt"])
    print(f"{label} ddt: max|g - r| {err.max():.3e}, max err / (2^-24 (|A| R + X)) "
          f"{np.max(err / np.maximum(U32 * scale, 1e-300)):.2f} (bar {eps / U32:.0f}), "
          f"max|r| {np.abs(ref['ddt']).max():.3e}")
    assert np.all(err <= bound), float(np.max(err / np.maximum(bound, 1e-300)))
    dscale = np.sum(inp["dt"].astype(np.float64) * R, axis=(0, 1))
    derr = np.abs(got_dA - ref["dA"])
    for h in range(len(derr)):
        print(f"{label} dA head {h}: {ref['dA'][h]:+.5e}, |g - r| {derr[h]:.2e}, relative "
              f"{derr[h] / max(abs(ref['dA'][h]), 1e-30):.2e}, err / (2^-24 sum dt R) "
              f"{derr[h] / max(U32 * dscale[h], 1e-300):.2f} (bar {eps / U32:.0f})")
    assert np.all(derr <= eps * dscale), (derr, dscale)


@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_backward_matches_oracle(case):
    _check_case(case, np.random.default_rng(100 + case[1] + 7 * case[2] + case[4]))


def _random_case(seed):
    rng = np.random.default_rng(500 + seed)
    G = int(rng.integers(1, 3))
    return (int(rng.integers(1, 3)), int(rng.integers(1, 700)), G * int(rng.integers(1, 4)),
            int(rng.choice([16, 32, 64, 128])), int(rng.choice([16, 32, 64, 128])), G,
            int(rng.choice([16, 32, 64, 128, 256])), str(rng.choice(["f32", "bf16"])),
            bool(rng.random() < 0.5), bool(rng.random() < 0.5))


@pytest.mark.parametrize("seed", range(12))
def test_backward_random_problems(seed):
    """Seeded random shapes (lengths across several 256-token tiles and none, groups, io,
    initial state and final-state gradient present or not) to the same bars."""
    _check_case(_random_case(seed), np.random.default_rng(seed))


def _check_case(case, rng):
    Bt, L, H, P, N, G, Q, io, h0, df = case
    inp, dy, dfinal = _inputs(rng, Bt, L, H, P, N, G, io, h0, df)
    note(f"backward {_case_id(case)}")
    d = {k: _dev(v, io, k in ("x", "B", "C")) for k, v in inp.items()}
    g = ssd.backward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], _dev(dy, io, True), Q,
                     d["initial_state"], _dev(dfinal, io, False))
    torch.cuda.synchronize()
    ref = oracle_backward(**inp, dy=dy, dfinal=dfinal)
    ref.pop("dlog_decay")
    got = {k: g[k].cpu().numpy().astype(np.float64) for k in ref if k != "dlog_decay_abs"}
    for k, gk in got.items():
        assert np.all(np.isfinite(gk)), k
    R, X = _decay_scales(inp, dy, ref)
    _check_decay(got["ddt"], got["dA"], ref, inp, R, X, _eps(N, P), _case_id(case))
    for k, r in ref.items():
        if k in ("ddt", "dA", "dlog_decay_abs"):
            continue
        gk = got[k]
        err = float(np.max(np.abs(gk - r)))
        scale = float(np.max(np.abs(r)))
        print(f"{k}: max|g - r| = {err:.3e}, max|r| = {scale:.3e}, ratio {err / max(scale, 1e-30):.2e}")
        assert err <= TOL * max(scale, 1e-30), f"{k}: {err:.3e} > {TOL} * {scale:.3e}"


def test_backward_of_forward_loss_matches_directional_derivative():
    """Consistency of the GPU backward with the GPU forward: for a random direction v in x,
    <dL/dx, v> equals (L(x + e v) - L(x - e v)) / 2e with L = sum(dy * y), both from libssd
    (fp32 io, so the finite difference is not swamped by output rounding)."""
    rng = np.random.default_rng(5)
    Bt, L, H, P, N, G, Q = 1, 80, 2, 32, 32, 1, 32
    inp, dy, _ = _inputs(rng, Bt, L, H, P, N, G, "f32", True, False)
    d = {k: _dev(v, "f32", False) for k, v in inp.items()}
    dyt = _dev(dy, "f32", False)
    note("backward directional derivative")
    g = ssd.backward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], dyt, Q, d["initial_state"])
    v = torch.from_numpy(rng.standard_normal(inp["x"].shape).astype(np.float32)).to(DEV)
    eps = 1.0  # y is linear in x: the central difference is exact up to rounding

    def loss(xx):
        y, _ = ssd.forward(xx, d["dt"], d["A"], d["B"], d["C"], d["D"], Q, d["initial_state"],
                           want_final=False)
        return float(torch.sum(dyt.double() * y.double()))

    fd = (loss(d["x"] + eps * v) - loss(d["x"] - eps * v)) / (2 * eps)
    an = float(torch.sum(g["dx"].double() * v.double()))
    torch.cuda.synchronize()
    assert abs(fd - an) <= 1e-4 * max(1.0, abs(an)), (fd, an)


def test_backward_full_size_sampled_heads():
    """The 2.7B-shaped layer (B=2, L=8192, H=80, P=64, N=128, bf16) at full size; the oracle is
    run for two heads over both batch entries (dx, ddt, dA, dD and the initial-state gradient of
    a head depend on that head only; dB and dC sum over all 80 heads and are checked above at
    sizes the oracle covers whole)."""
    from mamba_ssd_chunked_cumsum_amd import synth
    shape = synth.config("mamba2_2p7b_layer")
    inp = synth.make_inputs(shape, cfg_index=2)
    rng = np.random.default_rng(77)
    dy = _bf16_exact(rng.standard_normal(inp["x"].shape).astype(np.float32))
    dfinal = rng.standard_normal((shape.batch, shape.nheads, shape.headdim,
                                  shape.dstate)).astype(np.float32)
    note(f"backward full size {shape}")
    d = {k: _dev(v, "bf16", k in ("x", "B", "C")) for k, v in inp.items()}
    g = ssd.backward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], _dev(dy, "bf16", True),
                     shape.chunk_size, d["initial_state"], _dev(dfinal, "bf16", False))
    torch.cuda.synchronize()
    got = {k: (v.cpu().numpy().astype(np.float64) if v is not None else None) for k, v in g.items()}
    del g, d
    for h in (3, 61):
        sub = dict(x=inp["x"][:, :, h:h + 1], dt=inp["dt"][:, :, h:h + 1], A=inp["A"][h:h + 1],
                   B=inp["B"], C=inp["C"], D=inp["D"][h:h + 1], initial_state=None)
        ref = oracle_backward(**sub, dy=dy[:, :, h:h + 1], dfinal=dfinal[:, h:h + 1])
        R, X = _decay_scales(sub, dy[:, :, h:h + 1], ref)
        _check_decay(got["ddt"][:, :, h:h + 1], got["dA"][h:h + 1], ref, sub, R, X,
                     _eps(shape.dstate, shape.headdim),
                     f"full size, head {h}")
        pairs = dict(dx=(got["dx"][:, :, h:h + 1], ref["dx"]), dD=(got["dD"][h:h + 1], ref["dD"]),
                     dinitial_state=(got["dinitial_state"][:, h:h + 1], ref["dinitial_state"]))
        for k, (gk, r) in pairs.items():
            err = float(np.max(np.abs(gk - r)))
            scale = float(np.max(np.abs(r)))
            print(f"head {h} {k}: max|g - r| = {err:.3e}, scale = {scale:.3e}, "
                  f"ratio {err / max(scale, 1e-30):.2e} (bar {TOL})")
            assert err <= TOL * max(scale, 1e-30), f"head {h} {k}: {err:.3e} vs {scale:.3e}"


def test_backward_deterministic():
    """Two calls on the same inputs give bitwise equal gradients (no atomics, fixed reduction
    orders)."""
    rng = np.random.default_rng(9)
    Bt, L, H, P, N, G, Q = 2, 700, 4, 64, 128, 2, 64
    inp, dy, dfinal = _inputs(rng, Bt, L, H, P, N, G, "bf16", True, True)
    d = {k: _dev(v, "bf16", k in ("x", "B", "C")) for k, v in inp.items()}
    note("backward determinism")
    args = (d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], _dev(dy, "bf16", True), Q,
            d["initial_state"], _dev(dfinal, "bf16", False))
    ga = ssd.backward(*args)
    gb = ssd.backward(*args)
    torch.cuda.synchronize()
    for k in ga:
        if ga[k] is not None:
            assert torch.equal(ga[k], gb[k]), k
