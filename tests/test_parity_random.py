"""Seeded random problems on the GPU against the float64 oracle (C recurrence): shapes, chunk
lengths, run lengths, group layouts, io dtypes and variants drawn from one generator, to reach
combinations the hand-picked parity cases do not name (ragged lengths against several run and
chunk lengths at once, groups of one to five heads, odd head counts). Same bars as the other
parity tests."""

import numpy as np
import pytest

from mamba_ssd_chunked_cumsum_amd import synth

from gpu_util import check_shape

pytestmark = pytest.mark.gpu

FUSED = {(p, n) for p in (64, 128) for n in (64, 128, 256)}


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    io = "bf16" if rng.random() < 0.75 else "f32"
    if io == "bf16" and rng.random() < 0.8:
        P, N = [(64, 64), (64, 128), (64, 256), (128, 64), (128, 128), (128, 256)][
            rng.integers(6)]
    else:
        P = int(rng.choice([16, 32, 48, 64, 96, 128]))
        N = int(rng.choice([16, 32, 64, 128, 256]))
    G = int(rng.integers(1, 4))
    hpg = int(rng.integers(1, 6))
    Q = int(rng.choice([16, 32, 64, 128, 256]))
    L = int(rng.integers(1, 1200))
    Bt = int(rng.integers(1, 3))
    shape = synth.SSDShape(f"rand{seed}", Bt, L, G * hpg, P, N, G, Q, io=io,
                           init_state=bool(rng.random() < 0.5),
                           random_d=bool(rng.random() < 0.5))
    fused = io == "bf16" and (P, N) in FUSED
    variant = str(rng.choice(["auto", "fused", "unfused"])) if fused else \
        str(rng.choice(["auto", "unfused"]))
    run_chunks = int(rng.choice([0, 0, 1, 2, 3, 5])) if variant != "unfused" else 0
    return shape, variant, run_chunks


@pytest.mark.parametrize("seed", range(64))
def test_random_problem(seed):
    shape, variant, run_chunks = draw(seed)
    rep = check_shape(shape, seed=seed, variant=variant, run_chunks=run_chunks)
    assert rep["pass"], (shape, variant, run_chunks, rep)
