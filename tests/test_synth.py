"""The seeded input generator: reproducible, right shapes and dtypes, bf16-exact where needed."""

import numpy as np
import pytest
import torch

from mamba_ssd_chunked_cumsum_amd import synth


def test_configs_shapes():
    c = synth.CONFIGS
    assert [s.io for s in c] == ["f32", "bf16", "bf16", "bf16", "bf16"]
    assert (c[2].batch, c[2].seqlen, c[2].nheads, c[2].headdim, c[2].dstate, c[2].chunk_size) == \
        (2, 8192, 80, 64, 128, 256)
    assert c[3].init_state and c[3].nchunks == 1024
    assert c[4].ngroups == 8 and c[4].random_d


@pytest.mark.parametrize("idx", [0, 1])
def test_reproducible_and_shapes(idx):
    s = synth.CONFIGS[idx]
    a = synth.make_inputs(s)
    b = synth.make_inputs(s)
    for k in a:
        if a[k] is None:
            assert b[k] is None
            continue
        assert a[k].dtype == np.float32
        assert np.array_equal(a[k], b[k])
    assert a["x"].shape == (s.batch, s.seqlen, s.nheads, s.headdim)
    assert a["B"].shape == (s.batch, s.seqlen, s.ngroups, s.dstate)
    assert a["dt"].shape == (s.batch, s.seqlen, s.nheads)
    assert np.all(a["dt"] > 0) and np.all(a["A"] <= -1) and np.all(a["A"] >= -16)
    c = synth.make_inputs(s, seed=5)
    assert not np.array_equal(c["x"], a["x"])


def test_bf16_rounding_is_rne_and_exact():
    s = synth.config("mamba2_130m_layer").replace(seqlen=64)
    inp = synth.make_inputs(s)
    for k in ("x", "B", "C"):
        bits = synth.bf16_bits(inp[k])                       # raises if not bf16-exact
        back = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
        assert np.array_equal(back, inp[k])
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    assert np.array_equal(synth.round_to_bf16(r),
                          torch.from_numpy(r).to(torch.bfloat16).float().numpy())


def test_dt_distribution():
    s = synth.config("mamba2_130m_layer").replace(seqlen=512)
    dt = synth.make_inputs(s)["dt"]
    assert 1e-5 < dt.min() and dt.max() < 2.0
    med = np.median(dt, axis=(0, 1))            # per-head median tracks the log-uniform bias
    assert med.min() < 5e-3 and med.max() > 2e-2


def test_initial_state_and_d():
    s3 = synth.config("long_seq_layer").replace(seqlen=64)
    inp = synth.make_inputs(s3, cfg_index=3)
    assert inp["initial_state"].shape == (1, 32, 64, 128)
    s4 = synth.config("wide_grouped_layer").replace(seqlen=32)
    d = synth.make_inputs(s4, cfg_index=4)["D"]
    assert d.shape == (64,) and 0.5 < d.mean() < 1.5 and d.std() > 0.01
    assert np.all(synth.make_inputs(synth.config("tiny_fp32"))["D"] == 1.0)
