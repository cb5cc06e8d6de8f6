"""The binding checks every tensor's shape before anything reaches the C ABI (which sees only
pointers): a mismatched tensor raises ValueError naming it, before device, dtype or library
checks, so nothing is launched. Runs without a GPU (CPU tensors: a well-shaped call fails only
at the device check)."""

import pytest
import torch

from mamba_ssd_chunked_cumsum_amd import libssd

Bt, L, H, P, G, N = 2, 40, 6, 16, 3, 8


def _inputs():
    bf = dict(dtype=torch.bfloat16)
    return dict(x=torch.zeros(Bt, L, H, P, **bf), dt=torch.zeros(Bt, L, H), A=torch.zeros(H),
                B=torch.zeros(Bt, L, G, N, **bf), C=torch.zeros(Bt, L, G, N, **bf),
                D=torch.zeros(H))


def _forward(**kw):
    a = _inputs()
    a.update(kw)
    return libssd.forward(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], 16,
                          kw.get("initial_state"), out=kw.get("out"),
                          final_out=kw.get("final_out"), dt_bias=kw.get("dt_bias"))


def _backward(**kw):
    a = _inputs()
    a.update(kw)
    dy = kw.get("dy", torch.zeros_like(a["x"]))
    return libssd.backward(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], dy, 16,
                           kw.get("initial_state"), kw.get("dfinal"))


BF = dict(dtype=torch.bfloat16)
WRONG = [
    ("B", torch.zeros(Bt + 1, L, G, N, **BF)),          # B's last two dims set G and N
    ("B", torch.zeros(Bt, L - 1, G, N, **BF)),
    ("C", torch.zeros(Bt, L, G - 1, N, **BF)),
    ("C", torch.zeros(Bt, L, N, G, **BF)),            # transposed
    ("dt", torch.zeros(Bt, L, H + 1)),
    ("dt", torch.zeros(Bt, H, L)),                     # transposed
    ("A", torch.zeros(H - 1)),
    ("D", torch.zeros(H, 1)),
    ("initial_state", torch.zeros(Bt, H, N, P)),       # transposed
]


@pytest.mark.parametrize("name,t", WRONG, ids=[f"{n}{tuple(t.shape)}" for n, t in WRONG])
def test_forward_rejects_wrong_shapes(name, t):
    with pytest.raises(ValueError, match=f"^{name} has shape"):
        _forward(**{name: t})


@pytest.mark.parametrize("name,t", WRONG, ids=[f"{n}{tuple(t.shape)}" for n, t in WRONG])
def test_backward_rejects_wrong_shapes(name, t):
    with pytest.raises(ValueError, match=f"^{name} has shape"):
        _backward(**{name: t})


def test_forward_output_and_option_shapes():
    with pytest.raises(ValueError, match="^out has shape"):
        _forward(out=torch.zeros(Bt, L, H, P - 1, **BF))
    with pytest.raises(ValueError, match="^final_out has shape"):
        _forward(final_out=torch.zeros(Bt, H, P, N + 1))
    with pytest.raises(ValueError, match="^dt_bias has shape"):
        _forward(dt_bias=torch.zeros(H + 1))


def test_backward_gradient_shapes():
    with pytest.raises(ValueError, match="^dy has shape"):
        _backward(dy=torch.zeros(Bt, L, H, P + 1, **BF))
    with pytest.raises(ValueError, match="^dfinal has shape"):
        _backward(dfinal=torch.zeros(Bt, H, P))


def test_well_shaped_cpu_call_fails_only_at_the_device_check():
    with pytest.raises(ValueError, match="must be a device tensor"):
        _forward()
    with pytest.raises(ValueError, match="must be a device tensor"):
        _backward()
