"""Pins for the oracle's SwiGLU gate_up (CPU only): closed forms of silu, and
one-hot weights that make gate and up single activations, so the layer's
output has a closed form silu(x_a) * x_b."""

import math

import numpy as np
import pytest

import oracle

NV, MX = oracle.FMT_NVFP4, oracle.FMT_MXFP4


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    # sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4
    assert math.isclose(float(oracle.silu(math.log(3.0))), 0.75 * math.log(3.0), rel_tol=1e-15)
    assert math.isclose(float(oracle.silu(-math.log(3.0))), -0.25 * math.log(3.0), rel_tol=1e-15)
    v = np.linspace(-30, 30, 601)
    assert np.allclose(oracle.silu(v) - oracle.silu(-v), v, rtol=0, atol=1e-12)   # v (s(v) + s(-v)) = v
    assert oracle.silu(-1e4) == 0.0 and oracle.silu(1e4) == 1e4


def _one_hot_weight(n, k, col, fmt):
    # Row j: code 0x2 (1.0) at column col[j], zeros elsewhere; unit scales.
    codes = np.zeros((n, k), np.uint8)
    codes[np.arange(n), col] = 0x2
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    g = 16 if fmt == NV else 32
    scales = np.full((n, k // g), 0x38 if fmt == NV else 0x7F, np.uint8)
    return packed, scales


@pytest.mark.parametrize("fmt", [NV, MX])
def test_one_hot_swiglu_closed_form(fmt):
    n, k, m = 24, 64, 3
    rng = np.random.default_rng(5)
    a = rng.integers(0, k, size=n)
    b = rng.integers(0, k, size=n)
    pg, sg = _one_hot_weight(n, k, a, fmt)
    pu, su = _one_hot_weight(n, k, b, fmt)
    x = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32)))
    y = oracle.gate_up_swiglu(x, pg, sg, pu, su, k, fmt)
    xa = x[:, a].astype(np.float64)
    want = xa / (1.0 + np.exp(-xa)) * x[:, b].astype(np.float64)
    assert np.allclose(y, want, rtol=1e-15, atol=0)
