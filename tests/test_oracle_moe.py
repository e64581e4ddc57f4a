"""Pins for the oracle's grouped MoE decode (CPU only): the single-expert case
reduces to the dense layer, each pair's row matches the fp64 brute-force dot
products, and the routing is checked through constructed experts (a negated
weight, a reordered expert list) whose outputs are known without it."""

import numpy as np

import oracle
import synth

NV, MX = oracle.FMT_NVFP4, oracle.FMT_MXFP4


def _experts(count, n, k, fmt, seed):
    return [synth.packed_weight(synth.TINY, 90 + seed + e, n, k, fmt) for e in range(count)]


def test_single_expert_is_the_dense_layer():
    n, k, t = 48, 64, 5
    (packed, scales, g), = _experts(1, n, k, NV, 0)
    x = oracle.bf16_bits_to_f32(synth.activations(synth.TINY, t, k))
    y = oracle.moe_decode(x, [(packed, scales, g)], k, NV, [0, t], list(range(t)))
    assert np.array_equal(y, oracle.linear(x, packed, scales, k, NV, g))


def test_pairs_match_bruteforce():
    n, k, fmt = 16, 64, MX
    ex = _experts(3, n, k, fmt, 1)
    x = oracle.bf16_bits_to_f32(synth.activations(synth.TINY, 4, k))
    offsets = [0, 2, 2, 5]                 # expert 1 has no pairs
    tokens = [3, 0, 1, 3, 2]
    y = oracle.moe_decode(x, ex, k, fmt, offsets, tokens)
    owner = [0, 0, 2, 2, 2]
    for p, (e, t) in enumerate(zip(owner, tokens)):
        packed, scales, g = ex[e]
        ref = oracle.linear_f64_bruteforce(x[t:t + 1], packed, scales, k, fmt, g)[0]
        assert np.allclose(y[p], ref, rtol=1e-12, atol=1e-12), p


def test_negated_expert_and_reordered_experts():
    n, k, fmt = 32, 64, NV
    packed, scales, g = _experts(1, n, k, fmt, 2)[0]
    neg = packed ^ np.uint8(0x88)          # flip both nibbles' sign bits: w -> -w
    x = oracle.bf16_bits_to_f32(synth.activations(synth.TINY, 3, k))
    y = oracle.moe_decode(x, [(packed, scales, g), (neg, scales, g)], k, fmt, [0, 3, 6], [0, 1, 2, 0, 1, 2])
    assert np.array_equal(y[3:], -y[:3])
    # The same pairs with the experts listed the other way round.
    y2 = oracle.moe_decode(x, [(neg, scales, g), (packed, scales, g)], k, fmt, [0, 3, 6], [0, 1, 2, 0, 1, 2])
    assert np.array_equal(y2[:3], y[3:]) and np.array_equal(y2[3:], y[:3])
