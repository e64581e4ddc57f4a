"""GPU parity of the greedy argmax epilogue (fp4_w4a16_linear_argmax) against
the oracle: exact on one-hot activations (the logits are then single weights,
full of exact ties), and on random activations equal to the argmax of the
unfused call's own logits, whose winner is also within the layer's tolerance
of the oracle's maximum.  Covers the VALU GEMV (split and unsplit), the MFMA
decode (64-row tiles split and unsplit, 96- and 128-row tiles), the wave-split MFMA
decode and poisoned workspaces."""

import numpy as np
import pytest
import torch

import fp4_weight_only_e2m1_amd as fp4
import oracle
import synth
from gpu_util import DEV, decode_kernel, tolerance_violations, u8, x_dev, y_host_bits

pytestmark = pytest.mark.gpu

NV, MX = fp4.FMT_NVFP4, fp4.FMT_MXFP4

# (fmt, n, k): small layers (the wave-split kernel at m <= 8), k past 8192
# (GEMV and MFMA decode split along K), MFMA unsplit 64-row tiles, MFMA
# 128-row tiles, MFMA 96-row tiles (16800 rows pad to 16896); ragged n
# throughout.
SHAPES = [(NV, 1000, 1024), (MX, 777, 5120), (NV, 5000, 2048), (NV, 1000, 9216), (MX, 9000, 512),
          (NV, 131000, 256), (MX, 16800, 544)]


def _zero_canon(bits):
    """bf16 bits with -0 written as +0: a sum of signed zeros is +0 (IEEE), so
    a logit whose only nonzero-weight product is -0 comes out +0."""
    bits = np.asarray(bits, dtype=np.uint16)
    return np.where((bits & 0x7FFF) == 0, np.uint16(0), bits)


def _prep(fmt, n, k, tensor):
    packed, scales, g = synth.packed_weight(synth.TINY, tensor, n, k, fmt)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    return packed, scales, g, pc, ps


@pytest.mark.parametrize("fmt,n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 8, 16, 32])
def test_one_hot_argmax_exact(fmt, n, k, m):
    packed, scales, g, pc, ps = _prep(fmt, n, k, 80)
    ks = np.linspace(0, k - 1, m).astype(np.int64)
    x = np.zeros((m, k), np.float32)
    x[np.arange(m), ks] = 1.0
    xbits = oracle.f32_to_bf16_bits(x)
    info = fp4.fp4_dispatch_info()
    idx, val, y = fp4.fp4_w4a16_linear_argmax(x_dev(xbits), pc, ps, n, float(g), fmt, logits=True, info=info)
    assert info.kernel == decode_kernel(fmt, n, k, m)
    # Logits are bf16(w[:, k_i]) exactly (G is applied after the sum; -0 sums to +0).
    w = oracle.dequantize(packed, scales, k, fmt, g)
    logit_bits = _zero_canon(oracle.f32_to_bf16_bits(np.ascontiguousarray(w[:, ks].T)))
    want = oracle.greedy_argmax(oracle.bf16_bits_to_f32(logit_bits))
    got = idx.cpu().numpy()
    assert got.tolist() == want.tolist()
    vb = val.view(torch.int16).cpu().numpy().view(np.uint16)
    assert vb.tolist() == logit_bits[np.arange(m), want].tolist()
    assert np.array_equal(y_host_bits(y), logit_bits)


@pytest.mark.parametrize("fmt,n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 2, 4, 5, 8])
def test_argmax_matches_unfused_logits_and_oracle(fmt, n, k, m):
    packed, scales, g, pc, ps = _prep(fmt, n, k, 81)
    xbits = synth.activations(synth.TINY, m, k)
    xd = x_dev(xbits)
    y_ref_gpu = y_host_bits(fp4.fp4_w4a16_linear(xd, pc, ps, n, float(g), fmt))
    idx, val, y = fp4.fp4_w4a16_linear_argmax(xd, pc, ps, n, float(g), fmt, logits=True)
    got = idx.cpu().numpy()
    # Same bf16 logits as the unfused call, and their greedy token.
    assert np.array_equal(y_host_bits(y), y_ref_gpu)
    assert got.tolist() == oracle.greedy_argmax(oracle.bf16_bits_to_f32(y_ref_gpu)).tolist()
    vb = val.view(torch.int16).cpu().numpy().view(np.uint16)
    assert vb.tolist() == y_ref_gpu[np.arange(m), got].tolist()
    # Without the logits buffer the token is the same.
    idx2, _, y2 = fp4.fp4_w4a16_linear_argmax(xd, pc, ps, n, float(g), fmt)
    assert y2 is None and idx2.cpu().numpy().tolist() == got.tolist()
    # The winner's exact value is within the layer's tolerance of the exact maximum.
    y_ref = oracle.linear(oracle.bf16_bits_to_f32(xbits), packed, scales, k, fmt, g)
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    for i in range(m):
        top = y_ref[i].max()
        assert y_ref[i, got[i]] >= top - (2.0 ** -7 * abs(top) + 1e-3 * rms), i


@pytest.mark.parametrize("fmt,n,k,m", [(NV, 5000, 2048, 4), (MX, 777, 5120, 1), (NV, 131000, 256, 8),
                                       (NV, 1000, 9216, 1), (NV, 1000, 9216, 5)])
def test_argmax_workspace_poison_and_repeat(fmt, n, k, m):
    _, _, g, pc, ps = _prep(fmt, n, k, 82)
    xd = x_dev(synth.activations(synth.TINY, m, k))
    need = fp4.fp4_argmax_workspace_bytes(m, n, k, fmt)
    outs = []
    for fill in (0x00, 0xFF, 0x5A, 0x5A):
        ws = torch.full((need,), fill, dtype=torch.uint8, device=DEV)
        idx, val, _ = fp4.fp4_w4a16_linear_argmax(xd, pc, ps, n, float(g), fmt, workspace=ws)
        outs.append((idx.cpu().numpy().tolist(), val.view(torch.int16).cpu().numpy().tolist()))
    assert all(o == outs[0] for o in outs[1:])


def test_argmax_exact_ties_take_lowest_index():
    # Rows 7, 300 and 900 become copies of the row with the largest weight at
    # code k0; with x = e_k0 their logits tie exactly at the maximum and the
    # lowest index holding it must win, at every m and on every kernel.
    n, k, fmt = 1024, 512, NV
    packed, scales, g = synth.packed_weight(synth.TINY, 83, n, k, fmt)
    packed, scales = packed.copy(), scales.copy()
    k0 = 37
    src = int(np.argmax(oracle.dequantize(packed, scales, k, fmt, g)[:, k0]))
    for r in (7, 300, 900):
        packed[r], scales[r] = packed[src], scales[src]
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    col = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(oracle.dequantize(packed, scales, k, fmt, g)[:, k0]))
    assert np.count_nonzero(col == col.max()) >= 3
    want = int(oracle.greedy_argmax(col)[0])
    assert want == min(7, src)
    for m in (1, 2, 3, 8):
        x = np.zeros((m, k), np.float32)
        x[:, k0] = 1.0
        idx, _, _ = fp4.fp4_w4a16_linear_argmax(x_dev(oracle.f32_to_bf16_bits(x)), pc, ps, n, float(g), fmt)
        assert idx.cpu().numpy().tolist() == [want] * m, m
