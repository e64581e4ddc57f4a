"""GPU parity of the W4A4 MXFP4 variant against the oracle: the activation
quantizer bit for bit (codes, scales, padding, edge cases), the block-scaled
MFMA GEMM within the layer's tolerance at sizes spanning several tiles with
ragged edges and K-split tail tiles, the fused gate_up, sampled outputs at the
prefill gate_up shape, and determinism."""

import numpy as np
import pytest
import torch

import fp4_weight_only_e2m1_amd as fp4
import oracle
import synth
from gpu_util import DEV, assert_close, prepared, sample_rows, u8, x_dev, y_host, y_host_bits

pytestmark = pytest.mark.gpu

MX = fp4.FMT_MXFP4


def _unpack_act(codes, scales, m, k):
    """GPU quantized-activation buffers -> (codes [m, k], scale bytes [m, k/32]) in the oracle's form,
    plus the padding blocks (k .. K) of rows < m."""
    r, kk = -(-m // 256) * 256, -(-k // 128) * 128
    cb = codes.cpu().numpy()[: r * kk // 2].reshape(r, kk // 2)[:m]
    c = np.empty((m, kk), np.uint8)
    c[:, 0::2] = cb & 0x0F
    c[:, 1::2] = cb >> 4
    sb = scales.cpu().numpy()[: r * kk // 32].reshape(r // 16, kk // 32, 16)
    s = sb.transpose(0, 2, 1).reshape(r, kk // 32)[:m]
    return c[:, :k], s[:, : k // 32], c[:, k:], s[:, k // 32:]


def _x_bits(rng, m, k, spread=4.0):
    # bf16 activations with a per-row scale spread over 2^+-spread and a
    # sprinkling of exact ties of the E2M1 grid.
    x = rng.standard_normal((m, k)).astype(np.float32) * np.exp2(rng.uniform(-spread, spread, (m, 1))).astype(np.float32)
    bits = oracle.f32_to_bf16_bits(x)
    return bits


def _quant_check(xbits):
    m, k = xbits.shape
    codes, scales = fp4.fp4_quantize_act_mxfp4(x_dev(xbits))
    got_c, got_s, pad_c, pad_s = _unpack_act(codes, scales, m, k)
    want_c, want_s = oracle.quantize_act_mxfp4(oracle.bf16_bits_to_f32(xbits))
    assert np.array_equal(got_s, want_s), "scales differ at %s" % (np.argwhere(got_s != want_s)[:5].tolist(),)
    assert np.array_equal(got_c, want_c), "codes differ at %s" % (np.argwhere(got_c != want_c)[:5].tolist(),)
    assert not pad_c.any() and not pad_s.any()


@pytest.mark.parametrize("m,k", [(1, 32), (3, 96), (17, 256), (130, 4064), (64, 4096)])
def test_quantizer_bitwise(m, k):
    _quant_check(_x_bits(np.random.default_rng(m * 7 + k), m, k))


def test_quantizer_ties_and_edges():
    # Every E2M1 midpoint, both signs, at many block scales; zero blocks;
    # bf16 subnormals (scale byte 0); the largest bf16; -0.
    rng = np.random.default_rng(11)
    m, k = 48, 256
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 6.5], np.float64)
    x = np.zeros((m, k), np.float64)
    for r in range(m):
        for b in range(k // 32):
            e = int(rng.integers(-40, 40))
            blk = rng.choice(mids, 32) * rng.choice([-1.0, 1.0], 32)
            blk[int(rng.integers(0, 32))] = 4.0  # amax in [4, 8): the block scale is 2^e
            x[r, 32 * b:32 * b + 32] = blk * 2.0 ** e
    x[0, :32] = 0.0
    x[1, :32] = -0.0
    x[2, :32] = rng.integers(1, 128, 32) * 2.0 ** -133  # bf16 subnormals
    x[3, :32] = 2.0 ** -125
    x[4, :32] = 3.3895313892515355e38 * rng.uniform(-1, 1, 32)
    bits = oracle.f32_to_bf16_bits(x.astype(np.float32))
    bits[1, :32] = 0x8000
    bits[4, 0] = 0x7F7F  # largest finite bf16
    _quant_check(bits)


def test_quantizer_nonfinite_blocks():
    rng = np.random.default_rng(12)
    bits = _x_bits(rng, 4, 128)
    bits[0, 5] = 0x7F80   # +Inf
    bits[1, 40] = 0xFF80  # -Inf
    bits[2, 100] = 0x7FC0  # NaN
    _quant_check(bits)


def _w4a4_ref(xbits, packed, scales, k):
    return oracle.w4a4_linear(oracle.bf16_bits_to_f32(xbits), packed, scales, k)


@pytest.mark.parametrize("m,n,k", [
    (1, 512, 256),       # one tile, no split
    (5, 256, 32),        # the smallest k: one 32-code block, 96 zero-padded codes per stage
    (17, 300, 1056),     # ragged rows, columns and k (k % 128 = 32)
    (130, 1000, 4096),   # 1 x 4 tiles, ragged both ways
    (16, 5120, 17408),   # 20 tiles: tail split along K
    (300, 768, 2080),    # 2 x 3 tiles, k % 128 = 32
    (600, 1024, 512),    # 3 x 4 tiles, ragged rows
    (300, 15360, 1024),  # 120 tail tiles run as row halves; the second half of each lower tile is past m
])
def test_w4a4_linear_parity(m, n, k):
    packed, scales, _ = synth.packed_weight(synth.TINY, 80, n, k, MX)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, MX)
    xbits = _x_bits(np.random.default_rng(m + n + k), m, k, spread=2.0)
    info = fp4.fp4_dispatch_info()
    y = fp4.fp4_w4a4_linear(x_dev(xbits), pc, ps, n, info=info)
    assert info.kernel == 4
    assert_close(y_host(y), _w4a4_ref(xbits, packed, scales, k), "w4a4 m=%d n=%d k=%d" % (m, n, k))


def test_w4a4_split_plan_used():
    # The (16, 5120, 17408) case above runs its 20 tiles as K-split tail units.
    info = fp4.fp4_dispatch_info()
    n, k = 5120, 17408
    pc, ps, _ = prepared(synth.TINY, 81, n, k, MX)
    x = x_dev(_x_bits(np.random.default_rng(1), 16, k))
    fp4.fp4_w4a4_linear(x, pc, ps, n, info=info)
    assert info.splits > 1 and info.grid_y == 20 * info.splits


def test_w4a4_exact_activations_match_weight_only():
    # Activations that are exactly MXFP4 quantize to themselves, so the W4A4
    # result is the weight-only product of the same x (oracle: exact sums).
    rng = np.random.default_rng(13)
    m, n, k = 40, 512, 512
    codes = rng.integers(0, 16, (m, k)).astype(np.uint8)
    codes[:, ::32] = 6  # magnitude 4 in every block: scale 2^e exactly
    e = rng.integers(-6, 6, (m, k // 32))
    x = oracle.E2M1_TABLE[codes].astype(np.float64) * np.repeat(2.0 ** e, 32, axis=1)
    xbits = oracle.f32_to_bf16_bits(x.astype(np.float32))
    packed, scales, _ = synth.packed_weight(synth.TINY, 82, n, k, MX)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, MX)
    y = y_host(fp4.fp4_w4a4_linear(x_dev(xbits), pc, ps, n))
    assert_close(y, oracle.linear(oracle.bf16_bits_to_f32(xbits), packed, scales, k, MX), "exact x")


def test_w4a4_gate_up_parity():
    m, n_half, k = 70, 700, 1024
    pg, sg, _ = synth.packed_weight(synth.TINY, 83, n_half, k, MX)
    pu, su, _ = synth.packed_weight(synth.TINY, 84, n_half, k, MX)
    pc, ps = fp4.fp4_prepare_gate_up(u8(pg), u8(sg), u8(pu), u8(su), n_half, k, MX)
    xbits = _x_bits(np.random.default_rng(14), m, k, spread=1.0)
    y = y_host(fp4.fp4_w4a4_gate_up(x_dev(xbits), pc, ps, n_half))
    want = np.concatenate([_w4a4_ref(xbits, pg, sg, k), _w4a4_ref(xbits, pu, su, k)], axis=1)
    assert_close(y, want, "w4a4 gate_up")


def test_w4a4_prefill_gate_up_shape_sampled():
    # The prefill gate_up shape (m = 1024, 2 x 12288 rows, k = 4096), in the
    # launch configuration the benchmark times: sampled output rows and
    # columns against the oracle (quantization is per row, so sampled rows
    # quantize alone).
    m, n_half, k = 1024, 12288, 4096
    pg, sg, _ = synth.packed_weight(synth.GATE_UP, 0, n_half, k, MX)
    pu, su, _ = synth.packed_weight(synth.GATE_UP, 1, n_half, k, MX)
    pc, ps = fp4.fp4_prepare_gate_up(u8(pg), u8(sg), u8(pu), u8(su), n_half, k, MX)
    xbits = synth.activations(synth.GATE_UP, m, k)
    info = fp4.fp4_dispatch_info()
    y = y_host(fp4.fp4_w4a4_gate_up(x_dev(xbits), pc, ps, n_half, info=info))
    # 384 tiles: 256 whole, then the 128 tail tiles as 256 row halves over all of K.
    assert info.kernel == 4 and info.splits == 1 and (info.grid_x, info.grid_y) == (256, 256)
    rows = sample_rows(m, 24, seed=3)
    cols = sample_rows(n_half, 96, seed=4)
    x_s = oracle.bf16_bits_to_f32(xbits[rows])
    want_g = oracle.w4a4_linear(x_s, pg[cols], sg[cols], k)
    want_u = oracle.w4a4_linear(x_s, pu[cols], su[cols], k)
    assert_close(y[np.ix_(rows, cols)], want_g, "gate sampled")
    assert_close(y[np.ix_(rows, cols + n_half)], want_u, "up sampled")


def test_w4a4_deterministic_and_poisoned_workspace():
    m, n, k = 200, 5120, 5120
    pc, ps, _ = prepared(synth.TINY, 85, n, k, MX)
    x = x_dev(_x_bits(np.random.default_rng(15), m, k))
    need = fp4.fp4_w4a4_workspace_bytes(m, n, k)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    a = y_host_bits(fp4.fp4_w4a4_linear(x, pc, ps, n, workspace=ws))
    ws.fill_(0x7F)
    b = y_host_bits(fp4.fp4_w4a4_linear(x, pc, ps, n, workspace=ws))
    assert np.array_equal(a, b)
