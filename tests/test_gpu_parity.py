"""GPU parity of the HIP path against the oracle, at sizes the oracle finishes
in seconds: bitwise dequantization, the linear layer within the layer's
tolerance, and the invariants the kernels promise (one-hot layout, fused ==
split, batch invariance, determinism, poisoned workspace)."""

import numpy as np
import pytest
import torch

import fp4_weight_only_e2m1_amd as fp4
import oracle
import synth
from gpu_util import DEV, assert_close, decode_kernel, u8, x_dev, y_host, y_host_bits

pytestmark = pytest.mark.gpu

NV, MX = fp4.FMT_NVFP4, fp4.FMT_MXFP4
GS = {NV: 16, MX: 32}


def _canon_bits(a):
    """float32 bits with every NaN made the same quiet NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32).copy()
    a[np.isnan(a)] = np.float32(np.nan)
    return a.view(np.uint32)


def _quantized(fmt, n, k, tensor=0, workload=synth.TINY):
    packed, scales, g = synth.packed_weight(workload, 50 + tensor, n, k, fmt)
    return packed, scales, g


def _run_linear(packed, scales, g, fmt, n, k, xbits, info=None):
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    y = fp4.fp4_w4a16_linear(x_dev(xbits), pc, ps, n, float(g), fmt, info=info)
    return y


# ---------------------------------------------------------------- dequant


@pytest.mark.parametrize("fmt", [NV, MX])
@pytest.mark.parametrize("g", [1.0, 2.0 ** -7, 0.0123 / 2688])
def test_dequant_exhaustive_codes_and_scales(fmt, g):
    # Row r uses scale byte r for every group; each group holds all 16 codes.
    n, k = 256, 64
    codes = np.tile(np.arange(16, dtype=np.uint8), (n, k // 16))
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], k // GS[fmt], axis=1)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    out = fp4.fp4_dequantize(pc, ps, n, k, np.float32(g), fmt).cpu().numpy()
    want = oracle.dequantize(packed, scales, k, fmt, np.float32(g))
    mism = _canon_bits(out) != _canon_bits(want)
    if mism.any():
        r, c = np.argwhere(mism)[0]
        raise AssertionError("%d mismatches; first: scale byte %#x code %#x got %r want %r" %
                             (int(mism.sum()), r, codes[r, c], out[r, c], want[r, c]))


@pytest.mark.parametrize("fmt,n,k", [(NV, 512, 256), (MX, 512, 256), (NV, 300, 1056), (MX, 77, 2080)])
def test_dequant_synthetic_weights(fmt, n, k):
    packed, scales, g = _quantized(fmt, n, k)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    out = fp4.fp4_dequantize(pc, ps, n, k, float(g), fmt).cpu().numpy()
    assert np.array_equal(_canon_bits(out), _canon_bits(oracle.dequantize(packed, scales, k, fmt, g)))


def test_prepared_layout_bytes():
    # Codes: canonical bytes, zero padded to [n_pad, k_pad/2]; scales: within
    # groups of 16 rows, the rows' bytes of one 32-code segment are adjacent.
    n, k, fmt = 300, 1056, NV
    packed, scales, _ = _quantized(fmt, n, k)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    n_pad, k_pad = 512, 2048
    want_c = np.zeros((n_pad, k_pad // 2), np.uint8)
    want_c[:n, :k // 2] = packed
    kg_pad = k_pad // 16
    s_pad = np.zeros((n_pad, kg_pad), np.uint8)
    s_pad[:n, :k // 16] = scales
    # [n_pad/16][k_pad/32][16][2] for NVFP4 (two 16-code groups per segment)
    want_s = s_pad.reshape(n_pad // 16, 16, kg_pad // 2, 2).transpose(0, 2, 1, 3).reshape(-1)
    assert np.array_equal(pc.cpu().numpy(), want_c.reshape(-1))
    assert np.array_equal(ps.cpu().numpy(), want_s)


# ---------------------------------------------------------------- linear


SHAPES = [
    (NV, 512, 256),     # the tiny NVFP4 workload
    (MX, 512, 256),
    (NV, 640, 2048),    # two slabs
    (MX, 384, 3072),    # three slabs
    (NV, 300, 1056),    # ragged n and a ragged last slab
    (MX, 257, 96),      # k below one slab
    (NV, 256, 5120),    # k split in two (lm_head's k)
    (NV, 128, 17408),   # many splits (down_proj's k)
    (NV, 640, 9216),    # past the wave-split kernel's 32 K stages: the 64-row kernels, K split
    (MX, 16384, 1056),  # 256 64-row tiles: the 64-row kernels, unsplit, ragged last stage
]


@pytest.mark.parametrize("fmt,n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 9, 13, 16, 17, 24, 32])  # 9..16, 17..32: 16- and 32-row x stages
def test_gemv_matches_oracle(fmt, n, k, m):
    packed, scales, g = _quantized(fmt, n, k)
    xbits = synth.activations(synth.TINY, m, k)
    info = fp4.fp4_dispatch_info()
    y = _run_linear(packed, scales, g, fmt, n, k, xbits, info)
    assert info.kernel == decode_kernel(fmt, n, k, m)
    y_ref = oracle.linear(oracle.bf16_bits_to_f32(xbits), packed, scales, k, fmt, g)
    assert_close(y_host(y), y_ref, "gemv fmt=%d n=%d k=%d m=%d" % (fmt, n, k, m))


@pytest.mark.parametrize("fmt,n,k", [(NV, 512, 256), (MX, 640, 2048), (NV, 300, 1056), (MX, 256, 5120)])
@pytest.mark.parametrize("m", [33, 48, 64, 65, 128, 200])  # 64 bounds the 2-block tiles (1-block: SwiGLU, MoE)
def test_mfma_matches_oracle(fmt, n, k, m):
    packed, scales, g = _quantized(fmt, n, k)
    xbits = synth.activations(synth.TINY, m, k)
    info = fp4.fp4_dispatch_info()
    y = _run_linear(packed, scales, g, fmt, n, k, xbits, info)
    assert info.kernel == 1
    y_ref = oracle.linear(oracle.bf16_bits_to_f32(xbits), packed, scales, k, fmt, g)
    assert_close(y_host(y), y_ref, "mfma fmt=%d n=%d k=%d m=%d" % (fmt, n, k, m))


@pytest.mark.parametrize("fmt,n,k,m", [(NV, 25600, 2560, 130), (MX, 30720, 4096, 200)])
def test_two_way_tail_runs_whole(fmt, n, k, m):
    # 200 / 240 tiles of 128 x 256 against 512 workgroup slots: a tail that
    # would split only two ways along K runs as whole tiles, with no
    # workspace and no reduce launch; at m = 130 most of the lower row of
    # tiles is past m.
    assert fp4.fp4_workspace_bytes(m, n, k, fmt) == 0
    packed, scales, g = _quantized(fmt, n, k, tensor=6)
    xbits = synth.activations(synth.TINY, m, k)
    info = fp4.fp4_dispatch_info()
    y = _run_linear(packed, scales, g, fmt, n, k, xbits, info)
    tiles = -(-m // 128) * (n // 256)
    assert (info.kernel, info.splits, info.grid_x, info.grid_y) == (1, 1, tiles, 0)
    y_ref = oracle.linear(oracle.bf16_bits_to_f32(xbits), packed, scales, k, fmt, g)
    assert_close(y_host(y), y_ref, "whole tail fmt=%d n=%d k=%d m=%d" % (fmt, n, k, m))


@pytest.mark.parametrize("fmt,n,k,m", [(NV, 512, 2048, 1), (MX, 512, 2048, 4), (NV, 300, 5120, 8),
                                       (NV, 512, 2048, 16), (MX, 384, 1056, 40), (NV, 8192, 1024, 1),
                                       (MX, 8448, 2048, 5), (NV, 640, 9216, 2), (MX, 640, 9216, 7)])
def test_one_hot_selects_weight_column(fmt, n, k, m):
    # x row i = e_{k_i}: y[i, :] is bf16(w[:, k_i]) exactly (the global scale is
    # applied after the sum, and every other product is zero).
    packed, scales, g = _quantized(fmt, n, k, tensor=3)
    ks = np.linspace(0, k - 1, m).astype(np.int64)
    x = np.zeros((m, k), np.float32)
    x[np.arange(m), ks] = 1.0
    xbits = oracle.f32_to_bf16_bits(x)
    y = y_host(_run_linear(packed, scales, g, fmt, n, k, xbits))
    w = oracle.dequantize(packed, scales, k, fmt, g)
    want = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(w[:, ks].T)).astype(np.float64)
    assert np.array_equal(y, want)   # +0 and -0 compare equal


@pytest.mark.parametrize("fmt,nh,k", [(MX, 640, 2048), (NV, 300, 1056), (MX, 1024, 4096), (NV, 256, 17408)])
@pytest.mark.parametrize("m", [1, 2, 4, 8, 12, 20, 40])
def test_gate_up_fused_equals_split(fmt, nh, k, m):
    pg, sg, gg = synth.packed_weight(synth.TINY, 60, nh, k, fmt)
    pu, su, gu = synth.packed_weight(synth.TINY, 61, nh, k, fmt)
    xbits = synth.activations(synth.TINY, m, k)
    pc, ps = fp4.fp4_prepare_gate_up(u8(pg), u8(sg), u8(pu), u8(su), nh, k, fmt)
    y = y_host_bits(fp4.fp4_w4a16_gate_up(x_dev(xbits), pc, ps, nh, float(gg), float(gu), fmt))
    yg = y_host_bits(_run_linear(pg, sg, gg, fmt, nh, k, xbits))
    yu = y_host_bits(_run_linear(pu, su, gu, fmt, nh, k, xbits))
    assert np.array_equal(y[:, :nh], yg) and np.array_equal(y[:, nh:], yu)
    y_ref = oracle.gate_up(oracle.bf16_bits_to_f32(xbits), pg, sg, pu, su, k, fmt, gg, gu)
    assert_close(oracle.bf16_bits_to_f32(y).astype(np.float64), y_ref, "gate_up")


@pytest.mark.parametrize("fmt,n,k", [(NV, 512, 256), (MX, 384, 3072), (NV, 256, 17408), (NV, 300, 5120),
                                     (MX, 8192, 1056), (MX, 16384, 1056)])
def test_gemv_batch_invariance(fmt, n, k):
    # Within one decode kernel, row i of an m-row call equals the same row of
    # a call with more rows, bit for bit (the summation order never depends on
    # m): each call is compared with the call of the most rows that runs on
    # the same kernel.  (MFMA decode: m = 9..16 stage 16 x rows instead of 8,
    # m = 17..32 32 rows with a second MFMA per fragment -- the same MFMA sums
    # for every row; wave-split: x rows staged 2, 4 or 8 at a time.)
    packed, scales, g = _quantized(fmt, n, k)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    x32 = synth.activations(synth.TINY, 32, k)
    ys, kernels = {}, {}
    for m in range(1, 33):
        info = fp4.fp4_dispatch_info()
        ys[m] = y_host_bits(fp4.fp4_w4a16_linear(x_dev(x32[:m]), pc, ps, n, float(g), fmt, info=info))
        kernels[m] = info.kernel
        assert info.kernel == decode_kernel(fmt, n, k, m), m
    for m in range(1, 33):
        top = max(q for q in range(1, 33) if kernels[q] == kernels[m])
        assert np.array_equal(ys[m], ys[top][:m]), (m, top)


@pytest.mark.parametrize("fmt,n,k,m", [(NV, 300, 5120, 8), (MX, 256, 17408, 3), (NV, 640, 2048, 64),
                                       (NV, 640, 9216, 8), (MX, 640, 9216, 1)])
def test_deterministic_and_workspace_poison(fmt, n, k, m):
    packed, scales, g = _quantized(fmt, n, k)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    xd = x_dev(synth.activations(synth.TINY, m, k))
    need = fp4.fp4_workspace_bytes(m, n, k, fmt)
    outs = []
    for fill in (0x00, 0xFF, 0x7F):
        ws = torch.full((max(need, 16),), fill, dtype=torch.uint8, device=DEV)
        outs.append(y_host_bits(fp4.fp4_w4a16_linear(xd, pc, ps, n, float(g), fmt, workspace=ws)))
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("fmt,n,k,m", [(NV, 512, 17408, 1), (NV, 640, 9216, 2), (MX, 1024, 9216, 1),
                                        (NV, 640, 9216, 6), (NV, 512, 5120, 100), (MX, 300, 4096, 300),
                                        (NV, 256, 3872, 40)])
def test_split_k_handshake_repeated(fmt, n, k, m):
    # The split-K finish exchanges partials between workgroups in one launch
    # (decode GEMV and MFMA decode splits; prefill tail tiles, the last case with a ragged
    # final K step); 40 back-to-back calls on one workspace must all give the
    # same bytes.
    packed, scales, g = _quantized(fmt, n, k, tensor=5)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    xd = x_dev(synth.activations(synth.TINY, m, k))
    info = fp4.fp4_dispatch_info()
    ws = torch.full((fp4.fp4_workspace_bytes(m, n, k, fmt),), 0x5A, dtype=torch.uint8, device=DEV)
    ys = [fp4.fp4_w4a16_linear(xd, pc, ps, n, float(g), fmt, workspace=ws, info=info) for _ in range(40)]
    assert info.splits > 1
    first = y_host_bits(ys[0])
    assert all(np.array_equal(first, y_host_bits(y)) for y in ys[1:])
    y_ref = oracle.linear(oracle.bf16_bits_to_f32(synth.activations(synth.TINY, m, k)), packed, scales, k, fmt, g)
    assert_close(oracle.bf16_bits_to_f32(first).astype(np.float64), y_ref, "split-K repeated")


def test_zero_rows_is_a_no_op():
    n, k = 512, 256
    packed, scales, g = _quantized(NV, n, k)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, NV)
    x = torch.empty((0, k), dtype=torch.bfloat16, device=DEV)
    y = fp4.fp4_w4a16_linear(x, pc, ps, n, float(g), NV)
    torch.cuda.synchronize()
    assert y.shape == (0, n)


@pytest.mark.parametrize("fmt", [NV, MX])
def test_minimal_shape(fmt):
    n, k, m = 1, 32, 1
    packed, scales, g = _quantized(fmt, 8, k)
    packed, scales = packed[:1], scales[:1]
    xbits = synth.activations(synth.TINY, m, k)
    y = _run_linear(packed, scales, g, fmt, n, k, xbits)
    y_ref = oracle.linear(oracle.bf16_bits_to_f32(xbits), packed, scales, k, fmt, g)
    assert_close(y_host(y), y_ref, "n=1 k=32")


def test_unit_scales_sum_of_x():
    # Every code 1.0, unit scales, G = 1: y[m, n] = sum_k x[m, k] (closed form).
    n, k = 256, 1024
    packed = np.full((n, k // 2), 0x22, np.uint8)
    xbits = synth.activations(synth.TINY, 4, k)
    for fmt, sb in ((NV, 0x38), (MX, 0x7F)):
        scales = np.full((n, k // GS[fmt]), sb, np.uint8)
        for m in (4, 20):
            xb = np.tile(xbits, (m // 4, 1))
            y = y_host(_run_linear(packed, scales, 1.0, fmt, n, k, xb))
            want = oracle.bf16_bits_to_f32(xb).astype(np.float64).sum(axis=1)
            assert_close(y, np.repeat(want[:, None], n, axis=1), "unit scales m=%d" % m)


@pytest.mark.parametrize("fmt,n,k,m", [(NV, 131000, 320, 8), (MX, 131072, 544, 3), (NV, 131072, 512, 5)])
def test_decode_mfma_wide_tiles(fmt, n, k, m):
    # Layers of >= 131072 rows run the MFMA decode kernel on 128-row tiles (two
    # 16-row blocks per wave share each x fragment); ragged n and k included.
    packed, scales, g = _quantized(fmt, n, k, tensor=7)
    xbits = synth.activations(synth.TINY, m, k)
    info = fp4.fp4_dispatch_info()
    y = _run_linear(packed, scales, g, fmt, n, k, xbits, info)
    assert info.kernel == 2 and info.splits == 1
    assert info.grid_x == -(-n // 256) * 256 // 128
    y_ref = oracle.linear(oracle.bf16_bits_to_f32(xbits), packed, scales, k, fmt, g)
    assert_close(y_host(y), y_ref, "wide tiles fmt=%d n=%d k=%d m=%d" % (fmt, n, k, m))


@pytest.mark.parametrize("fmt,nh,k,m", [(MX, 65536, 256, 4), (NV, 65536, 320, 8)])
def test_wide_tile_fused_equals_split(fmt, nh, k, m):
    # The fused launch (131072 rows: 128-row tiles) equals the two separate
    # 65536-row launches (64-row tiles) bit for bit: the tile size never
    # changes an output's summation order.
    pg, sg, gg = synth.packed_weight(synth.TINY, 62, nh, k, fmt)
    pu, su, gu = synth.packed_weight(synth.TINY, 63, nh, k, fmt)
    xbits = synth.activations(synth.TINY, m, k)
    pc, ps = fp4.fp4_prepare_gate_up(u8(pg), u8(sg), u8(pu), u8(su), nh, k, fmt)
    info = fp4.fp4_dispatch_info()
    y = y_host_bits(fp4.fp4_w4a16_gate_up(x_dev(xbits), pc, ps, nh, float(gg), float(gu), fmt, info=info))
    assert info.kernel == 2 and info.grid_x == 2 * nh // 128
    info1 = fp4.fp4_dispatch_info()
    yg = y_host_bits(_run_linear(pg, sg, gg, fmt, nh, k, xbits, info1))
    assert info1.grid_x == nh // 64
    yu = y_host_bits(_run_linear(pu, su, gu, fmt, nh, k, xbits))
    assert np.array_equal(y[:, :nh], yg) and np.array_equal(y[:, nh:], yu)
    y_ref = oracle.gate_up(oracle.bf16_bits_to_f32(xbits), pg, sg, pu, su, k, fmt, gg, gu)
    assert_close(oracle.bf16_bits_to_f32(y).astype(np.float64), y_ref, "wide gate_up")
