"""Bitwise pins of the compute kernels' own weight decode, and of the
dequantization export on the benchmark workloads' full weights.

The exhaustive table: row r of the weight takes scale byte r % 256 in every
group and its codes run 0, 1, ..., 15, 0, 1, ... along k.  With one-hot
activation rows (x row j = e_{c_j}, value 1.0) every output of a call is one
decoded weight: the kernels apply the NVFP4 global scale after the sum over
k, and every other product is x = 0 times a finite weight, so

  y[j, r] = bf16(fl32(fl32(E2M1(code[r, c_j]) * S(r)) * G))

bit for bit; a row that holds an infinite or NaN weight anywhere in [0, k)
gives NaN (0 * inf and NaN propagate), and a zero sum is +0 (the other
products include +0).  So all 16 codes x 256 scale bytes go through each
kernel's decoder -- the VALU GEMV (m = 1, 2), the MFMA decode on 64- and
128-row tiles, with and without a K split, the wave-split MFMA decode, and
the tile GEMM, whole tiles and split tail tiles -- for both formats and
several global scales.
Expected values come from the oracle's decode (oracle.dequantize); the
IEEE rule for the NaN rows is applied on top of it here.
"""

import numpy as np
import pytest
import torch

import fp4_weight_only_e2m1_amd as fp4
import oracle
from gpu_util import DEV, u8, weight, x_dev, y_host_bits

pytestmark = pytest.mark.gpu

NV, MX = fp4.FMT_NVFP4, fp4.FMT_MXFP4
GS = {NV: 16, MX: 32}
G_VALUES = {NV: [1.0, 2.0 ** -7, 0.0123 / 2688], MX: [1.0]}


def table_weight(fmt, n, k):
    """Row r: scale byte r % 256 in every group; codes 0..15 repeating along k."""
    codes = np.tile((np.arange(k) % 16).astype(np.uint8), (n, 1))
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = np.repeat((np.arange(n) % 256).astype(np.uint8)[:, None], k // GS[fmt], axis=1)
    return packed, scales


def one_hot(cols, k):
    x = np.zeros((len(cols), k), np.float32)
    x[np.arange(len(cols)), cols] = 1.0
    return oracle.f32_to_bf16_bits(x)


def expected_bits(packed, scales, k, fmt, g, cols):
    """bf16 bits of the one-hot outputs from the oracle's decoded weights."""
    w = oracle.dequantize(packed, scales, k, fmt, np.float32(g))          # [n, k] float32
    y = np.ascontiguousarray(w[:, cols].T)                                  # [m, n]
    for j, c in enumerate(cols):
        others = np.delete(w, c, axis=1)
        y[j, ~np.isfinite(others).all(axis=1)] = np.nan                     # 0 * inf, NaN elsewhere in the row
    y[y == 0] = 0.0                                                         # the sum of +0 and -0 is +0
    return oracle.f32_to_bf16_bits(y)


def canon(bits):
    """bf16 bits with every NaN made one pattern and -0 made +0."""
    b = np.array(bits, dtype=np.uint16, copy=True)
    b[((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)] = 0x7FC0
    b[b == 0x8000] = 0
    return b


def check(got, want, what):
    got, want = canon(got), canon(want)
    bad = got != want
    if bad.any():
        j, r = np.argwhere(bad)[0]
        raise AssertionError("%s: %d of %d outputs differ; first: row %d (scale byte %#x) x row %d: got %#06x "
                             "want %#06x" % (what, int(bad.sum()), bad.size, r, r % 256, j, got[j, r], want[j, r]))


def run(packed, scales, n, k, fmt, g, cols, kernel, splits=None, grid_x=None):
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    info = fp4.fp4_dispatch_info()
    y = fp4.fp4_w4a16_linear(x_dev(one_hot(cols, k)), pc, ps, n, float(np.float32(g)), fmt, info=info)
    got = y_host_bits(y)
    assert info.kernel == kernel, info.as_dict()
    if splits is not None:
        assert (info.splits > 1) == splits, info.as_dict()
    if grid_x is not None:
        assert info.grid_x == grid_x, info.as_dict()
    return got


# (n, m, k, column sets, kernel, split expected): each set is one call;
# together they cover codes 0..15 (the code of column c is c % 16).  Layers
# of fewer than 8192 rows with k <= 8192 run the wave-split kernel at m <= 8
# (MXFP4 at m <= 2 up to 16383 rows); the 64-row kernels are reached with
# more rows or k past 8192.
CASES = [
    # VALU GEMV: one or two rows, one column per row.
    ("gemv m=1", 16384, 1, 32, [[c] for c in range(16)], 0, False),
    ("gemv m=2", 16384, 2, 32, [[2 * c, 2 * c + 17] for c in range(8)], 0, False),
    # VALU GEMV with k = 8448: three K splits; the ones sit in the second split.
    ("gemv m=1 split", 256, 1, 8448, [[4096 + 37 * c] for c in range(16)], 0, True),
    # MFMA decode, 64-row tiles: 16 rows (one activation group), 32 rows (two), 3 rows.
    ("decode m=16", 256, 16, 32, [list(range(16))], 2, False),
    ("decode m=32", 256, 32, 64, [list(range(32))], 2, False),
    ("decode m=3", 8192, 3, 32, [[c, c + 5, c + 10] for c in range(0, 16, 3)], 2, False),
    # MFMA decode with k = 8448 on 4 tiles: eight K splits; row j's one in split j.
    ("decode m=8 split", 256, 8, 8448, [[1024 * j + 17 * j + c for j in range(8)] for c in (0, 8)], 2, True),
    # Wave-split MFMA decode: one stage (waves 1..3 idle), the ones in all four
    # waves' K quarters (k = 1024: one stage each), and 8 stages per wave.
    ("wave-split m=1", 256, 1, 32, [[c] for c in range(16)], 6, False),
    ("wave-split m=4", 256, 4, 1024, [[256 * w + 4 * q + w for w in range(4)] for q in range(4)], 6, False),
    ("wave-split m=8", 256, 8, 8192, [[1024 * j + 17 * j + c for j in range(8)] for c in (0, 8)], 6, False),
    # Tile GEMM: 64 rows (2-block instances), 128 rows (4-block instances).
    ("gemm m=64", 256, 64, 64, [list(range(64))], 1, False),
    ("gemm m=128", 256, 128, 128, [list(range(128))], 1, False),
    # Tile GEMM with k = 5120 on one tile: its K split 4 ways, summed by the reduce launch.
    ("gemm m=40 split", 256, 40, 5120, [[128 * j + (j % 16) for j in range(40)]], 1, True),
]


@pytest.mark.parametrize("fmt", [NV, MX])
@pytest.mark.parametrize("name,n,m,k,colsets,kernel,split", CASES, ids=[c[0] for c in CASES])
def test_exhaustive_table_through_kernel(fmt, name, n, m, k, colsets, kernel, split):
    packed, scales = table_weight(fmt, n, k)
    for g in G_VALUES[fmt]:
        for cols in colsets:
            assert len(cols) == m
            got = run(packed, scales, n, k, fmt, g, cols, kernel, splits=split)
            check(got, expected_bits(packed, scales, k, fmt, g, cols), "%s fmt=%d G=%r cols=%s" % (name, fmt, g,
                                                                                                   cols[:4]))


@pytest.mark.parametrize("fmt", [NV, MX])
def test_exhaustive_table_through_wide_decode_tiles(fmt):
    # 131072 rows (512 repeats of the 256 scale bytes): the MFMA decode kernel
    # on 128-row tiles, where each wave decodes two 16-row blocks.
    n, k = 131072, 32
    packed, scales = table_weight(fmt, n, k)
    want_rows = slice(0, 256)
    for g in G_VALUES[fmt][:2]:
        for cols in (list(range(8)), list(range(8, 16))):
            got = run(packed, scales, n, k, fmt, g, cols, 2, splits=False, grid_x=n // 128)
            want = expected_bits(packed[want_rows], scales[want_rows], k, fmt, g, cols)
            # Every block of 256 rows repeats the table.
            check(got, np.tile(want, (1, n // 256)), "wide tiles fmt=%d G=%r" % (fmt, g))


@pytest.mark.parametrize("fmt", [NV, MX])
def test_exhaustive_table_fused_gate_up(fmt):
    # The fused gate_up launch over [table; table reversed] applies each
    # half's global scale to its own outputs.
    n, k = 256, 32
    pg, sg = table_weight(fmt, n, k)
    pu, su = pg[::-1].copy(), sg[::-1].copy()
    gg, gu = (2.0 ** -7, 0.0123 / 2688) if fmt == NV else (1.0, 1.0)
    pc, ps = fp4.fp4_prepare_gate_up(u8(pg), u8(sg), u8(pu), u8(su), n, k, fmt)
    for m in (1, 8):
        cols = list(range(m))
        y = fp4.fp4_w4a16_gate_up(x_dev(one_hot(cols, k)), pc, ps, n, float(np.float32(gg)), float(np.float32(gu)), fmt)
        got = y_host_bits(y)
        want = np.concatenate([expected_bits(pg, sg, k, fmt, gg, cols), expected_bits(pu, su, k, fmt, gu, cols)], axis=1)
        check(got, want, "gate_up fmt=%d m=%d" % (fmt, m))


# ---------------------------------------------------------------- dequant on the workloads' weights


def _canon32(a):
    a = np.ascontiguousarray(a, dtype=np.float32).copy()
    a[np.isnan(a)] = np.float32(np.nan)
    return a.view(np.uint32)


# (workload, tensor, n, k, fmt): the benchmark's weights (gate_up's gate and
# up, lm_head, down_proj, o_proj, the prefill GEMM's NVFP4 and MXFP4).
FULL = [(1, 0, 12288, 4096, MX), (1, 1, 12288, 4096, MX), (2, 0, 248320, 5120, NV), (3, 0, 5120, 17408, NV),
        (3, 1, 5120, 6144, NV), (4, 0, 17408, 5120, NV), (4, 1, 17408, 5120, MX)]


@pytest.mark.parametrize("wid,tensor,n,k,fmt", FULL, ids=["gate", "up", "lm_head", "down_proj", "o_proj",
                                                          "prefill_nvfp4", "prefill_mxfp4"])
def test_dequant_bitwise_full_weights(wid, tensor, n, k, fmt):
    # fp4_dequantize of the whole prepared weight against the oracle, in
    # chunks of 4096 rows (sub-ranges of the prepared buffers: a chunk that
    # starts at a multiple of 16 rows is itself a prepared weight).
    packed, scales, g = weight(wid, tensor, n, k, fmt)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    cb, sb = fp4.fp4_prepared_bytes(n, k, fmt)
    n_pad = cb * 2 // (-(-k // 1024) * 1024)
    cb_row, sb_row = cb // n_pad, sb // n_pad
    chunk = 4096
    out = torch.empty((chunk, k), dtype=torch.float32, device=DEV)
    for r0 in range(0, n, chunk):
        rows = min(chunk, n - r0)
        o = out[:rows]
        fp4.fp4_dequantize(pc[r0 * cb_row:(r0 + rows) * cb_row], ps[r0 * sb_row:(r0 + rows) * sb_row], rows, k,
                           float(g), fmt, out=o)
        got = o.cpu().numpy()
        want = oracle.dequantize(packed[r0:r0 + rows], scales[r0:r0 + rows], k, fmt, g)
        if not np.array_equal(_canon32(got), _canon32(want)):
            bad = np.argwhere(_canon32(got) != _canon32(want))[0]
            raise AssertionError("rows %d..%d: first mismatch at %s: got %r want %r" %
                                 (r0, r0 + rows, tuple(bad), got[tuple(bad)], want[tuple(bad)]))
