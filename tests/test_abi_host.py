"""The C-ABI library on the host, without a GPU: it loads, exports every
symbol include/fp4w4a16.h declares, sizes buffers as documented, and rejects
bad arguments before touching the device."""

import ctypes
import os
import re

import pytest

import fp4_weight_only_e2m1_amd as fp4
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "fp4w4a16.h")
ST = {"OK": 0, "EINVAL": -1, "EFMT": -2, "EALIGN": -3, "EWORKSPACE": -4, "EHIP": -5}
NV, MX = fp4.FMT_NVFP4, fp4.FMT_MXFP4


@pytest.fixture(scope="module")
def lib():
    return fp4.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(fp4_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("fp4_prepared_bytes", "fp4_prepare", "fp4_prepare_gate_up", "fp4_workspace_bytes",
                 "fp4_w4a16_linear", "fp4_w4a16_gate_up", "fp4_dequantize", "fp4_status_string"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in fp4._SIGNATURES, name


def test_status_values_match_header():
    text = open(HEADER).read()
    for key, val in ST.items():
        assert re.search(r"FP4_%s\s*=\s*%d" % (key, val), text), key
    assert fp4.fp4_status_string(0) == "ok"
    assert "workspace" in fp4.fp4_status_string(ST["EWORKSPACE"])


@pytest.mark.parametrize("n,k,fmt", [(512, 256, NV), (24576, 4096, MX), (248320, 5120, NV), (5120, 17408, NV),
                                     (17408, 5120, MX), (1, 32, NV), (300, 1056, MX)])
def test_prepared_bytes(n, k, fmt):
    g = 16 if fmt == NV else 32
    n_pad = -(-n // 256) * 256
    k_pad = -(-k // 1024) * 1024
    cb, sb = fp4.fp4_prepared_bytes(n, k, fmt)
    assert cb == n_pad * k_pad // 2
    assert sb == n_pad * k_pad // g


def test_lm_head_prepared_bytes_equal_packed_bytes():
    # The 248320 x 5120 head needs no padding: the prepared weight is exactly
    # the packed checkpoint's 0.6660 GiB ("keep the ModelOpt NVFP4 lm_head packed").
    cb, sb = fp4.fp4_prepared_bytes(248320, 5120, NV)
    assert cb + sb == 248320 * 2560 + 248320 * 320


@pytest.mark.parametrize("n,k,fmt,bad", [(0, 256, NV, "EINVAL"), (512, 0, NV, "EINVAL"), (512, 48, NV, "EINVAL"),
                                         (512, 256, 2, "EFMT"), (512, 256, -1, "EFMT"),
                                         (1 << 25, 256, NV, "EINVAL"), (512, (1 << 20) + 32, MX, "EINVAL")])
def test_prepared_bytes_rejects(lib, n, k, fmt, bad):
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.fp4_prepared_bytes(n, k, fmt, ctypes.byref(cb), ctypes.byref(sb)) == ST[bad]


def _prefill_workspace(m, n, k, projections=1):
    # Prefill tiles are 128 x 256; 512 workgroups are resident at once.  Tiles
    # that do not fill a whole round are split along K (at most 512 / tail
    # ways, at least 20 K steps of 64 each) into fp32 partial tiles.
    tiles = -(-m // 128) * (projections * (-(-n // 256) * 256) // 256)
    # A tail that would split only two ways runs whole.
    tail = tiles % 512
    s = min(512 // tail, -(-k // 64) // 20) if tail else 1
    return 0 if s <= 2 else tail * s * 128 * 256 * 4


def test_workspace_bytes_policy():
    # m > 32 runs the prefill GEMM, whose tail tiles split K.
    assert fp4.fp4_workspace_bytes(33, 17408, 5120, NV) == _prefill_workspace(33, 17408, 5120) == 68 * 4 * 131072
    # m = 9..32 still runs the MFMA decode kernel: 272 tiles, no split; the
    # down_proj shape splits 6 ways as at m = 8, with partials for m rows.
    assert fp4.fp4_workspace_bytes(16, 17408, 5120, NV) == 0
    assert fp4.fp4_workspace_bytes(32, 17408, 5120, NV) == 0
    assert fp4.fp4_workspace_bytes(16, 5120, 17408, NV) == 6 * 16 * 5120 * 4 + 5120 // 64 * 6 * 8
    assert fp4.fp4_workspace_bytes(32, 5120, 17408, NV) == 6 * 32 * 5120 * 4 + 5120 // 64 * 6 * 8
    # The SwiGLU gate_up leaves the decode kernels above 16 rows.
    assert fp4.fp4_swiglu_workspace_bytes(17, 1024, 12288, MX) == _prefill_workspace(17, 1024, 12288, 2)
    assert fp4.fp4_workspace_bytes(1024, 17408, 5120, MX) == _prefill_workspace(1024, 17408, 5120) == 32 * 4 * 131072
    assert fp4.fp4_workspace_bytes(4096, 17408, 5120, NV) == _prefill_workspace(4096, 17408, 5120)
    assert fp4.fp4_workspace_bytes(65536, 256, 5120, NV) == 0      # 512 tiles: one full round, no tail
    assert fp4.fp4_workspace_bytes(200, 300, 256, NV) == 0         # 4 K steps: too short to split
    assert fp4.fp4_workspace_bytes(33, 1024, 12288, MX, 2) == _prefill_workspace(33, 1024, 12288, 2)
    # SwiGLU gate_up: the same plan as the fused gate_up, except at 17..32
    # rows, where the SwiGLU call takes the tile GEMM and gate_up the decode kernel.
    assert fp4.fp4_swiglu_workspace_bytes(1024, 12288, 4096, MX) == fp4.fp4_workspace_bytes(1024, 12288, 4096, MX, 2)
    for m in (1, 2, 8, 16):
        assert fp4.fp4_swiglu_workspace_bytes(m, 1024, 12288, MX) == fp4.fp4_workspace_bytes(m, 1024, 12288, MX, 2)
    for m in (17, 24, 32):
        assert fp4.fp4_swiglu_workspace_bytes(m, 1024, 12288, MX) == _prefill_workspace(m, 1024, 12288, 2)
        assert fp4.fp4_swiglu_workspace_bytes(m, 1024, 12288, MX) != fp4.fp4_workspace_bytes(m, 1024, 12288, MX, 2)
    # The lm_head GEMV splits K=5120 (5 slabs of 1024) in two; splitting never depends on m.
    # splits * m * rows fp32 partials, then one 8-byte flag per (64-row tile, split).
    ws1 = fp4.fp4_workspace_bytes(1, 248320, 5120, NV)
    ws8 = fp4.fp4_workspace_bytes(8, 248320, 5120, NV)
    flags = 248320 // 64 * 2 * 8
    assert ws1 == 2 * 1 * 248320 * 4 + flags
    # m >= 3 runs the MFMA decode kernel: 64-row tiles, K split only for layers
    # under 128 tiles, to about 512 workgroups (at least 4 stages of 256 codes each).
    assert ws8 == 0                                             # 3880 tiles: no split
    down = fp4.fp4_workspace_bytes(8, 5120, 17408, NV)          # 80 tiles: 6 splits
    assert down == 6 * 8 * 5120 * 4 + 5120 // 64 * 6 * 8
    # Layers under 128 tiles with k <= 8192 take the wave-split kernel at
    # m = 1..8 (K split over the waves of one workgroup: no workspace), the
    # 64-row kernel above 8 rows (24 stages: 6 splits).
    for m in range(1, 9):
        assert fp4.fp4_workspace_bytes(m, 5120, 6144, NV) == 0
        assert fp4.fp4_workspace_bytes(m, 2048, 1024, MX, 2) == 0
    assert fp4.fp4_workspace_bytes(9, 5120, 6144, NV) == 6 * 9 * 5120 * 4 + 80 * 6 * 8
    assert fp4.fp4_workspace_bytes(8, 5120, 8192, NV) == 0
    assert fp4.fp4_workspace_bytes(8, 5120, 8448, NV) == 6 * 8 * 5120 * 4 + 80 * 6 * 8   # 33 stages
    assert fp4.fp4_workspace_bytes(8, 8192, 4096, NV) == 0                                 # 128 tiles: unsplit
    # Greedy argmax on the wave-split kernel: no partials, one key per
    # (16-row tile, activation row).
    assert fp4.fp4_argmax_workspace_bytes(4, 5000, 2048, NV) == 5120 // 16 * 4 * 8
    # The SwiGLU gate_up stays on the 64-row kernel (its 16-row tiles would
    # hold only gate or only up rows): 2048 rows per half, 32 tiles each,
    # 16 stages: min(512 / 32, 16 / 4) = 4 splits over 4096 rows.
    assert fp4.fp4_swiglu_workspace_bytes(4, 2048, 4096, NV) == 4 * 4 * 4096 * 4 + 4096 // 64 * 4 * 8
    assert fp4.fp4_workspace_bytes(4, 2048, 4096, NV, 2) == 0
    # gate_up: two projections, each split like the separate linear.
    one = fp4.fp4_workspace_bytes(4, 12288, 4096, MX, 1)
    two = fp4.fp4_workspace_bytes(4, 12288, 4096, MX, 2)
    assert two == 2 * one
    assert fp4.fp4_workspace_bytes(1, 512, 256, NV) == 0


def test_plan_follows_cu_count_only_in_the_xcd_deal():
    # A device of fewer compute units (a partition, a smaller part) gets the
    # same kernel, tiles and K splits -- so the same summation order and the
    # same output bits -- and only deals the tile GEMM's tiles over its own XCDs
    # (32 CUs each).
    shapes = [(1024, 17408, 5120, NV, 1), (1024, 17408, 5120, MX, 1), (4096, 17408, 5120, NV, 1),
              (33, 1024, 12288, MX, 2), (200, 248320, 5120, NV, 1), (1024, 12288, 4096, MX, 2),
              (1, 12288, 4096, MX, 2), (8, 5120, 17408, NV, 1), (24, 5120, 6144, NV, 1), (2, 248320, 5120, NV, 1)]
    for m, n, k, fmt, proj in shapes:
        full = fp4.fp4_plan(m, n, k, fmt, proj, 256).as_dict()
        for cus, xcds in [(256, 8), (304, 8), (224, 7), (128, 4), (64, 2), (32, 1), (20, 1)]:
            got = fp4.fp4_plan(m, n, k, fmt, proj, cus).as_dict()
            want = dict(full, xcds=xcds if m > 32 else 0)
            assert got == want, (m, n, k, cus, got, want)
    # The plans the headline shapes run: the 17408 x 5120 prefill GEMM at
    # m = 1024 has 8 x 68 = 544 tiles: 512 whole, 32 tail tiles in 4 K splits.
    p = fp4.fp4_plan(1024, 17408, 5120, NV, 1, 256)
    assert (p.kernel, p.splits, p.grid_x, p.grid_y, p.block, p.xcds) == (1, 4, 512, 128, 256, 8)
    # gate_up 2 x 12288 x 4096 at m = 1024: 768 tiles; a tail of 256 would
    # split only two ways, so all 768 run whole.
    p = fp4.fp4_plan(1024, 12288, 4096, MX, 2, 256)
    assert (p.kernel, p.splits, p.grid_x, p.grid_y) == (1, 1, 768, 0)
    assert fp4.fp4_workspace_bytes(1024, 12288, 4096, MX, 2) == 0
    # Decode: the MFMA kernel on 64-row tiles, down_proj split 6 ways along K.
    p = fp4.fp4_plan(8, 5120, 17408, NV, 1, 32)
    assert (p.kernel, p.splits, p.grid_x, p.grid_y, p.block, p.xcds) == (2, 6, 80, 6, 256, 0)
    p = fp4.fp4_plan(1, 248320, 5120, NV, 1, 256)
    assert (p.kernel, p.splits, p.grid_x, p.grid_y) == (0, 2, 248320 // 64, 2)
    # o_proj (5120 x 6144): the wave-split kernel at m = 1..8, 320 16-row
    # workgroups; the 64-row MFMA decode split 6 ways above.
    for m in (1, 2, 4, 8):
        p = fp4.fp4_plan(m, 5120, 6144, NV, 1, 256)
        assert (p.kernel, p.splits, p.grid_x, p.grid_y, p.block, p.xcds) == (6, 1, 320, 1, 256, 0)
    p = fp4.fp4_plan(9, 5120, 6144, NV, 1, 256)
    assert (p.kernel, p.splits, p.grid_x, p.grid_y) == (2, 6, 80, 6)
    p = fp4.fp4_plan(4, 5120, 6144, MX, 2, 256)
    assert (p.kernel, p.splits, p.grid_x, p.grid_y) == (6, 1, 640, 1)
    # The MXFP4 gate_up (2 x 12288 x 4096): the wave-split kernel at m = 1, 2
    # (1536 workgroups), the MFMA decode from m = 3: on 96-row tiles (256
    # six-wave workgroups) at m = 3..8, on 64-row tiles from m = 9; the
    # separate 12288-row halves keep 64-row tiles.  NVFP4 keeps the GEMV at
    # m = 1, 2.
    for m in (1, 2):
        p = fp4.fp4_plan(m, 12288, 4096, MX, 2, 256)
        assert (p.kernel, p.splits, p.grid_x, p.grid_y) == (6, 1, 1536, 1)
        assert fp4.fp4_plan(m, 12288, 4096, NV, 2, 256).kernel == 0
    for m in range(3, 9):
        for fmt in (NV, MX):
            p = fp4.fp4_plan(m, 12288, 4096, fmt, 2, 256)
            assert (p.kernel, p.splits, p.grid_x, p.grid_y, p.block) == (2, 1, 256, 1, 384)
            p = fp4.fp4_plan(m, 12288, 4096, fmt, 1, 256)
            assert (p.kernel, p.splits, p.grid_x, p.grid_y, p.block) == (2, 1, 192, 1, 256)
    p = fp4.fp4_plan(9, 12288, 4096, MX, 2, 256)
    assert (p.kernel, p.splits, p.grid_x, p.grid_y, p.block) == (2, 1, 384, 1, 256)
    assert fp4.fp4_plan(1, 16384, 4096, MX, 1, 256).kernel == 0      # 256 tiles
    assert fp4.fp4_plan(1, 12288, 8448, MX, 1, 256).kernel == 0      # 33 K stages
    p = fp4.fp4_plan(0, 512, 256, NV, 1, 256)
    assert p.as_dict() == dict(kernel=0, splits=0, grid_x=0, grid_y=0, block=0, xcds=0)


@pytest.mark.parametrize("args", [(1, 512, 256, NV, 1, 0), (1, 512, 256, NV, 3, 256), (-1, 512, 256, NV, 1, 256),
                                  (1, 0, 256, NV, 1, 256), (1, 512, 48, NV, 1, 256)])
def test_plan_rejects(lib, args):
    info = fp4.fp4_dispatch_info()
    assert lib.fp4_plan(*args, ctypes.byref(info)) == ST["EINVAL"]
    assert lib.fp4_plan(1, 512, 256, 5, 1, 256, ctypes.byref(info)) == ST["EFMT"]
    assert lib.fp4_plan(1, 512, 256, NV, 1, 256, None) == ST["EINVAL"]


FAKE = 0x10000  # an aligned address that is never dereferenced: every call below fails validation first


def _linear(lib, m=1, k=256, n=512, fmt=NV, x=FAKE, c=FAKE, s=FAKE, y=FAKE, ws=None, ws_bytes=0):
    return lib.fp4_w4a16_linear(x, m, k, c, s, n, 1.0, fmt, y, ws, ws_bytes, None, None)


def test_linear_argument_checks(lib):
    assert _linear(lib, fmt=7) == ST["EFMT"]
    assert _linear(lib, k=48) == ST["EINVAL"]
    assert _linear(lib, k=0) == ST["EINVAL"]
    assert _linear(lib, n=0) == ST["EINVAL"]
    assert _linear(lib, m=-1) == ST["EINVAL"]
    assert _linear(lib, x=None) == ST["EINVAL"]
    assert _linear(lib, y=None) == ST["EINVAL"]
    assert _linear(lib, x=FAKE + 2) == ST["EALIGN"]
    assert _linear(lib, c=FAKE + 8) == ST["EALIGN"]
    assert _linear(lib, y=FAKE + 4) == ST["EALIGN"]
    # m == 0 is a valid empty call: nothing to do, nothing enqueued.
    assert _linear(lib, m=0, x=None, y=None) == ST["OK"]
    # A split-K shape needs a workspace.
    need = fp4.fp4_workspace_bytes(1, 5120, 17408, NV)
    assert need > 0
    assert _linear(lib, k=17408, n=5120, ws=FAKE, ws_bytes=need - 1) == ST["EWORKSPACE"]
    assert _linear(lib, k=17408, n=5120, ws=None, ws_bytes=need) == ST["EINVAL"]
    assert _linear(lib, k=17408, n=5120, ws=FAKE + 4, ws_bytes=need) == ST["EALIGN"]


def test_gate_up_and_prepare_argument_checks(lib):
    assert lib.fp4_w4a16_gate_up(FAKE, 1, 100, FAKE, FAKE, 512, 1.0, 1.0, NV, FAKE, None, 0, None, None) == \
        ST["EINVAL"]
    assert lib.fp4_w4a16_gate_up(FAKE, 1, 256, FAKE, FAKE, 512, 1.0, 1.0, 3, FAKE, None, 0, None, None) == ST["EFMT"]
    assert lib.fp4_w4a16_gate_up(FAKE, 1, 256, FAKE, FAKE, 1 << 24, 1.0, 1.0, NV, FAKE, None, 0, None, None) == \
        ST["EINVAL"]
    assert lib.fp4_prepare(FAKE, FAKE, 512, 256, NV, FAKE + 1, FAKE, None) == ST["EALIGN"]
    assert lib.fp4_prepare(None, FAKE, 512, 256, NV, FAKE, FAKE, None) == ST["EINVAL"]
    assert lib.fp4_prepare(FAKE, FAKE, 512, 250, NV, FAKE, FAKE, None) == ST["EINVAL"]
    assert lib.fp4_prepare_gate_up(FAKE, FAKE, FAKE, None, 512, 256, MX, FAKE, FAKE, None) == ST["EINVAL"]
    assert lib.fp4_dequantize(FAKE, FAKE, 512, 256, 1.0, 9, FAKE, None) == ST["EFMT"]
    assert lib.fp4_dequantize(FAKE, FAKE, 512, 256, 1.0, NV, FAKE + 4, None) == ST["EALIGN"]
    sz = ctypes.c_size_t()
    assert lib.fp4_workspace_bytes(1, 512, 256, NV, 3, ctypes.byref(sz)) == ST["EINVAL"]


def test_split_count_independent_of_m_and_fusion():
    # The workspace is splits * (m * rows * 4 + one 8-byte flag per workgroup
    # tile); dividing out recovers the split count, which must not change with
    # m within a kernel: the VALU GEMV (m = 1, 2; 64-row tiles for layers of at
    # least 512 of them, else 32-row tiles) and the MFMA decode kernel (m = 3..8,
    # 64-row tiles).
    for n, k, fmt in [(5120, 17408, NV), (7168, 12288, NV), (12288, 4096, MX), (248320, 5120, NV)]:
        rows = -(-n // 256) * 256
        for ms, tile in [(range(1, 3), 64 if rows // 64 >= 512 else 32), (range(3, 9), 64)]:
            counts = set()
            for m in ms:
                ws = fp4.fp4_workspace_bytes(m, n, k, fmt)
                per_split = 4 * m * rows + rows // tile * 8
                assert ws % per_split == 0
                counts.add(ws // per_split)
            assert len(counts) == 1


def test_argmax_workspace_bytes():
    # The call's own workspace (256-byte aligned), then one 8-byte key per
    # (workgroup tile, activation row).
    # lm_head m = 1: the GEMV, 64-row tiles (3880), K split 2 ways.
    base = 2 * 1 * 248320 * 4 + 3880 * 2 * 8
    assert fp4.fp4_argmax_workspace_bytes(1, 248320, 5120, NV) == -(-base // 256) * 256 + 3880 * 1 * 8
    # lm_head m = 8: the MFMA decode on 128-row tiles (1940), unsplit.
    assert fp4.fp4_argmax_workspace_bytes(8, 248320, 5120, NV) == 1940 * 8 * 8
    # A small layer at m = 4: the wave-split kernel, 16-row tiles, 32 of them.
    assert fp4.fp4_argmax_workspace_bytes(4, 512, 256, MX) == 32 * 4 * 8
    assert fp4.fp4_argmax_workspace_bytes(0, 512, 256, MX) == 0


def _argmax(lib, m=1, k=256, n=512, fmt=NV, x=FAKE, y=None, idx=FAKE, val=None, ws=FAKE, ws_bytes=1 << 20):
    return lib.fp4_w4a16_linear_argmax(x, m, k, FAKE, FAKE, n, 1.0, fmt, y, idx, val, ws, ws_bytes, None, None)


def test_argmax_argument_checks(lib):
    sz = ctypes.c_size_t()
    # The documented limit: m = 1..32 (the decode kernels), FP4_EINVAL above.
    assert lib.fp4_argmax_workspace_bytes(32, 512, 256, NV, ctypes.byref(sz)) == ST["OK"]
    assert sz.value == 8 * 32 * 8      # 8 tiles of 64 rows, one key per (tile, row), no split
    assert lib.fp4_argmax_workspace_bytes(33, 512, 256, NV, ctypes.byref(sz)) == ST["EINVAL"]
    assert _argmax(lib, m=33) == ST["EINVAL"]         # decode rows only (m <= 32)
    # m = 32 passes every check (the failure left is the missing workspace).
    assert _argmax(lib, m=32, ws=None) == ST["EINVAL"]
    assert _argmax(lib, m=32, ws_bytes=8 * 32 * 8 - 1) == ST["EWORKSPACE"]
    assert _argmax(lib, idx=None) == ST["EINVAL"]
    assert _argmax(lib, x=None) == ST["EINVAL"]
    assert _argmax(lib, fmt=5) == ST["EFMT"]
    assert _argmax(lib, idx=FAKE + 2) == ST["EALIGN"]
    assert _argmax(lib, val=FAKE + 1) == ST["EALIGN"]
    assert _argmax(lib, y=FAKE + 4) == ST["EALIGN"]
    need = fp4.fp4_argmax_workspace_bytes(1, 512, 256, NV)
    assert _argmax(lib, ws_bytes=need - 1) == ST["EWORKSPACE"]
    assert _argmax(lib, ws=None) == ST["EINVAL"]


def _w4a4_workspace(m, n, k, projections=1):
    # Quantized activations: rows padded to 256-row tiles, k to 128 codes;
    # codes (half a byte each) then one E8M0 byte per 32 codes; 256-byte
    # aligned.  Then the tail partials of the 256 x 256 tile plan: 256
    # workgroups resident (one per CU), K stepping 128 codes, splits of at
    # least 4 steps.
    r, kk = -(-m // 256) * 256, -(-k // 128) * 128
    act = -(-(r * kk // 2 + r * kk // 32) // 256) * 256
    tiles = -(-m // 256) * (projections * (-(-n // 256) * 256) // 256)
    tail = tiles % 256
    s = min(256 // tail, -(-k // 128) // 4) if tail else 1
    # Where that split is two ways, the tail tiles run as two 128-row halves
    # over all of K instead, with no partials.
    return act + (0 if s <= 2 else tail * s * 256 * 256 * 4)


def test_w4a4_sizes():
    assert fp4.fp4_w4a4_act_bytes(1, 256) == (256 * 128, 256 * 8)
    assert fp4.fp4_w4a4_act_bytes(1024, 4096) == (1024 * 2048, 1024 * 128)
    assert fp4.fp4_w4a4_act_bytes(257, 4064) == (512 * 2048, 512 * 128)
    assert fp4.fp4_w4a4_workspace_bytes(1, 512, 256) == _w4a4_workspace(1, 512, 256) == 34816
    # gate_up at m = 1024: 384 tiles; the 128 past the first round run as row halves.
    assert fp4.fp4_w4a4_workspace_bytes(1024, 12288, 4096, 2) == _w4a4_workspace(1024, 12288, 4096, 2)
    assert fp4.fp4_w4a4_workspace_bytes(1024, 12288, 4096, 2) == 2228224
    # k = 5120, n = 17408: 16 tail tiles split 10 ways along K.
    assert fp4.fp4_w4a4_workspace_bytes(1024, 17408, 5120) == 1024 * 2560 + 1024 * 160 + 16 * 10 * 262144
    for m, n, k in [(16, 17408, 5120), (4096, 17408, 5120), (300, 300, 1056), (9, 5120, 17408)]:
        assert fp4.fp4_w4a4_workspace_bytes(m, n, k) == _w4a4_workspace(m, n, k), (m, n, k)
    assert fp4.fp4_w4a4_workspace_bytes(0, 512, 256) == 0


def _w4a4(lib, m=16, k=256, n=512, fmt=MX, x=FAKE, c=FAKE, s=FAKE, y=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return lib.fp4_w4a4_linear(x, m, k, c, s, n, fmt, y, ws, ws_bytes, None, None)


def test_w4a4_argument_checks(lib):
    # NVFP4 weights (E4M3 block-16 scales) cannot feed the block-scaled MFMA.
    assert _w4a4(lib, fmt=NV) == ST["EFMT"]
    assert _w4a4(lib, fmt=9) == ST["EFMT"]
    assert _w4a4(lib, k=48) == ST["EINVAL"]
    assert _w4a4(lib, n=0) == ST["EINVAL"]
    assert _w4a4(lib, m=-1) == ST["EINVAL"]
    assert _w4a4(lib, x=None) == ST["EINVAL"]
    assert _w4a4(lib, y=None) == ST["EINVAL"]
    assert _w4a4(lib, ws=None) == ST["EINVAL"]      # the quantized activations live in the workspace
    assert _w4a4(lib, x=FAKE + 2) == ST["EALIGN"]
    assert _w4a4(lib, ws=FAKE + 8) == ST["EALIGN"]
    assert _w4a4(lib, ws_bytes=fp4.fp4_w4a4_workspace_bytes(16, 512, 256) - 1) == ST["EWORKSPACE"]
    assert _w4a4(lib, m=0, x=None, y=None, ws=None) == ST["OK"]
    assert lib.fp4_w4a4_gate_up(FAKE, 16, 256, FAKE, FAKE, 512, NV, FAKE, FAKE, 1 << 30, None, None) == ST["EFMT"]
    assert lib.fp4_quantize_act_mxfp4(FAKE, 4, 48, FAKE, FAKE, None) == ST["EINVAL"]
    assert lib.fp4_quantize_act_mxfp4(FAKE, 4, 64, FAKE + 4, FAKE, None) == ST["EALIGN"]
    assert lib.fp4_quantize_act_mxfp4(None, 0, 64, None, None, None) == ST["OK"]
    sz = ctypes.c_size_t()
    assert lib.fp4_w4a4_workspace_bytes(16, 512, 256, 3, ctypes.byref(sz)) == ST["EINVAL"]


def _moe(lib, name, tokens=4, k=256, n=512, experts=8, fmt=NV, x=FAKE, gs=FAKE, offsets=FAKE, ptok=FAKE,
         pairs=16, y=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return getattr(lib, name)(x, tokens, k, FAKE, FAKE, n, experts, gs, fmt, offsets, ptok, pairs, y, ws, ws_bytes,
                              None, None)


@pytest.mark.parametrize("name", ["fp4_w4a16_moe_decode", "fp4_w4a16_moe_prefill"])
def test_moe_argument_checks(lib, name):
    assert _moe(lib, name, fmt=3) == ST["EFMT"]
    assert _moe(lib, name, experts=0) == ST["EINVAL"]
    assert _moe(lib, name, experts=65536) == ST["EINVAL"]
    assert _moe(lib, name, pairs=-1) == ST["EINVAL"]
    assert _moe(lib, name, k=100) == ST["EINVAL"]
    assert _moe(lib, name, tokens=0) == ST["EINVAL"]
    assert _moe(lib, name, gs=None) == ST["EINVAL"]            # NVFP4 needs the global scales
    assert _moe(lib, name, offsets=None) == ST["EINVAL"]
    assert _moe(lib, name, offsets=FAKE + 2) == ST["EALIGN"]
    assert _moe(lib, name, ptok=FAKE + 1) == ST["EALIGN"]
    assert _moe(lib, name, y=FAKE + 8) == ST["EALIGN"]
    # Both routes fetch each pair's x row by its token id: no workspace.
    assert fp4.fp4_moe_workspace_bytes(16, 256) == 0
    assert fp4.fp4_moe_workspace_bytes(1 << 20, 1 << 20) == 0
    # No pairs: nothing to compute, nothing checked beyond the sizes.
    assert _moe(lib, name, pairs=0, x=None, y=None, ws=None) == ST["OK"]


def test_moe_prefill_grid_limit(lib):
    # ceil(pairs / 128) + min(experts, pairs) tile slots x ceil(n / 256)
    # weight tiles of 256 threads must stay below 2^32 threads.
    assert _moe(lib, "fp4_w4a16_moe_prefill", pairs=1 << 20, experts=65535, n=1 << 24) == ST["EINVAL"]


def _moe_swiglu(lib, tokens=4, k=256, n_half=512, experts=8, fmt=NV, x=FAKE, gs=FAKE, offsets=FAKE, ptok=FAKE,
                pairs=16, y=FAKE):
    return lib.fp4_w4a16_moe_prefill_swiglu(x, tokens, k, FAKE, FAKE, n_half, experts, gs, fmt, offsets, ptok, pairs,
                                            y, None, None)


def test_moe_prefill_swiglu_argument_checks(lib):
    assert _moe_swiglu(lib, fmt=2) == ST["EFMT"]
    assert _moe_swiglu(lib, experts=0) == ST["EINVAL"]
    assert _moe_swiglu(lib, n_half=0) == ST["EINVAL"]
    assert _moe_swiglu(lib, k=48) == ST["EINVAL"]
    assert _moe_swiglu(lib, gs=None) == ST["EINVAL"]           # NVFP4 needs the [experts][2] global scales
    assert _moe_swiglu(lib, gs=FAKE + 2) == ST["EALIGN"]
    assert _moe_swiglu(lib, x=FAKE + 8) == ST["EALIGN"]
    assert _moe_swiglu(lib, ptok=None) == ST["EINVAL"]
    # Two projections of n_half rows must fit the row limit.
    assert _moe_swiglu(lib, n_half=(1 << 23) + 1) == ST["EINVAL"]
    assert _moe_swiglu(lib, pairs=0, x=None, y=None) == ST["OK"]


def test_w4a4_nvfp4_sizes_and_argument_checks(lib):
    # Workspace: the bf16 quantized activations (256-byte aligned), then the
    # W4A16 call's own workspace.
    for m, n, k, proj in [(1, 5120, 17408, 1), (8, 5120, 17408, 1), (1024, 17408, 5120, 1), (3, 12288, 4096, 2)]:
        want = -(-2 * m * k // 256) * 256 + fp4.fp4_workspace_bytes(m, n, k, NV, proj)
        assert fp4.fp4_w4a4_nvfp4_workspace_bytes(m, n, k, proj) == want
    assert fp4.fp4_w4a4_nvfp4_workspace_bytes(0, 512, 256) == 0
    info = fp4.fp4_dispatch_info()

    def lin(m=4, k=256, n=512, gx=0.01, ws=FAKE, ws_bytes=1 << 30, x=FAKE, y=FAKE):
        return lib.fp4_w4a4_nvfp4_linear(x, m, k, FAKE, FAKE, n, 1.0, gx, y, ws, ws_bytes, None, ctypes.byref(info))

    for gx in (0.0, -1.0, float("inf"), float("nan")):
        assert lin(gx=gx) == ST["EINVAL"]
        assert lib.fp4_quantize_act_nvfp4(FAKE, 4, 256, ctypes.c_float(gx), FAKE, FAKE, None) == ST["EINVAL"]
    assert lin(k=48) == ST["EINVAL"]
    assert lin(m=-1) == ST["EINVAL"]
    assert lin(ws=None) == ST["EINVAL"]
    assert lin(x=FAKE + 8) == ST["EALIGN"]
    assert lin(ws_bytes=2 * 4 * 256 - 1) == ST["EWORKSPACE"]
    assert lin(m=0, x=None, y=None, ws=None, ws_bytes=0) == ST["OK"]
    assert lib.fp4_quantize_act_nvfp4(FAKE, 4, 48, ctypes.c_float(1.0), FAKE, FAKE, None) == ST["EINVAL"]
    assert lib.fp4_quantize_act_nvfp4(FAKE + 4, 4, 64, ctypes.c_float(1.0), FAKE, FAKE, None) == ST["EALIGN"]
    assert lib.fp4_quantize_act_nvfp4(None, 0, 64, ctypes.c_float(1.0), None, None, None) == ST["OK"]
    assert lib.fp4_w4a4_nvfp4_gate_up(FAKE, 4, 256, FAKE, FAKE, (1 << 23) + 1, 1.0, 1.0, 0.01, FAKE, FAKE, 1 << 30,
                                      None, None) == ST["EINVAL"]


def test_decode_dispatch_rule_over_a_grid():
    # The decode kernel fp4_plan reports (the one the calls take, checked on
    # the GPU by test_gpu_plan) against the rule the GPU tests restate
    # (gpu_util.decode_kernel), over rows, k, formats, m and both layouts.
    from gpu_util import decode_kernel, decode_splits, decode_tile_rows
    tiles96 = 0
    for fmt in (NV, MX):
        for n in (17, 300, 2048, 5120, 7936, 8192, 8448, 9216, 12288, 16128, 16384, 131072):
            for k in (32, 544, 1056, 6144, 8192, 8448, 17408):
                for m in (1, 2, 3, 4, 8, 9, 16, 32):
                    for proj in (1, 2):
                        p = fp4.fp4_plan(m, n, k, fmt, proj, 256)
                        assert p.kernel == decode_kernel(fmt, n, k, m), (fmt, n, k, m, proj, p.as_dict())
                        rows = proj * (-(-n // 256) * 256)
                        if p.kernel == 6:
                            assert (p.splits, p.grid_x, p.block) == (1, rows // 16, 256)
                            assert fp4.fp4_workspace_bytes(m, n, k, fmt, proj) == 0
                        if p.kernel == 2:
                            tr = decode_tile_rows(n, k, m, proj)
                            want = (decode_splits(n, k), rows // tr, decode_splits(n, k), 384 if tr == 96 else 256)
                            assert (p.splits, p.grid_x, p.grid_y, p.block) == want, (fmt, n, k, m, proj, p.as_dict())
                            tiles96 += tr == 96
    assert tiles96 > 0
