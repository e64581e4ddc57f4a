"""fp4_w4a16_linear_noalloc through the C ABI: the same output as
fp4_w4a16_linear with a caller workspace, bit for bit, on two calls in a row
(the second with a smaller input), for the split-K decode kernels and the tile
GEMM's split tail tiles -- the paths that use a workspace -- and within the
layer's tolerance of the oracle; and the size limit of the library's scratch."""

import ctypes

import numpy as np
import pytest
import torch

import fp4_weight_only_e2m1_amd as fp4
import oracle
import synth
from gpu_util import DEV, assert_close, u8, x_dev, y_host, y_host_bits

pytestmark = pytest.mark.gpu

NV, MX = fp4.FMT_NVFP4, fp4.FMT_MXFP4
SCRATCH = 64 << 20


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _noalloc(lib, x, pc, ps, n, g, fmt, y, info):
    return lib.fp4_w4a16_linear_noalloc(_ptr(x), x.shape[0], x.shape[1], _ptr(pc), _ptr(ps), n, float(g), fmt,
                                        _ptr(y), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),
                                        ctypes.byref(info))


# Pairs of calls: the second smaller than the first.  Each call needs a
# workspace: split-K decode (GEMV m = 1, 2 and MFMA decode m = 3..32 on small
# layers past the wave-split kernel's k) or split tail tiles of the tile GEMM.
PAIRS = [
    [(NV, 5120, 17408, 8), (NV, 5120, 9216, 4)],    # MFMA decode, 6 K splits each
    [(MX, 1024, 9216, 2), (NV, 512, 9216, 1)],      # VALU GEMV, K split in three
    [(NV, 4096, 5120, 300), (MX, 512, 4096, 40)],   # tile GEMM, split tail tiles
]


@pytest.mark.parametrize("pair", PAIRS, ids=["decode", "gemv", "gemm"])
def test_noalloc_equals_linear_on_two_calls(pair):
    lib = fp4.load_library()
    for call, (fmt, n, k, m) in enumerate(pair):
        need = fp4.fp4_workspace_bytes(m, n, k, fmt)
        assert 0 < need <= SCRATCH, (fmt, n, k, m, need)
        packed, scales, g = synth.packed_weight(synth.TINY, 90 + call, n, k, fmt)
        pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
        xbits = synth.activations(synth.TINY, m, k)
        x = x_dev(xbits)
        info_ref, info = fp4.fp4_dispatch_info(), fp4.fp4_dispatch_info()
        y_ref = fp4.fp4_w4a16_linear(x, pc, ps, n, float(g), fmt, info=info_ref)
        y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
        assert _noalloc(lib, x, pc, ps, n, g, fmt, y, info) == 0
        assert info.as_dict() == info_ref.as_dict() and info.splits > 1
        assert np.array_equal(y_host_bits(y), y_host_bits(y_ref)), (call, fmt, n, k, m)
        y_or = oracle.linear(oracle.bf16_bits_to_f32(xbits), packed, scales, k, fmt, g)
        assert_close(y_host(y), y_or, "noalloc fmt=%d n=%d k=%d m=%d" % (fmt, n, k, m))


def test_noalloc_rejects_calls_beyond_the_scratch():
    # A GEMV shape whose split-K workspace is over 64 MiB: k = 2^20 makes
    # 256 K splits of fp32 partials for 2 rows of 65536 outputs (128 MiB).
    lib = fp4.load_library()
    m, n, k, fmt = 2, 65536, 1 << 20, NV
    assert fp4.fp4_workspace_bytes(m, n, k, fmt) > SCRATCH
    x = torch.zeros((m, 256), dtype=torch.bfloat16, device=DEV)   # never read: the call is rejected first
    pc = torch.zeros(256, dtype=torch.uint8, device=DEV)
    y = torch.zeros((m, n), dtype=torch.bfloat16, device=DEV)
    info = fp4.fp4_dispatch_info()
    st = lib.fp4_w4a16_linear_noalloc(_ptr(x), m, k, _ptr(pc), _ptr(pc), n, 1.0, fmt, _ptr(y), None,
                                      ctypes.byref(info))
    assert st == -4  # FP4_EWORKSPACE
