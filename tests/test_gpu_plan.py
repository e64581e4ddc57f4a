"""fp4_plan against the device: for every kernel a W4A16 call can take, the
plan the host utility computes from the device's compute-unit count is the
fp4_dispatch_info the call itself reports (kernel, K splits, grid, block and
the XCDs the tile order is dealt over)."""

import pytest
import torch

import fp4_weight_only_e2m1_amd as fp4
from gpu_util import DEV

pytestmark = pytest.mark.gpu

NV, MX = fp4.FMT_NVFP4, fp4.FMT_MXFP4

# (m, n, k, fmt, projections): the GEMV, the MFMA decode on 64- and 128-row
# tiles with and without K splits, the wave-split MFMA decode, the tile GEMM
# whole, with split tail tiles
# and with a two-way tail run whole, linear and fused gate_up.
SHAPES = [(1, 12288, 4096, MX, 2), (2, 248320, 5120, NV, 1), (1, 5120, 17408, NV, 1), (8, 5120, 17408, NV, 1),
          (8, 248320, 5120, NV, 1), (24, 5120, 6144, NV, 1), (4, 12288, 4096, MX, 2), (33, 17408, 5120, NV, 1),
          (1024, 17408, 5120, NV, 1), (1024, 17408, 5120, MX, 1), (1024, 12288, 4096, MX, 2),
          (1280, 5120, 17408, NV, 1), (4096, 4096, 5120, NV, 1), (4, 5120, 6144, NV, 1), (1, 2048, 4096, MX, 2),
          (8, 300, 1056, NV, 1)]


def test_plan_matches_the_calls():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for m, n, k, fmt, proj in SHAPES:
        cb, sb = fp4.fp4_prepared_bytes(n, k, fmt)
        pc = torch.zeros(proj * cb, dtype=torch.uint8, device=DEV)
        ps = torch.zeros(proj * sb, dtype=torch.uint8, device=DEV)
        x = torch.zeros((m, k), dtype=torch.bfloat16, device=DEV)
        info = fp4.fp4_dispatch_info()
        if proj == 1:
            fp4.fp4_w4a16_linear(x, pc, ps, n, 1.0, fmt, info=info)
        else:
            fp4.fp4_w4a16_gate_up(x, pc, ps, n, 1.0, 1.0, fmt, info=info)
        torch.cuda.synchronize()
        want = fp4.fp4_plan(m, n, k, fmt, proj, cus).as_dict()
        assert info.as_dict() == want, (m, n, k, fmt, proj, cus, info.as_dict(), want)
        if m > 32:
            assert info.xcds == min(8, max(1, cus // 32))
