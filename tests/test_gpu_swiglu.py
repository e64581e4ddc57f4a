"""GPU parity of the SwiGLU gate_up (fp4_w4a16_gate_up_swiglu) against the
oracle: the interleaved prepared layout byte for byte, and y = silu(gate) * up
within the layer's tolerance on every kernel (VALU GEMV split and unsplit,
MFMA decode split and unsplit, the tile GEMM's partial-tile route with a
ragged tail), plus determinism under poisoned workspaces."""

import numpy as np
import pytest
import torch

import fp4_weight_only_e2m1_amd as fp4
import oracle
import synth
from gpu_util import DEV, assert_close, u8, x_dev, y_host, y_host_bits

pytestmark = pytest.mark.gpu

NV, MX = fp4.FMT_NVFP4, fp4.FMT_MXFP4


def _weights(fmt, nh, k, seed):
    pg, sg, gg = synth.packed_weight(synth.TINY, 110 + seed, nh, k, fmt)
    pu, su, gu = synth.packed_weight(synth.TINY, 111 + seed, nh, k, fmt)
    return pg, sg, gg, pu, su, gu


def test_interleaved_layout_bytes():
    fmt, nh, k = NV, 300, 1056
    pg, sg, _, pu, su, _ = _weights(fmt, nh, k, 0)
    pc, ps = fp4.fp4_prepare_gate_up_interleaved(u8(pg), u8(sg), u8(pu), u8(su), nh, k, fmt)
    # The plain prepared halves, re-ordered by the interleave rule, must give the same bytes.
    cg, cs = fp4.fp4_prepare(u8(pg), u8(sg), nh, k, fmt)
    cu, cu_s = fp4.fp4_prepare(u8(pu), u8(su), nh, k, fmt)
    n_pad = 512          # n rounded up to 256; k_pad = 2048 codes = 1024 bytes per row
    row_bytes = 1024
    c = pc.cpu().numpy().reshape(2 * n_pad, row_bytes)
    g = cg.cpu().numpy().reshape(n_pad, row_bytes)
    u = cu.cpu().numpy().reshape(n_pad, row_bytes)
    for R in range(2 * n_pad):
        src = g if (R >> 4) & 1 == 0 else u
        assert np.array_equal(c[R], src[(R >> 5) * 16 + (R & 15)]), R
    # Scales: prepared 16-row groups alternate gate, up.
    grp = ps.cpu().numpy().reshape(2 * n_pad // 16, -1)
    gs_ = cs.cpu().numpy().reshape(n_pad // 16, -1)
    us_ = cu_s.cpu().numpy().reshape(n_pad // 16, -1)
    for q in range(2 * n_pad // 16):
        assert np.array_equal(grp[q], (gs_ if q % 2 == 0 else us_)[q // 2]), q


@pytest.mark.parametrize("fmt,nh,k", [(MX, 640, 2048), (NV, 300, 1056), (NV, 256, 17408), (MX, 1024, 4096)])
@pytest.mark.parametrize("m", [1, 2, 3, 5, 8, 16, 24, 100, 300])
def test_swiglu_matches_oracle(fmt, nh, k, m):
    pg, sg, gg, pu, su, gu = _weights(fmt, nh, k, 1)
    pc, ps = fp4.fp4_prepare_gate_up_interleaved(u8(pg), u8(sg), u8(pu), u8(su), nh, k, fmt)
    xbits = synth.activations(synth.TINY, m, k)
    info = fp4.fp4_dispatch_info()
    y = fp4.fp4_w4a16_gate_up_swiglu(x_dev(xbits), pc, ps, nh, float(gg), float(gu), fmt, info=info)
    assert info.kernel == (0 if m < 3 else 2 if m <= 16 else 1)
    ref = oracle.gate_up_swiglu(oracle.bf16_bits_to_f32(xbits), pg, sg, pu, su, k, fmt, gg, gu)
    assert_close(y_host(y), ref, "swiglu fmt=%d nh=%d k=%d m=%d" % (fmt, nh, k, m))


@pytest.mark.parametrize("fmt,nh,k,m", [(MX, 12288, 2560, 130), (NV, 12288, 2560, 200)])
def test_swiglu_two_way_tail_runs_whole(fmt, nh, k, m):
    # 192 tiles of 128 x 256 past no full round: a tail that would split only
    # two ways along K runs as whole tiles (no workspace); at m = 130 most of
    # the lower row of tiles is past m.
    assert fp4.fp4_swiglu_workspace_bytes(m, nh, k, fmt) == 0
    test_swiglu_matches_oracle(fmt, nh, k, m)


@pytest.mark.parametrize("fmt,nh,k,m", [(NV, 300, 5120, 8), (MX, 640, 17408, 1), (NV, 512, 5120, 40)])
def test_swiglu_deterministic_and_workspace_poison(fmt, nh, k, m):
    pg, sg, gg, pu, su, gu = _weights(fmt, nh, k, 2)
    pc, ps = fp4.fp4_prepare_gate_up_interleaved(u8(pg), u8(sg), u8(pu), u8(su), nh, k, fmt)
    xd = x_dev(synth.activations(synth.TINY, m, k))
    need = fp4.fp4_swiglu_workspace_bytes(m, nh, k, fmt)
    outs = []
    for fill in (0x00, 0xFF, 0x7F):
        ws = torch.full((max(need, 16),), fill, dtype=torch.uint8, device=DEV)
        outs.append(y_host_bits(fp4.fp4_w4a16_gate_up_swiglu(xd, pc, ps, nh, float(gg), float(gu), fmt,
                                                             workspace=ws)))
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
