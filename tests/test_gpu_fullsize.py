"""GPU parity at the workloads' full sizes, through the same entry points and
launch configuration the benchmark times.  The oracle computes a sample of
output columns one by one (every activation row, a few hundred weight rows
spread over n, plus both ends); fused gate_up is also checked bit for bit
against the two separate launches at full size, and the SwiGLU gate_up on the
same weights at decode and prefill row counts."""

import numpy as np
import pytest

import fp4_weight_only_e2m1_amd as fp4
import oracle
import synth
from gpu_util import assert_close, prepared, sample_rows, u8, weight, x_dev, y_host, y_host_bits

pytestmark = pytest.mark.gpu

NV, MX = fp4.FMT_NVFP4, fp4.FMT_MXFP4

# name, workload, tensor, fmt, n, k, activation rows
CASES = [
    ("tiny_nvfp4", synth.TINY, 0, NV, 512, 256, [1]),
    ("lm_head", synth.LM_HEAD, 0, NV, 248320, 5120, [1, 8, 16, 32]),
    ("down_proj", synth.DECODE_27B, 0, NV, 5120, 17408, [1, 2, 4, 8, 16, 32]),
    ("o_proj", synth.DECODE_27B, 1, NV, 5120, 6144, [1, 2, 4, 8, 16]),
    ("prefill_nvfp4", synth.PREFILL, 0, NV, 17408, 5120, [256, 1024, 4096]),
    ("prefill_mxfp4", synth.PREFILL, 1, MX, 17408, 5120, [256, 1024, 4096]),
]


@pytest.mark.parametrize("name,workload,tensor,fmt,n,k,ms", CASES, ids=[c[0] for c in CASES])
def test_full_size_sampled(name, workload, tensor, fmt, n, k, ms):
    packed, scales, g = weight(workload, tensor, n, k, fmt)
    pc, ps, _ = prepared(workload, tensor, n, k, fmt)
    rows = sample_rows(n, 512 if n > 512 else n, seed=workload)
    for m in ms:
        xbits = synth.activations(workload, m, k)
        y = y_host(fp4.fp4_w4a16_linear(x_dev(xbits), pc, ps, n, float(g), fmt))
        y_ref = oracle.linear_rows(oracle.bf16_bits_to_f32(xbits), packed, scales, k, fmt, g, rows)
        assert np.isfinite(y).all()
        assert_close(y[:, rows], y_ref, "%s m=%d" % (name, m))


@pytest.mark.parametrize("m", [1, 2, 4, 8, 16, 32])
def test_gate_up_full_size(m):
    nh, k, fmt = 12288, 4096, MX
    pg, sg, gg = weight(synth.GATE_UP, 0, nh, k, fmt)
    pu, su, gu = weight(synth.GATE_UP, 1, nh, k, fmt)
    cg, cs, _ = prepared(synth.GATE_UP, 0, nh, k, fmt)
    uc, us, _ = prepared(synth.GATE_UP, 1, nh, k, fmt)
    import torch
    fc = torch.cat([cg, uc])
    fs = torch.cat([cs, us])
    xbits = synth.activations(synth.GATE_UP, m, k)
    xd = x_dev(xbits)
    y = y_host_bits(fp4.fp4_w4a16_gate_up(xd, fc, fs, nh, float(gg), float(gu), fmt))
    yg = y_host_bits(fp4.fp4_w4a16_linear(xd, cg, cs, nh, float(gg), fmt))
    yu = y_host_bits(fp4.fp4_w4a16_linear(xd, uc, us, nh, float(gu), fmt))
    assert np.array_equal(y[:, :nh], yg)
    assert np.array_equal(y[:, nh:], yu)
    rows = sample_rows(nh, 384, seed=m)
    x = oracle.bf16_bits_to_f32(xbits)
    yf = oracle.bf16_bits_to_f32(y).astype(np.float64)
    ref_g = oracle.linear_rows(x, pg, sg, k, fmt, gg, rows)
    ref_u = oracle.linear_rows(x, pu, su, k, fmt, gu, rows)
    assert_close(np.concatenate([yf[:, rows], yf[:, nh + rows]], axis=1),
                 np.concatenate([ref_g, ref_u], axis=1), "gate_up m=%d" % m)


@pytest.mark.parametrize("m", [1, 2, 4, 8, 16, 1024])
def test_swiglu_gate_up_full_size(m):
    # The SwiGLU gate_up on the benchmark's 2 x 12288 x 4096 MXFP4 weights,
    # through each kernel the benchmark times (GEMV, MFMA decode, tile GEMM):
    # sampled output columns against the oracle on the same weight rows (each
    # column depends only on its gate and up rows).
    nh, k, fmt = 12288, 4096, MX
    pg, sg, gg = weight(synth.GATE_UP, 0, nh, k, fmt)
    pu, su, gu = weight(synth.GATE_UP, 1, nh, k, fmt)
    pc, ps = fp4.fp4_prepare_gate_up_interleaved(u8(pg), u8(sg), u8(pu), u8(su), nh, k, fmt)
    xbits = synth.activations(synth.GATE_UP, m, k)
    info = fp4.fp4_dispatch_info()
    y = y_host(fp4.fp4_w4a16_gate_up_swiglu(x_dev(xbits), pc, ps, nh, float(gg), float(gu), fmt, info=info))
    assert info.kernel == (0 if m < 3 else 2 if m <= 16 else 1)
    rows = sample_rows(nh, 384, seed=100 + m)
    ref = oracle.gate_up_swiglu(oracle.bf16_bits_to_f32(xbits), pg[rows], sg[rows], pu[rows], su[rows], k, fmt,
                                gg, gu)
    assert np.isfinite(y).all()
    assert_close(y[:, rows], ref, "swiglu gate_up m=%d" % m)


@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_lm_head_argmax_full_size(m):
    # The fused greedy argmax over all 248320 logits equals the argmax of the
    # unfused call's logits (lowest index on ties), and the winner's oracle
    # value is within tolerance of the oracle's value at the unfused maximum.
    n, k, fmt = 248320, 5120, NV
    packed, scales, g = weight(synth.LM_HEAD, 0, n, k, fmt)
    pc, ps, _ = prepared(synth.LM_HEAD, 0, n, k, fmt)
    xbits = synth.activations(synth.LM_HEAD, m, k)
    xd = x_dev(xbits)
    ybits = y_host_bits(fp4.fp4_w4a16_linear(xd, pc, ps, n, float(g), fmt))
    idx, val, _ = fp4.fp4_w4a16_linear_argmax(xd, pc, ps, n, float(g), fmt)
    got = idx.cpu().numpy()
    want = oracle.greedy_argmax(oracle.bf16_bits_to_f32(ybits))
    assert got.tolist() == want.tolist()
    import torch
    assert val.view(torch.int16).cpu().numpy().view(np.uint16).tolist() == ybits[np.arange(m), got].tolist()
    # Oracle values at the winner and at a sample of other rows.
    rows = np.unique(np.concatenate([sample_rows(n, 512, seed=m), got]))
    y_ref = oracle.linear_rows(oracle.bf16_bits_to_f32(xbits), packed, scales, k, fmt, g, rows)
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    for i in range(m):
        at = y_ref[i, np.searchsorted(rows, got[i])]
        top = y_ref[i].max()
        assert at >= top - (2.0 ** -7 * abs(top) + 1e-3 * rms), i
