"""RED checks of the parity comparisons: each comparison that passes against
the oracle must fail against a mutated oracle.

For every family of parity test (the VALU GEMV, the MFMA decode with and
without a K split, the wave-split MFMA decode, the tile GEMM whole and with split tail tiles, the fused
gate_up, the greedy argmax, the grouped MoE and the SwiGLU gate_up), the GPU
result is first checked green against the oracle with the layer's tolerance,
then the same comparison is run against the oracle evaluated on mutated
inputs -- nibbles of each code byte swapped, the NVFP4 global scale dropped,
the block-scale index shifted by one group, the weight rows shifted by one,
the activation rows reversed, gate and up swapped -- and must flag a large
share of the outputs.  Nothing is mutated on the GPU: the kernels always run
on the real inputs; only the oracle's inputs change, on the host.
"""

import numpy as np
import pytest
import torch

import fp4_weight_only_e2m1_amd as fp4
import oracle
import synth
from gpu_util import DEV, tolerance_violations, u8, x_dev, y_host, y_host_bits

pytestmark = pytest.mark.gpu

NV, MX = fp4.FMT_NVFP4, fp4.FMT_MXFP4
RED_SHARE = 0.25   # a mutation must push at least this share of outputs out of tolerance


def swap_nibbles(packed):
    return ((packed & 0x0F) << 4 | (packed >> 4)).astype(np.uint8)


def shift_scale_groups(scales):
    return np.roll(scales, 1, axis=1)


def shift_rows(a):
    return np.roll(a, 1, axis=0)


def mutations(fmt, packed, scales, g, x):
    """(name, packed, scales, G, x) of the mutated oracle inputs."""
    out = [("nibbles swapped", swap_nibbles(packed), scales, g, x),
           ("scale index shifted one group", packed, shift_scale_groups(scales), g, x),
           ("weight rows shifted", shift_rows(packed), shift_rows(scales), g, x)]
    if fmt == NV:
        out.append(("global scale dropped", packed, scales, np.float32(1.0), x))
    if x.shape[0] > 1:
        out.append(("activation rows reversed", packed, scales, g, x[::-1].copy()))
    return out


def assert_green_then_red(y, ref, reds, what):
    bad, _ = tolerance_violations(y, ref)
    assert not bad.any(), "%s: %d outputs outside tolerance against the oracle" % (what, int(bad.sum()))
    for name, mref in reds:
        bad, _ = tolerance_violations(y, mref)
        share = float(bad.mean())
        assert share >= RED_SHARE, "%s: the comparison did not catch '%s' (%.1f%% flagged)" % (what, name,
                                                                                             100 * share)


# (fmt, n, k, m, kernel, split): one case per kernel path.
LINEAR = [
    (NV, 8192, 1024, 1, 0, False),    # VALU GEMV
    (MX, 384, 8448, 2, 0, True),      # VALU GEMV, K split in three
    (NV, 640, 6144, 4, 6, False),     # wave-split MFMA decode
    (MX, 300, 1056, 8, 6, False),     # wave-split MFMA decode, ragged n and last stage
    (NV, 8192, 2048, 8, 2, False),    # MFMA decode (128 tiles: unsplit)
    (MX, 16896, 544, 4, 2, False),    # MFMA decode on 96-row tiles
    (NV, 256, 17408, 4, 2, True),     # MFMA decode, K split
    (MX, 640, 1024, 24, 2, False),    # MFMA decode, two activation groups
    (NV, 1024, 1024, 200, 1, False),  # tile GEMM
    (MX, 256, 5120, 100, 1, True),    # tile GEMM, split tail tile
]


@pytest.mark.parametrize("fmt,n,k,m,kernel,split", LINEAR)
def test_red_linear(fmt, n, k, m, kernel, split):
    packed, scales, g = synth.packed_weight(synth.TINY, 70, n, k, fmt)
    xbits = synth.activations(synth.TINY, m, k)
    x = oracle.bf16_bits_to_f32(xbits)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    info = fp4.fp4_dispatch_info()
    y = y_host(fp4.fp4_w4a16_linear(x_dev(xbits), pc, ps, n, float(g), fmt, info=info))
    assert info.kernel == kernel and (info.splits > 1) == split, info.as_dict()
    ref = oracle.linear(x, packed, scales, k, fmt, g)
    reds = [(name, oracle.linear(xm, pm, sm, k, fmt, gm)) for name, pm, sm, gm, xm in mutations(fmt, packed, scales, g, x)]
    assert_green_then_red(y, ref, reds, "linear fmt=%d n=%d k=%d m=%d" % (fmt, n, k, m))


@pytest.mark.parametrize("fmt,m", [(NV, 4), (MX, 1), (NV, 64)])
def test_red_gate_up(fmt, m):
    nh, k = 512, 2048
    pg, sg, gg = synth.packed_weight(synth.TINY, 71, nh, k, fmt)
    pu, su, gu = synth.packed_weight(synth.TINY, 72, nh, k, fmt)
    xbits = synth.activations(synth.TINY, m, k)
    x = oracle.bf16_bits_to_f32(xbits)
    pc, ps = fp4.fp4_prepare_gate_up(u8(pg), u8(sg), u8(pu), u8(su), nh, k, fmt)
    y = y_host(fp4.fp4_w4a16_gate_up(x_dev(xbits), pc, ps, nh, float(gg), float(gu), fmt))
    ref = oracle.gate_up(x, pg, sg, pu, su, k, fmt, gg, gu)
    reds = [("gate and up swapped", oracle.gate_up(x, pu, su, pg, sg, k, fmt, gu, gg)),
            ("nibbles swapped", oracle.gate_up(x, swap_nibbles(pg), sg, swap_nibbles(pu), su, k, fmt, gg, gu)),
            ("scale index shifted one group", oracle.gate_up(x, pg, shift_scale_groups(sg), pu, shift_scale_groups(su),
                                                             k, fmt, gg, gu))]
    if fmt == NV:
        reds.append(("global scales dropped", oracle.gate_up(x, pg, sg, pu, su, k, fmt, 1.0, 1.0)))
    assert_green_then_red(y, ref, reds, "gate_up fmt=%d m=%d" % (fmt, m))


def test_red_swiglu():
    fmt, nh, k, m = NV, 512, 2048, 4
    pg, sg, gg = synth.packed_weight(synth.TINY, 73, nh, k, fmt)
    pu, su, gu = synth.packed_weight(synth.TINY, 74, nh, k, fmt)
    xbits = synth.activations(synth.TINY, m, k)
    x = oracle.bf16_bits_to_f32(xbits)
    pc, ps = fp4.fp4_prepare_gate_up_interleaved(u8(pg), u8(sg), u8(pu), u8(su), nh, k, fmt)
    y = y_host(fp4.fp4_w4a16_gate_up_swiglu(x_dev(xbits), pc, ps, nh, float(gg), float(gu), fmt))
    ref = oracle.gate_up_swiglu(x, pg, sg, pu, su, k, fmt, gg, gu)
    reds = [("gate and up swapped", oracle.gate_up_swiglu(x, pu, su, pg, sg, k, fmt, gu, gg)),
            ("nibbles swapped", oracle.gate_up_swiglu(x, swap_nibbles(pg), sg, swap_nibbles(pu), su, k, fmt, gg, gu))]
    assert_green_then_red(y, ref, reds, "swiglu")


def test_red_argmax():
    # The greedy token must differ from the argmax of mutated logits.
    fmt, n, k, m = NV, 4096, 2048, 8
    packed, scales, g = synth.packed_weight(synth.TINY, 75, n, k, fmt)
    xbits = synth.activations(synth.TINY, m, k)
    x = oracle.bf16_bits_to_f32(xbits)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    idx, _, _ = fp4.fp4_w4a16_linear_argmax(x_dev(xbits), pc, ps, n, float(g), fmt)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    ref = oracle.linear(x, packed, scales, k, fmt, g)
    # Green: the chosen logit is the oracle's maximum within tolerance.
    bound = 2.0 ** -7 * np.abs(ref.max(axis=1)) + 1e-3 * np.sqrt(np.mean(ref ** 2))
    assert np.all(ref.max(axis=1) - ref[np.arange(m), got] <= bound)
    for name, pm, sm, gm, xm in mutations(fmt, packed, scales, g, x):
        mref = oracle.linear(xm, pm, sm, k, fmt, gm)
        if name == "global scale dropped":
            continue  # a positive global scale does not move the argmax
        miss = mref.max(axis=1) - mref[np.arange(m), got] > 2.0 ** -7 * np.abs(mref.max(axis=1)) + \
            1e-3 * np.sqrt(np.mean(mref ** 2))
        assert miss.mean() >= 0.5, "argmax: the check did not catch '%s'" % name


def test_red_moe():
    # Grouped MoE decode: pairs computed with the wrong expert's weight, or
    # with their tokens permuted, must be flagged.
    fmt, n, k, experts, tokens, topk = NV, 256, 1024, 8, 4, 2
    ws = [synth.packed_weight(synth.TINY, 80 + e, n, k, fmt) for e in range(experts)]
    rng = np.random.default_rng(3)
    pairs = sorted((int(e), t) for t in range(tokens) for e in rng.choice(experts, size=topk, replace=False))
    offsets = np.searchsorted([p[0] for p in pairs], np.arange(experts + 1)).astype(np.int32)
    ptok = np.array([p[1] for p in pairs], dtype=np.int32)
    xbits = synth.activations(synth.TINY, tokens, k)
    x = oracle.bf16_bits_to_f32(xbits)
    pc = torch.cat([fp4.fp4_prepare(u8(p), u8(s), n, k, fmt)[0] for p, s, _ in ws])
    ps = torch.cat([fp4.fp4_prepare(u8(p), u8(s), n, k, fmt)[1] for p, s, _ in ws])
    gs = torch.tensor([float(g) for _, _, g in ws], dtype=torch.float32, device=DEV)
    y = y_host(fp4.fp4_w4a16_moe_decode(x_dev(xbits), pc, ps, n, experts, gs, fmt,
                                        torch.from_numpy(offsets).to(DEV), torch.from_numpy(ptok).to(DEV)))
    ref = oracle.moe_decode(x, ws, k, fmt, offsets, ptok)
    wrong_expert = oracle.moe_decode(x, ws[1:] + ws[:1], k, fmt, offsets, ptok)
    perm_tokens = oracle.moe_decode(x, ws, k, fmt, offsets, (ptok + 1) % tokens)
    assert_green_then_red(y, ref, [("wrong expert weights", wrong_expert), ("tokens permuted", perm_tokens)], "moe")
