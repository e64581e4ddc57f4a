"""GPU parity of the grouped MoE decode (fp4_w4a16_moe_decode) against the
oracle's per-pair reference: random top-k routings over several experts
(empty experts, an expert with more than 8 pairs), pair independence bit for
bit, and routing tables that point outside the buffers."""

import numpy as np
import pytest
import torch

import fp4_weight_only_e2m1_amd as fp4
import oracle
import synth
from gpu_util import DEV, assert_close, u8, x_dev, y_host, y_host_bits

pytestmark = pytest.mark.gpu

NV, MX = fp4.FMT_NVFP4, fp4.FMT_MXFP4


def _stacked(experts, n, k, fmt, seed):
    host, codes, scales = [], [], []
    for e in range(experts):
        packed, sc, g = synth.packed_weight(synth.TINY, 100 + seed + e, n, k, fmt)
        pc, ps = fp4.fp4_prepare(u8(packed), u8(sc), n, k, fmt)
        host.append((packed, sc, g))
        codes.append(pc)
        scales.append(ps)
    gs = torch.tensor([float(h[2]) for h in host], dtype=torch.float32, device=DEV)
    return host, torch.cat(codes), torch.cat(scales), gs


def _routing(tokens, experts, topk, seed):
    """Top-k distinct experts per token, pairs sorted by expert (then token)."""
    rng = np.random.default_rng(seed)
    pairs = sorted((int(e), t) for t in range(tokens) for e in rng.choice(experts, size=topk, replace=False))
    offsets = np.searchsorted([p[0] for p in pairs], np.arange(experts + 1)).astype(np.int32)
    return offsets, np.array([p[1] for p in pairs], dtype=np.int32)


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def _moe_tile_rows(tokens, n, k):
    # The experts of one or two tokens run on the wave-split kernel (16-row tiles)
    # where it takes them (fewer than 128 64-row tiles, at most 32 K stages of
    # 256); otherwise 64-row tiles.
    small = -(-n // 256) * 256 // 64 < 128 and -(-k // 256) <= 32
    return 16 if tokens <= 2 and small else 64


@pytest.mark.parametrize("fmt,n,k", [(NV, 768, 2048), (MX, 300, 1056), (NV, 520, 4096), (MX, 1024, 512),
                                     (MX, 300, 8448)])
@pytest.mark.parametrize("tokens,experts,topk", [(1, 16, 4), (2, 16, 4), (4, 16, 4), (8, 32, 8), (8, 4, 3)])
def test_moe_decode_matches_oracle(fmt, n, k, tokens, experts, topk):
    host, pc, ps, gs = _stacked(experts, n, k, fmt, 0)
    offsets, ptok = _routing(tokens, experts, topk, seed=tokens * 100 + experts)
    xbits = synth.activations(synth.TINY, tokens, k)
    info = fp4.fp4_dispatch_info()
    y = fp4.fp4_w4a16_moe_decode(x_dev(xbits), pc, ps, n, experts, gs if fmt == NV else None, fmt,
                                 _i32(offsets), _i32(ptok), info=info)
    # One expert slot per expert that can have pairs: min(experts, pairs).
    assert info.kernel == 3 and info.grid_y == min(experts, tokens * topk)
    assert info.grid_x == -(-n // 256) * 256 // _moe_tile_rows(tokens, n, k)
    y_ref = oracle.moe_decode(oracle.bf16_bits_to_f32(xbits), host, k, fmt, offsets, ptok)
    assert_close(y_host(y), y_ref, "moe fmt=%d n=%d k=%d T=%d E=%d" % (fmt, n, k, tokens, experts))


@pytest.mark.parametrize("fmt,tokens,experts,topk", [(NV, 1, 128, 8), (MX, 2, 100, 8), (NV, 3, 70, 5)])
def test_moe_many_experts(fmt, tokens, experts, topk):
    # More experts than one wave scans at once (64): the slot -> expert search
    # crosses chunks, and most experts have no pairs.
    n, k = 256, 512
    host, pc, ps, gs = _stacked(experts, n, k, fmt, 3)
    offsets, ptok = _routing(tokens, experts, topk, seed=experts + tokens)
    xbits = synth.activations(synth.TINY, tokens, k)
    info = fp4.fp4_dispatch_info()
    y = fp4.fp4_w4a16_moe_decode(x_dev(xbits), pc, ps, n, experts, gs if fmt == NV else None, fmt,
                                 _i32(offsets), _i32(ptok), info=info)
    assert info.grid_y == tokens * topk
    y_ref = oracle.moe_decode(oracle.bf16_bits_to_f32(xbits), host, k, fmt, offsets, ptok)
    assert_close(y_host(y), y_ref, "moe many experts E=%d" % experts)


@pytest.mark.parametrize("fmt,n,k,experts,topk,tokens", [(NV, 1536, 2048, 24, 8, 1), (MX, 300, 1056, 16, 5, 1),
                                                          (NV, 1536, 2048, 24, 8, 2), (MX, 300, 1056, 6, 5, 2)])
def test_moe_decode_few_tokens_equals_linear_per_expert(fmt, n, k, experts, topk, tokens):
    # One or two tokens: each expert's pairs run on the wave-split kernel as
    # the fp4_w4a16_linear call on its expert's weight and those tokens does,
    # bit for bit.
    host, pc, ps, gs = _stacked(experts, n, k, fmt, 21)
    offsets, ptok = _routing(tokens, experts, topk, seed=77)
    xbits = synth.activations(synth.TINY, tokens, k)
    xd = x_dev(xbits)
    info = fp4.fp4_dispatch_info()
    y = y_host_bits(fp4.fp4_w4a16_moe_decode(xd, pc, ps, n, experts, gs if fmt == NV else None, fmt, _i32(offsets),
                                             _i32(ptok), info=info))
    assert info.kernel == 3 and info.grid_x == -(-n // 256) * 256 // 16
    cb, sb = fp4.fp4_prepared_bytes(n, k, fmt)
    for e in range(experts):
        toks = ptok[offsets[e]:offsets[e + 1]]
        if len(toks) == 0:
            continue
        ye = y_host_bits(fp4.fp4_w4a16_linear(x_dev(xbits[toks]), pc[e * cb:(e + 1) * cb], ps[e * sb:(e + 1) * sb], n,
                                              float(host[e][2]), fmt))
        assert np.array_equal(y[offsets[e]:offsets[e + 1]], ye), e
    y_ref = oracle.moe_decode(oracle.bf16_bits_to_f32(xbits), host, k, fmt, offsets, ptok)
    assert_close(oracle.bf16_bits_to_f32(y).astype(np.float64), y_ref, "moe few tokens")


def test_moe_pairs_independent_and_long_expert():
    # 12 tokens all routed to expert 2 (two passes of 8 and 4), plus others;
    # dropping pairs leaves every remaining pair's output bit for bit.
    fmt, n, k, experts, tokens = NV, 640, 2048, 5, 12
    host, pc, ps, gs = _stacked(experts, n, k, fmt, 7)
    xbits = synth.activations(synth.TINY, tokens, k)
    xd = x_dev(xbits)
    full = [(0, 3), (0, 7)] + [(2, t) for t in range(tokens)] + [(4, 1), (4, 5), (4, 11)]
    sub = [p for i, p in enumerate(full) if i % 3 != 1]

    def run(pairs):
        e_of = np.array([p[0] for p in pairs])
        offsets = np.searchsorted(e_of, np.arange(experts + 1)).astype(np.int32)
        ptok = np.array([p[1] for p in pairs], dtype=np.int32)
        y = y_host_bits(fp4.fp4_w4a16_moe_decode(xd, pc, ps, n, experts, gs, fmt, _i32(offsets), _i32(ptok)))
        return offsets, ptok, y

    off, ptok, y_full = run(full)
    _, _, y_sub = run(sub)
    rows = {p: i for i, p in enumerate(full)}
    for j, p in enumerate(sub):
        assert np.array_equal(y_sub[j], y_full[rows[p]]), p
    y_ref = oracle.moe_decode(oracle.bf16_bits_to_f32(xbits), host, k, fmt, off, ptok)
    assert_close(oracle.bf16_bits_to_f32(y_full).astype(np.float64), y_ref, "moe long expert")


def test_moe_out_of_range_routing_is_contained():
    # Offsets beyond the pair count are clamped; token ids outside x read zero
    # rows (their outputs are exactly zero); nothing else is touched.
    fmt, n, k, experts, tokens = MX, 256, 1024, 3, 2
    host, pc, ps, _ = _stacked(experts, n, k, fmt, 9)
    xbits = synth.activations(synth.TINY, tokens, k)
    offsets = np.array([0, 2, 9, 1 << 30], dtype=np.int32)
    ptok = np.array([0, -5, 1, 7], dtype=np.int32)
    y = torch.full((4, n), 3.0, dtype=torch.bfloat16, device=DEV)
    fp4.fp4_w4a16_moe_decode(x_dev(xbits), pc, ps, n, experts, None, fmt, _i32(offsets), _i32(ptok), y=y)
    got = y_host(y)
    assert np.isfinite(got).all()
    assert (got[1] == 0).all() and (got[3] == 0).all()
    ref = oracle.moe_decode(oracle.bf16_bits_to_f32(xbits), host, k, fmt, [0, 2, 4, 4], [0, 0, 1, 0])
    assert_close(got[[0, 2]], ref[[0, 2]], "moe clamped")


@pytest.mark.parametrize("fmt", [NV, MX])
def test_moe_bad_token_ids_on_64_row_tiles(fmt):
    # Five tokens (the 64-row tile route): pairs whose token id lies outside
    # x give exactly zero outputs, one expert mixing good and bad pairs in a
    # pass; the good pairs match the oracle, and each equals bit for bit the
    # dense call on its expert's weight at m = 9 (the unsplit 64-row MFMA
    # decode, the route's summation order; the dense call takes the
    # wave-split kernel at m <= 8 on this layer).
    n, k, experts, tokens = 320, 1056, 3, 5
    host, pc, ps, gs = _stacked(experts, n, k, fmt, 13)
    xbits = synth.activations(synth.TINY, tokens, k)
    offsets = np.array([0, 3, 7, 9], dtype=np.int32)
    ptok = np.array([4, -1, 0, 2, 5, 1, 1 << 20, 3, -7], dtype=np.int32)
    good = [0, 2, 3, 5, 7]
    info = fp4.fp4_dispatch_info()
    y = fp4.fp4_w4a16_moe_decode(x_dev(xbits), pc, ps, n, experts, gs if fmt == NV else None, fmt, _i32(offsets),
                                 _i32(ptok), info=info)
    assert info.kernel == 3 and info.grid_x == 512 // 64, info.as_dict()
    bits = y_host_bits(y)
    for p in (1, 4, 6, 8):
        assert (bits[p] & 0x7FFF == 0).all(), p
    ref = oracle.moe_decode(oracle.bf16_bits_to_f32(xbits), host, k, fmt, offsets, np.where(
        (ptok >= 0) & (ptok < tokens), ptok, 0))
    assert_close(oracle.bf16_bits_to_f32(bits[good]).astype(np.float64), ref[good], "moe bad tokens")
    for p in good:
        e = int(np.searchsorted(offsets, p, side="right") - 1)
        x9 = np.repeat(xbits[ptok[p]:ptok[p] + 1], 9, axis=0)
        dinfo = fp4.fp4_dispatch_info()
        w = fp4.fp4_w4a16_linear(x_dev(x9), pc[e * pc.numel() // experts:], ps[e * ps.numel() // experts:], n,
                                 float(host[e][2]), fmt, info=dinfo)
        assert (dinfo.kernel, dinfo.splits, dinfo.grid_x) == (2, 1, 512 // 64), dinfo.as_dict()
        assert np.array_equal(y_host_bits(w)[0], bits[p]), p


def test_moe_no_pairs_is_a_no_op():
    fmt, n, k = NV, 256, 512
    _, pc, ps, gs = _stacked(2, n, k, fmt, 11)
    y = fp4.fp4_w4a16_moe_decode(x_dev(synth.activations(synth.TINY, 1, k)), pc, ps, n, 2, gs, fmt,
                                 _i32([0, 0, 0]), torch.empty(0, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert y.shape == (0, n)


# ---- grouped MoE on the tile GEMM (fp4_w4a16_moe_prefill) ----

def _oracle_moe(xbits, host, k, fmt, offsets, ptok):
    """oracle.linear per expert over its pairs' x rows (the layer is row-wise,
    so this is oracle.moe_decode's result, one weight dequantization per expert)."""
    x = oracle.bf16_bits_to_f32(xbits)
    n = host[0][0].shape[0]
    y = np.zeros((len(ptok), n), dtype=np.float64)
    for e, (packed, sc, g) in enumerate(host):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 > p0:
            y[p0:p1] = oracle.linear(x[ptok[p0:p1]], packed, sc, k, fmt, g)
    return y


def _slots(pairs, experts, n):
    return (-(-pairs // 128) + min(experts, pairs)) * (-(-n // 256))


def _offsets_from_counts(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


@pytest.mark.parametrize("fmt,n,k,tokens,experts,topk", [
    (NV, 768, 2048, 200, 8, 2),      # ~50 pairs per expert
    (MX, 300, 1056, 150, 6, 3),      # ragged n and k, ~75 per expert
    (NV, 520, 4096, 64, 16, 8),      # 32 per expert
    (MX, 1024, 512, 40, 100, 8),     # 100 experts: the tile search crosses 64-expert chunks
    (NV, 256, 512, 700, 4, 1),       # ~175 per expert: two tiles per expert
])
def test_moe_prefill_matches_oracle(fmt, n, k, tokens, experts, topk):
    host, pc, ps, gs = _stacked(experts, n, k, fmt, 20)
    offsets, ptok = _routing(tokens, experts, topk, seed=7 * tokens + experts)
    xbits = synth.activations(synth.TINY, tokens, k)
    info = fp4.fp4_dispatch_info()
    y = fp4.fp4_w4a16_moe_prefill(x_dev(xbits), pc, ps, n, experts, gs if fmt == NV else None, fmt,
                                  _i32(offsets), _i32(ptok), info=info)
    assert info.kernel == 5 and info.grid_x == _slots(len(ptok), experts, n) and info.block == 256
    assert_close(y_host(y), _oracle_moe(xbits, host, k, fmt, offsets, ptok),
                 "moe prefill fmt=%d n=%d k=%d T=%d E=%d" % (fmt, n, k, tokens, experts))


@pytest.mark.parametrize("fmt", [NV, MX])
def test_moe_prefill_tile_boundaries(fmt):
    # Expert pair counts at the 32 / 64 / 128-row boundaries of the tiles and
    # of their 1-, 2- and 4-block instances, with empty experts between.
    counts = [0, 1, 31, 32, 0, 33, 64, 65, 127, 128, 129, 0, 257]
    n, k, tokens = 256, 512, 97
    experts = len(counts)
    host, pc, ps, gs = _stacked(experts, n, k, fmt, 30)
    offsets = _offsets_from_counts(counts)
    ptok = np.random.default_rng(5).integers(0, tokens, size=int(offsets[-1])).astype(np.int32)
    xbits = synth.activations(synth.TINY, tokens, k)
    y = fp4.fp4_w4a16_moe_prefill(x_dev(xbits), pc, ps, n, experts, gs if fmt == NV else None, fmt,
                                  _i32(offsets), _i32(ptok))
    assert_close(y_host(y), _oracle_moe(xbits, host, k, fmt, offsets, ptok), "moe prefill boundaries")


def test_moe_prefill_equals_dense_linear_and_is_pair_independent():
    # Expert 1 gets all 300 tokens in order: its rows are the dense m = 300
    # call's (whole tiles, same MFMA order), bit for bit.  Dropping pairs
    # (300 -> 200 rows: other tile sizes and instances) leaves every
    # remaining pair's output bit for bit, and the decode route agrees within
    # the tolerance.
    fmt, n, k, experts, tokens = NV, 512, 1024, 3, 300
    host, pc, ps, gs = _stacked(experts, n, k, fmt, 40)
    xbits = synth.activations(synth.TINY, tokens, k)
    xd = x_dev(xbits)
    full = [(0, 5), (0, 17)] + [(1, t) for t in range(tokens)] + [(2, 0), (2, 299)]
    sub = [p for i, p in enumerate(full) if i % 3 != 2]

    def run(pairs, entry):
        e_of = np.array([p[0] for p in pairs])
        offsets = np.searchsorted(e_of, np.arange(experts + 1)).astype(np.int32)
        ptok = np.array([p[1] for p in pairs], dtype=np.int32)
        return offsets, ptok, y_host_bits(entry(xd, pc, ps, n, experts, gs, fmt, _i32(offsets), _i32(ptok)))

    off, ptok, y_full = run(full, fp4.fp4_w4a16_moe_prefill)
    cb, sb = fp4.fp4_prepared_bytes(n, k, fmt)
    dinfo = fp4.fp4_dispatch_info()
    dense = y_host_bits(fp4.fp4_w4a16_linear(xd, pc[cb:2 * cb], ps[sb:2 * sb], n, float(host[1][2]), fmt,
                                             info=dinfo))
    assert dinfo.kernel == 1 and dinfo.splits == 1  # every row over all of K (no K-split partials)
    assert np.array_equal(y_full[2:2 + tokens], dense)
    _, _, y_sub = run(sub, fp4.fp4_w4a16_moe_prefill)
    rows = {p: i for i, p in enumerate(full)}
    for j, p in enumerate(sub):
        assert np.array_equal(y_sub[j], y_full[rows[p]]), p
    _, _, y_dec = run(full, fp4.fp4_w4a16_moe_decode)
    y_ref = _oracle_moe(xbits, host, k, fmt, off, ptok)
    assert_close(oracle.bf16_bits_to_f32(y_full).astype(np.float64), y_ref, "moe prefill full")
    assert_close(oracle.bf16_bits_to_f32(y_dec).astype(np.float64), y_ref, "moe decode route, same routing")


def test_moe_prefill_out_of_range_routing_is_contained():
    fmt, n, k, experts, tokens = MX, 256, 1024, 3, 2
    host, pc, ps, _ = _stacked(experts, n, k, fmt, 9)
    xbits = synth.activations(synth.TINY, tokens, k)
    offsets = np.array([0, 2, 9, 1 << 30], dtype=np.int32)
    ptok = np.array([0, -5, 1, 7], dtype=np.int32)
    y = torch.full((4, n), 3.0, dtype=torch.bfloat16, device=DEV)
    fp4.fp4_w4a16_moe_prefill(x_dev(xbits), pc, ps, n, experts, None, fmt, _i32(offsets), _i32(ptok), y=y)
    got = y_host(y)
    assert np.isfinite(got).all()
    assert (got[1] == 0).all() and (got[3] == 0).all()
    ref = oracle.moe_decode(oracle.bf16_bits_to_f32(xbits), host, k, fmt, [0, 2, 4, 4], [0, 0, 1, 0])
    assert_close(got[[0, 2]], ref[[0, 2]], "moe prefill clamped")
    # Decreasing offsets: experts 1 and 2 get empty ranges after clamping,
    # and row 3, which no expert owns, is not written.
    offsets = np.array([0, 3, 2, 2], dtype=np.int32)
    ptok = np.array([0, 1, 0, 1], dtype=np.int32)
    y = torch.full((4, n), 3.0, dtype=torch.bfloat16, device=DEV)
    fp4.fp4_w4a16_moe_prefill(x_dev(xbits), pc, ps, n, experts, None, fmt, _i32(offsets), _i32(ptok), y=y)
    got = y_host(y)
    assert (got[3] == 3.0).all()
    ref = _oracle_moe(xbits, host, k, fmt, [0, 3, 3, 3], ptok[:3])
    assert_close(got[:3], ref, "moe prefill decreasing offsets")


def test_moe_prefill_no_pairs_is_a_no_op():
    fmt, n, k = NV, 256, 512
    _, pc, ps, gs = _stacked(2, n, k, fmt, 11)
    info = fp4.fp4_dispatch_info()
    y = fp4.fp4_w4a16_moe_prefill(x_dev(synth.activations(synth.TINY, 1, k)), pc, ps, n, 2, gs, fmt,
                                  _i32([0, 0, 0]), torch.empty(0, dtype=torch.int32, device=DEV), info=info)
    torch.cuda.synchronize()
    assert y.shape == (0, n) and info.kernel == 5 and info.grid_x == 0


# ---- grouped MoE tile route with the SwiGLU epilogue (fp4_w4a16_moe_prefill_swiglu) ----

def _stacked_swiglu(experts, nh, k, fmt, seed):
    host, codes, scales, gvals = [], [], [], []
    for e in range(experts):
        pg, sg, gg = synth.packed_weight(synth.TINY, 300 + seed + 2 * e, nh, k, fmt)
        pu, su, gu = synth.packed_weight(synth.TINY, 301 + seed + 2 * e, nh, k, fmt)
        pc, ps = fp4.fp4_prepare_gate_up_interleaved(u8(pg), u8(sg), u8(pu), u8(su), nh, k, fmt)
        host.append((pg, sg, gg, pu, su, gu))
        codes.append(pc)
        scales.append(ps)
        gvals += [float(gg), float(gu)]
    gs = torch.tensor(gvals, dtype=torch.float32, device=DEV)
    return host, torch.cat(codes), torch.cat(scales), gs


def _oracle_moe_swiglu(xbits, host, k, fmt, offsets, ptok):
    x = oracle.bf16_bits_to_f32(xbits)
    y = np.zeros((len(ptok), host[0][0].shape[0]), dtype=np.float64)
    for e, (pg, sg, gg, pu, su, gu) in enumerate(host):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 > p0:
            y[p0:p1] = oracle.gate_up_swiglu(x[ptok[p0:p1]], pg, sg, pu, su, k, fmt, gg, gu)
    return y


@pytest.mark.parametrize("fmt,nh,k,tokens,experts,topk", [
    (NV, 384, 2048, 160, 8, 2),      # ~40 pairs per expert
    (MX, 300, 1056, 150, 6, 3),      # ragged n_half and k
    (NV, 256, 512, 700, 4, 1),       # two tiles per expert
])
def test_moe_prefill_swiglu_matches_oracle(fmt, nh, k, tokens, experts, topk):
    host, pc, ps, gs = _stacked_swiglu(experts, nh, k, fmt, 0)
    offsets, ptok = _routing(tokens, experts, topk, seed=11 * tokens + experts)
    xbits = synth.activations(synth.TINY, tokens, k)
    info = fp4.fp4_dispatch_info()
    y = fp4.fp4_w4a16_moe_prefill_swiglu(x_dev(xbits), pc, ps, nh, experts, gs if fmt == NV else None, fmt,
                                         _i32(offsets), _i32(ptok), info=info)
    assert info.kernel == 5 and info.grid_x == _slots(len(ptok), experts, 2 * (-(-nh // 256) * 256))
    assert y.shape == (len(ptok), nh)
    assert_close(y_host(y), _oracle_moe_swiglu(xbits, host, k, fmt, offsets, ptok),
                 "moe swiglu fmt=%d nh=%d k=%d" % (fmt, nh, k))


def test_moe_prefill_swiglu_equals_dense_swiglu():
    # One expert with all 300 tokens in order: its rows are the dense SwiGLU
    # gate_up call's bit for bit (every row over all of K, same epilogue).
    fmt, nh, k, experts, tokens = NV, 256, 1024, 3, 300
    host, pc, ps, gs = _stacked_swiglu(experts, nh, k, fmt, 50)
    xbits = synth.activations(synth.TINY, tokens, k)
    xd = x_dev(xbits)
    pairs = [(0, 4)] + [(1, t) for t in range(tokens)] + [(2, 7), (2, 8)]
    e_of = np.array([p[0] for p in pairs])
    offsets = np.searchsorted(e_of, np.arange(experts + 1)).astype(np.int32)
    ptok = np.array([p[1] for p in pairs], dtype=np.int32)
    y = y_host_bits(fp4.fp4_w4a16_moe_prefill_swiglu(xd, pc, ps, nh, experts, gs, fmt, _i32(offsets), _i32(ptok)))
    cb, sb = fp4.fp4_prepared_bytes(nh, k, fmt)
    dinfo = fp4.fp4_dispatch_info()
    _, _, gg, _, _, gu = host[1]
    dense = y_host_bits(fp4.fp4_w4a16_gate_up_swiglu(xd, pc[2 * cb:4 * cb], ps[2 * sb:4 * sb], nh, float(gg),
                                                     float(gu), fmt, info=dinfo))
    assert dinfo.kernel == 1 and dinfo.splits == 1
    assert np.array_equal(y[1:1 + tokens], dense)
    assert_close(oracle.bf16_bits_to_f32(y).astype(np.float64),
                 _oracle_moe_swiglu(xbits, host, k, fmt, offsets, ptok), "moe swiglu vs dense")


def test_moe_prefill_graph_replay():
    # Serving loops replay captured calls: a graph of both MoE tile routes,
    # replayed with new activations written in place between replays, gives
    # the eager results bit for bit every time.
    fmt, n, k, experts, tokens = NV, 512, 1024, 6, 96
    host, pc, ps, gs = _stacked(experts, n, k, fmt, 60)
    shost, spc, sps, sgs = _stacked_swiglu(experts, 256, k, fmt, 70)
    offsets, ptok = _routing(tokens, experts, 2, seed=3)
    off_d, ptok_d = _i32(offsets), _i32(ptok)
    x = x_dev(synth.activations(synth.TINY, tokens, k))
    y = torch.empty((len(ptok), n), dtype=torch.bfloat16, device=DEV)
    ys = torch.empty((len(ptok), 256), dtype=torch.bfloat16, device=DEV)

    def step():
        fp4.fp4_w4a16_moe_prefill(x, pc, ps, n, experts, gs, fmt, off_d, ptok_d, y=y)
        fp4.fp4_w4a16_moe_prefill_swiglu(x, spc, sps, 256, experts, sgs, fmt, off_d, ptok_d, y=ys)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        xb = synth.activations(synth.TINY + 1 + r, tokens, k)
        x.copy_(x_dev(xb))
        step()
        want, wants = y_host_bits(y).copy(), y_host_bits(ys).copy()
        y.fill_(7.0)
        ys.fill_(7.0)
        g.replay()
        assert np.array_equal(y_host_bits(y), want), r
        assert np.array_equal(y_host_bits(ys), wants), r


@pytest.mark.parametrize("swiglu", [False, True])
def test_moe_prefill_bench_workload_sampled(swiglu):
    # The moe_prefill / moe_prefill_swiglu benchmark configuration: 128
    # experts of 1536 rows (or 768 + 768 gate_up pairs) over k = 2048, NVFP4,
    # 1024 tokens routed top-8 (8192 pairs), 8 distinct expert weights
    # repeated over the 128.  The oracle checks every pair of 6 experts.
    experts, topk, tokens, n, k, fmt, distinct = 128, 8, 1024, 1536, 2048, NV, 8
    host, codes, scales, gv = [], [], [], []
    for e in range(distinct):
        p, s, g = synth.packed_weight(synth.TINY, 500 + e, n, k, fmt)
        if swiglu:
            h = n // 2
            pc, ps = fp4.fp4_prepare_gate_up_interleaved(u8(p[:h]), u8(s[:h]), u8(p[h:]), u8(s[h:]), h, k, fmt)
        else:
            pc, ps = fp4.fp4_prepare(u8(p), u8(s), n, k, fmt)
        host.append((p, s, g))
        codes.append(pc)
        scales.append(ps)
        gv.append(float(g))
    idx = [e % distinct for e in range(experts)]
    pc_all, ps_all = torch.cat([codes[i] for i in idx]), torch.cat([scales[i] for i in idx])
    gs = torch.tensor([gv[i] for i in idx for _ in range(2 if swiglu else 1)], dtype=torch.float32, device=DEV)
    offsets, ptok = _routing(tokens, experts, topk, seed=77)
    xbits = synth.activations(synth.TINY, tokens, k)
    if swiglu:
        y = fp4.fp4_w4a16_moe_prefill_swiglu(x_dev(xbits), pc_all, ps_all, n // 2, experts, gs, fmt, _i32(offsets),
                                             _i32(ptok))
    else:
        y = fp4.fp4_w4a16_moe_prefill(x_dev(xbits), pc_all, ps_all, n, experts, gs, fmt, _i32(offsets), _i32(ptok))
    got = y_host(y)
    assert np.isfinite(got).all()
    x = oracle.bf16_bits_to_f32(xbits)
    for e in (0, 1, 37, 64, 101, 127):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        p, s, g = host[e % distinct]
        xs = x[ptok[p0:p1]]
        if swiglu:
            h = n // 2
            ref = oracle.gate_up_swiglu(xs, p[:h], s[:h], p[h:], s[h:], k, fmt, g, g)
        else:
            ref = oracle.linear(xs, p, s, k, fmt, g)
        assert_close(got[p0:p1], ref, "moe bench workload expert %d swiglu=%s" % (e, swiglu))
