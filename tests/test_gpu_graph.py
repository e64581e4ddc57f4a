"""HIP-graph replay of the layer: a captured call replayed several times, with
new activations written in place and eager calls on the same workspace in
between, must give every time the bytes an eager call gives for the same
inputs.  Covers the split-K finish of both 64-row-family decode kernels
(whose arrival flags carry a token fixed at capture time), the wave-split
decode and the prefill GEMM's tail reduce, next to an unsplit call."""

import numpy as np
import pytest
import torch

import fp4_weight_only_e2m1_amd as fp4
import synth
from gpu_util import DEV, u8, x_dev, y_host_bits

pytestmark = pytest.mark.gpu

NV, MX = fp4.FMT_NVFP4, fp4.FMT_MXFP4


@pytest.mark.parametrize("fmt,n,k,m,split", [
    (NV, 512, 17408, 1, True),    # VALU GEMV, K split 5 ways
    (NV, 300, 9216, 8, True),     # MFMA decode, K split
    (NV, 300, 5120, 8, False),    # wave-split MFMA decode
    (MX, 300, 5120, 24, True),    # MFMA decode, two 16-row activation groups, K split
    (MX, 8192, 1024, 4, False),   # MFMA decode, unsplit (128 row tiles)
    (MX, 16896, 1024, 8, False),  # MFMA decode on 96-row tiles
    (NV, 512, 5120, 100, True),   # prefill GEMM, tail tiles split along K
])
def test_graph_replay_matches_eager(fmt, n, k, m, split):
    packed, scales, g = synth.packed_weight(synth.TINY, 70, n, k, fmt)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    need = fp4.fp4_workspace_bytes(m, n, k, fmt)
    assert (need > 0) == split
    ws = torch.full((max(need, 16),), 0xA5, dtype=torch.uint8, device=DEV)
    x = x_dev(synth.activations(synth.TINY, m, k))
    y_graph = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    y_eager = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)

    def call(y):
        fp4.fp4_w4a16_linear(x, pc, ps, n, float(g), fmt, y=y, workspace=ws)

    call(y_graph)  # warm-up outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(y_graph)
    torch.cuda.synchronize()

    rng = np.random.default_rng(7)
    for rep in range(4):
        xb = (rng.standard_normal((m, k), dtype=np.float32)).astype(np.float32)
        bits = (xb.view(np.uint32) >> 16).astype(np.uint16)  # truncated to bf16: any bf16 input will do
        x.copy_(x_dev(bits))
        graph.replay()
        torch.cuda.synchronize()
        got = y_host_bits(y_graph)
        call(y_eager)  # eager call on the same workspace, new token
        want = y_host_bits(y_eager)
        assert np.array_equal(got, want), "replay %d differs from eager" % rep
        # An eager call between replays must not disturb the next replay.
        call(y_eager)
        torch.cuda.synchronize()


@pytest.mark.parametrize("fmt,n,k,m", [(NV, 9000, 5120, 2), (NV, 5000, 2048, 6)])
def test_graph_replay_argmax(fmt, n, k, m):
    # The greedy-argmax call (decode kernel epilogue + reduce launch; the VALU
    # GEMV with a K split, the wave-split MFMA decode) replayed from a graph
    # with new activations gives the eager call's token ids.
    packed, scales, g = synth.packed_weight(synth.TINY, 71, n, k, fmt)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    ws = torch.full((fp4.fp4_argmax_workspace_bytes(m, n, k, fmt),), 0xA5, dtype=torch.uint8, device=DEV)
    x = x_dev(synth.activations(synth.TINY, m, k))
    idx = torch.empty(m, dtype=torch.int32, device=DEV)
    val = torch.empty(m, dtype=torch.bfloat16, device=DEV)

    def call():
        fp4.fp4_w4a16_linear_argmax(x, pc, ps, n, float(g), fmt, idx=idx, val=val, workspace=ws)

    call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    for rep in range(4):
        xb = rng.standard_normal((m, k), dtype=np.float32)
        x.copy_(x_dev((xb.view(np.uint32) >> 16).astype(np.uint16)))
        graph.replay()
        torch.cuda.synchronize()
        got = idx.cpu().numpy().tolist()
        call()
        torch.cuda.synchronize()
        assert got == idx.cpu().numpy().tolist(), rep



def test_graph_replay_w4a4():
    # The W4A4 call (quantizer, tile GEMM with K-split tail tiles, reduce)
    # replayed from a graph with new activations gives the eager call's bytes.
    n, k, m = 5120, 5120, 300
    packed, scales, _ = synth.packed_weight(synth.TINY, 72, n, k, MX)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, MX)
    ws = torch.full((fp4.fp4_w4a4_workspace_bytes(m, n, k),), 0xA5, dtype=torch.uint8, device=DEV)
    x = x_dev(synth.activations(synth.TINY, m, k))
    y_graph = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    y_eager = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    info = fp4.fp4_dispatch_info()

    def call(y):
        fp4.fp4_w4a4_linear(x, pc, ps, n, y=y, workspace=ws, info=info)

    call(y_graph)
    torch.cuda.synchronize()
    assert info.kernel == 4 and info.splits > 1
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(y_graph)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    for rep in range(4):
        xb = rng.standard_normal((m, k), dtype=np.float32)
        x.copy_(x_dev((xb.view(np.uint32) >> 16).astype(np.uint16)))
        graph.replay()
        torch.cuda.synchronize()
        got = y_host_bits(y_graph)
        call(y_eager)
        want = y_host_bits(y_eager)
        assert np.array_equal(got, want), "replay %d differs from eager" % rep
        call(y_eager)
        torch.cuda.synchronize()


@pytest.mark.parametrize("n,k,m,split", [(5120, 9216, 4, True), (5120, 6144, 4, False), (512, 5120, 100, True)])
def test_graph_replay_w4a4_nvfp4(n, k, m, split):
    # The NVFP4 W4A4 call (quantizer into the workspace, then the W4A16 call on
    # it: the MFMA decode with a K split, the wave-split MFMA decode, or the
    # tile GEMM with split tail tiles and the reduce) replayed from a graph
    # with new activations gives the eager call's bytes, on a workspace that
    # starts poisoned.
    packed, scales, g = synth.packed_weight(synth.TINY, 73, n, k, NV)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, NV)
    ws = torch.full((fp4.fp4_w4a4_nvfp4_workspace_bytes(m, n, k),), 0xA5, dtype=torch.uint8, device=DEV)
    x = x_dev(synth.activations(synth.TINY, m, k))
    y_graph = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    y_eager = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    info = fp4.fp4_dispatch_info()

    def call(y):
        fp4.fp4_w4a4_nvfp4_linear(x, pc, ps, n, float(g), 0.004, y=y, workspace=ws, info=info)

    call(y_graph)
    torch.cuda.synchronize()
    assert (info.splits > 1) == split, info.as_dict()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(y_graph)
    torch.cuda.synchronize()
    rng = np.random.default_rng(10)
    for rep in range(4):
        xb = rng.standard_normal((m, k), dtype=np.float32)
        x.copy_(x_dev((xb.view(np.uint32) >> 16).astype(np.uint16)))
        graph.replay()
        torch.cuda.synchronize()
        got = y_host_bits(y_graph)
        call(y_eager)
        want = y_host_bits(y_eager)
        assert np.array_equal(got, want), "replay %d differs from eager" % rep
        call(y_eager)
        torch.cuda.synchronize()
