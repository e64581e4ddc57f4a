"""Python binding of libfp4w4a16: W4A16 FP4 weight-only linear layers on MI355X (gfx950).

Thin ctypes marshalling over the C ABI declared in include/fp4w4a16.h; every
function here has the name of the C entry point it calls.  PyTorch supplies
device memory and the current HIP stream; all computation happens in the
library's HIP kernels.  There is no fallback: if the library cannot be loaded,
or a call fails, an exception is raised.
"""

import ctypes
import os

import torch

FMT_NVFP4 = 0
FMT_MXFP4 = 1
GROUP = {FMT_NVFP4: 16, FMT_MXFP4: 32}

FP4_OK = 0

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4w4a16.so")


class Fp4Error(RuntimeError):
    """A libfp4w4a16 call returned an error status."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (fn, fp4_status_string(status), status))


class fp4_dispatch_info(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("splits", ctypes.c_int), ("grid_x", ctypes.c_int),
                ("grid_y", ctypes.c_int), ("block", ctypes.c_int), ("xcds", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_i = ctypes.c_int
_f = ctypes.c_float
_SIGNATURES = {
    "fp4_prepared_bytes": (_i, [_i, _i, _i, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    "fp4_prepare": (_i, [_vp, _vp, _i, _i, _i, _vp, _vp, _vp]),
    "fp4_prepare_gate_up": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp]),
    "fp4_workspace_bytes": (_i, [_i, _i, _i, _i, _i, ctypes.POINTER(_sz)]),
    "fp4_plan": (_i, [_i, _i, _i, _i, _i, _i, ctypes.POINTER(fp4_dispatch_info)]),
    "fp4_w4a16_linear": (_i, [_vp, _i, _i, _vp, _vp, _i, _f, _i, _vp, _vp, _sz, _vp,
                              ctypes.POINTER(fp4_dispatch_info)]),
    "fp4_w4a16_linear_noalloc": (_i, [_vp, _i, _i, _vp, _vp, _i, _f, _i, _vp, _vp,
                                      ctypes.POINTER(fp4_dispatch_info)]),
    "fp4_w4a16_gate_up": (_i, [_vp, _i, _i, _vp, _vp, _i, _f, _f, _i, _vp, _vp, _sz, _vp,
                               ctypes.POINTER(fp4_dispatch_info)]),
    "fp4_argmax_workspace_bytes": (_i, [_i, _i, _i, _i, ctypes.POINTER(_sz)]),
    "fp4_w4a16_linear_argmax": (_i, [_vp, _i, _i, _vp, _vp, _i, _f, _i, _vp, _vp, _vp, _vp, _sz, _vp,
                                     ctypes.POINTER(fp4_dispatch_info)]),
    "fp4_prepare_gate_up_interleaved": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp]),
    "fp4_swiglu_workspace_bytes": (_i, [_i, _i, _i, _i, ctypes.POINTER(_sz)]),
    "fp4_w4a16_gate_up_swiglu": (_i, [_vp, _i, _i, _vp, _vp, _i, _f, _f, _i, _vp, _vp, _sz, _vp,
                                      ctypes.POINTER(fp4_dispatch_info)]),
    "fp4_moe_workspace_bytes": (_i, [_i, _i, ctypes.POINTER(_sz)]),
    "fp4_w4a16_moe_decode": (_i, [_vp, _i, _i, _vp, _vp, _i, _i, _vp, _i, _vp, _vp, _i, _vp, _vp, _sz, _vp,
                                  ctypes.POINTER(fp4_dispatch_info)]),
    "fp4_w4a16_moe_prefill": (_i, [_vp, _i, _i, _vp, _vp, _i, _i, _vp, _i, _vp, _vp, _i, _vp, _vp, _sz, _vp,
                                   ctypes.POINTER(fp4_dispatch_info)]),
    "fp4_w4a16_moe_prefill_swiglu": (_i, [_vp, _i, _i, _vp, _vp, _i, _i, _vp, _i, _vp, _vp, _i, _vp, _vp,
                                          ctypes.POINTER(fp4_dispatch_info)]),
    "fp4_w4a4_act_bytes": (_i, [_i, _i, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    "fp4_quantize_act_mxfp4": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
    "fp4_w4a4_workspace_bytes": (_i, [_i, _i, _i, _i, ctypes.POINTER(_sz)]),
    "fp4_w4a4_linear": (_i, [_vp, _i, _i, _vp, _vp, _i, _i, _vp, _vp, _sz, _vp, ctypes.POINTER(fp4_dispatch_info)]),
    "fp4_w4a4_gate_up": (_i, [_vp, _i, _i, _vp, _vp, _i, _i, _vp, _vp, _sz, _vp, ctypes.POINTER(fp4_dispatch_info)]),
    "fp4_quantize_act_nvfp4": (_i, [_vp, _i, _i, _f, _vp, _vp, _vp]),
    "fp4_w4a4_nvfp4_workspace_bytes": (_i, [_i, _i, _i, _i, ctypes.POINTER(_sz)]),
    "fp4_w4a4_nvfp4_linear": (_i, [_vp, _i, _i, _vp, _vp, _i, _f, _f, _vp, _vp, _sz, _vp,
                                   ctypes.POINTER(fp4_dispatch_info)]),
    "fp4_w4a4_nvfp4_gate_up": (_i, [_vp, _i, _i, _vp, _vp, _i, _f, _f, _f, _vp, _vp, _sz, _vp,
                                    ctypes.POINTER(fp4_dispatch_info)]),
    "fp4_dequantize": (_i, [_vp, _vp, _i, _i, _f, _i, _vp, _vp]),
    "fp4_status_string": (ctypes.c_char_p, [_i]),
}

_lib = None


def load_library():
    """Load (building first only if no library exists) libfp4w4a16.so and declare its symbols."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def fp4_status_string(status):
    return load_library().fp4_status_string(int(status)).decode()


def _check(fn, status):
    if status != FP4_OK:
        raise Fp4Error(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor on the GPU" % (name, dtype))


def fp4_prepared_bytes(n, k, fmt):
    """(code_bytes, scale_bytes) of a prepared weight of n rows and k columns."""
    cb, sb = _sz(), _sz()
    _check("fp4_prepared_bytes", load_library().fp4_prepared_bytes(n, k, fmt, ctypes.byref(cb), ctypes.byref(sb)))
    return cb.value, sb.value


def fp4_workspace_bytes(m, n, k, fmt, projections=1):
    out = _sz()
    _check("fp4_workspace_bytes", load_library().fp4_workspace_bytes(m, n, k, fmt, projections, ctypes.byref(out)))
    return out.value


def fp4_plan(m, n, k, fmt, projections=1, cus=256):
    """The fp4_dispatch_info a W4A16 call would report on a device of `cus` compute units (host only)."""
    info = fp4_dispatch_info()
    _check("fp4_plan", load_library().fp4_plan(m, n, k, fmt, projections, cus, ctypes.byref(info)))
    return info


def fp4_prepare(codes, scales, n, k, fmt, prep_codes=None, prep_scales=None, stream=None):
    """Repack canonical codes uint8 [n, k/2] and scales uint8 [n, k/g] into the prepared layout."""
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    if codes.numel() != n * (k // 2) or scales.numel() != n * (k // GROUP[fmt]):
        raise ValueError("codes / scales do not have the canonical [n, k/2] / [n, k/g] sizes")
    cb, sb = fp4_prepared_bytes(n, k, fmt)
    if prep_codes is None:
        prep_codes = torch.empty(cb, dtype=torch.uint8, device=codes.device)
    if prep_scales is None:
        prep_scales = torch.empty(sb, dtype=torch.uint8, device=codes.device)
    _need(prep_codes, torch.uint8, "prep_codes")
    _need(prep_scales, torch.uint8, "prep_scales")
    if prep_codes.numel() < cb or prep_scales.numel() < sb:
        raise ValueError("prepared buffers too small")
    _check("fp4_prepare", load_library().fp4_prepare(_ptr(codes), _ptr(scales), n, k, fmt, _ptr(prep_codes),
                                                     _ptr(prep_scales), _stream(stream)))
    return prep_codes, prep_scales


def fp4_prepare_gate_up(gate_codes, gate_scales, up_codes, up_scales, n_half, k, fmt,
                        prep_codes=None, prep_scales=None, stream=None):
    """Prepare the fused [gate; up] weight (gate rows, then up rows)."""
    for t, nm in ((gate_codes, "gate_codes"), (gate_scales, "gate_scales"), (up_codes, "up_codes"),
                  (up_scales, "up_scales")):
        _need(t, torch.uint8, nm)
    if gate_codes.numel() != n_half * (k // 2) or up_codes.numel() != n_half * (k // 2):
        raise ValueError("gate / up codes do not have the canonical [n_half, k/2] size")
    if gate_scales.numel() != n_half * (k // GROUP[fmt]) or up_scales.numel() != n_half * (k // GROUP[fmt]):
        raise ValueError("gate / up scales do not have the canonical [n_half, k/g] size")
    cb, sb = fp4_prepared_bytes(n_half, k, fmt)
    if prep_codes is None:
        prep_codes = torch.empty(2 * cb, dtype=torch.uint8, device=gate_codes.device)
    if prep_scales is None:
        prep_scales = torch.empty(2 * sb, dtype=torch.uint8, device=gate_codes.device)
    _need(prep_codes, torch.uint8, "prep_codes")
    _need(prep_scales, torch.uint8, "prep_scales")
    if prep_codes.numel() < 2 * cb or prep_scales.numel() < 2 * sb:
        raise ValueError("prepared buffers too small")
    _check("fp4_prepare_gate_up", load_library().fp4_prepare_gate_up(
        _ptr(gate_codes), _ptr(gate_scales), _ptr(up_codes), _ptr(up_scales), n_half, k, fmt,
        _ptr(prep_codes), _ptr(prep_scales), _stream(stream)))
    return prep_codes, prep_scales


def _linear_common(x, n_out, workspace, ws_need, y):
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [m, k]")
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, n_out), dtype=torch.bfloat16, device=x.device)
    _need(y, torch.bfloat16, "y")
    if y.numel() != m * n_out:
        raise ValueError("y must hold m x n values")
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return m, y, workspace, ws_bytes


def fp4_w4a16_linear(x, prep_codes, prep_scales, n, global_scale, fmt, y=None, workspace=None,
                     stream=None, info=None):
    """y = x @ w.T for bf16 x [m, k] and a prepared FP4 weight of n rows; returns y bf16 [m, n].

    ``info``, if given, is an fp4_dispatch_info filled with the kernel choice.
    """
    _need(prep_codes, torch.uint8, "prep_codes")
    _need(prep_scales, torch.uint8, "prep_scales")
    k = x.shape[1]
    cb, sb = fp4_prepared_bytes(n, k, fmt)
    if prep_codes.numel() < cb or prep_scales.numel() < sb:
        raise ValueError("prepared buffers smaller than fp4_prepared_bytes(n, k, fmt)")
    m, y, workspace, ws_bytes = _linear_common(x, n, workspace, fp4_workspace_bytes(x.shape[0], n, k, fmt, 1), y)
    _check("fp4_w4a16_linear", load_library().fp4_w4a16_linear(
        _ptr(x), m, k, _ptr(prep_codes), _ptr(prep_scales), n, float(global_scale), fmt, _ptr(y),
        _ptr(workspace), ws_bytes, _stream(stream), None if info is None else ctypes.byref(info)))
    return y


def fp4_w4a16_linear_noalloc(x, prep_codes, prep_scales, n, global_scale, fmt, y, stream=None, info=None):
    """fp4_w4a16_linear with the library's own scratch as its workspace: the
    call allocates nothing, so y (bf16 [m, n]) must be given.  Calls that may
    overlap on one GPU share that scratch and race."""
    _need(x, torch.bfloat16, "x")
    _need(y, torch.bfloat16, "y")
    _need(prep_codes, torch.uint8, "prep_codes")
    _need(prep_scales, torch.uint8, "prep_scales")
    if x.dim() != 2 or y.numel() != x.shape[0] * n:
        raise ValueError("x must be [m, k] and y hold m x n values")
    k = x.shape[1]
    cb, sb = fp4_prepared_bytes(n, k, fmt)
    if prep_codes.numel() < cb or prep_scales.numel() < sb:
        raise ValueError("prepared buffers smaller than fp4_prepared_bytes(n, k, fmt)")
    _check("fp4_w4a16_linear_noalloc", load_library().fp4_w4a16_linear_noalloc(
        _ptr(x), x.shape[0], k, _ptr(prep_codes), _ptr(prep_scales), n, float(global_scale), fmt, _ptr(y),
        _stream(stream), None if info is None else ctypes.byref(info)))
    return y


def fp4_w4a16_gate_up(x, prep_codes, prep_scales, n_half, global_gate, global_up, fmt, y=None,
                      workspace=None, stream=None, info=None):
    """Fused gate_up: returns bf16 [m, 2*n_half] = [x @ gate.T | x @ up.T]."""
    _need(prep_codes, torch.uint8, "prep_codes")
    _need(prep_scales, torch.uint8, "prep_scales")
    k = x.shape[1]
    cb, sb = fp4_prepared_bytes(n_half, k, fmt)
    if prep_codes.numel() < 2 * cb or prep_scales.numel() < 2 * sb:
        raise ValueError("prepared buffers smaller than twice fp4_prepared_bytes(n_half, k, fmt)")
    m, y, workspace, ws_bytes = _linear_common(
        x, 2 * n_half, workspace, fp4_workspace_bytes(x.shape[0], n_half, k, fmt, 2), y)
    _check("fp4_w4a16_gate_up", load_library().fp4_w4a16_gate_up(
        _ptr(x), m, k, _ptr(prep_codes), _ptr(prep_scales), n_half, float(global_gate), float(global_up), fmt,
        _ptr(y), _ptr(workspace), ws_bytes, _stream(stream), None if info is None else ctypes.byref(info)))
    return y


def fp4_argmax_workspace_bytes(m, n, k, fmt):
    out = _sz()
    _check("fp4_argmax_workspace_bytes", load_library().fp4_argmax_workspace_bytes(m, n, k, fmt, ctypes.byref(out)))
    return out.value


def fp4_w4a16_linear_argmax(x, prep_codes, prep_scales, n, global_scale, fmt, logits=False, y=None,
                            idx=None, val=None, workspace=None, stream=None, info=None):
    """Greedy token per activation row of the decode logits x @ w.T (m <= 32).

    Returns (idx int32 [m], val bf16 [m], y) where val holds the winning logits
    and y is the bf16 [m, n] logits when ``logits`` is true (or ``y`` is given),
    else None.  Exact ties go to the lowest index.
    """
    _need(prep_codes, torch.uint8, "prep_codes")
    _need(prep_scales, torch.uint8, "prep_scales")
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [m, k]")
    m, k = x.shape
    cb, sb = fp4_prepared_bytes(n, k, fmt)
    if prep_codes.numel() < cb or prep_scales.numel() < sb:
        raise ValueError("prepared buffers smaller than fp4_prepared_bytes(n, k, fmt)")
    if y is None and logits:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    if y is not None:
        _need(y, torch.bfloat16, "y")
        if y.numel() != m * n:
            raise ValueError("y must hold m x n values")
    if idx is None:
        idx = torch.empty(m, dtype=torch.int32, device=x.device)
    if val is None:
        val = torch.empty(m, dtype=torch.bfloat16, device=x.device)
    _need(idx, torch.int32, "idx")
    _need(val, torch.bfloat16, "val")
    if idx.numel() != m or val.numel() != m:
        raise ValueError("idx and val must hold m values")
    need = fp4_argmax_workspace_bytes(m, n, k, fmt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("fp4_w4a16_linear_argmax", load_library().fp4_w4a16_linear_argmax(
        _ptr(x), m, k, _ptr(prep_codes), _ptr(prep_scales), n, float(global_scale), fmt, _ptr(y), _ptr(idx),
        _ptr(val), _ptr(workspace), ws_bytes, _stream(stream), None if info is None else ctypes.byref(info)))
    return idx, val, y


def fp4_prepare_gate_up_interleaved(gate_codes, gate_scales, up_codes, up_scales, n_half, k, fmt,
                                    prep_codes=None, prep_scales=None, stream=None):
    """Prepare a gate_up weight for fp4_w4a16_gate_up_swiglu (gate and up rows interleaved by 16)."""
    for t, nm in ((gate_codes, "gate_codes"), (gate_scales, "gate_scales"), (up_codes, "up_codes"),
                  (up_scales, "up_scales")):
        _need(t, torch.uint8, nm)
    if gate_codes.numel() != n_half * (k // 2) or up_codes.numel() != n_half * (k // 2):
        raise ValueError("gate / up codes do not have the canonical [n_half, k/2] size")
    if gate_scales.numel() != n_half * (k // GROUP[fmt]) or up_scales.numel() != n_half * (k // GROUP[fmt]):
        raise ValueError("gate / up scales do not have the canonical [n_half, k/g] size")
    cb, sb = fp4_prepared_bytes(n_half, k, fmt)
    if prep_codes is None:
        prep_codes = torch.empty(2 * cb, dtype=torch.uint8, device=gate_codes.device)
    if prep_scales is None:
        prep_scales = torch.empty(2 * sb, dtype=torch.uint8, device=gate_codes.device)
    _need(prep_codes, torch.uint8, "prep_codes")
    _need(prep_scales, torch.uint8, "prep_scales")
    if prep_codes.numel() < 2 * cb or prep_scales.numel() < 2 * sb:
        raise ValueError("prepared buffers too small")
    _check("fp4_prepare_gate_up_interleaved", load_library().fp4_prepare_gate_up_interleaved(
        _ptr(gate_codes), _ptr(gate_scales), _ptr(up_codes), _ptr(up_scales), n_half, k, fmt,
        _ptr(prep_codes), _ptr(prep_scales), _stream(stream)))
    return prep_codes, prep_scales


def fp4_swiglu_workspace_bytes(m, n_half, k, fmt):
    out = _sz()
    _check("fp4_swiglu_workspace_bytes", load_library().fp4_swiglu_workspace_bytes(m, n_half, k, fmt,
                                                                                   ctypes.byref(out)))
    return out.value


def fp4_w4a16_gate_up_swiglu(x, prep_codes, prep_scales, n_half, global_gate, global_up, fmt, y=None,
                             workspace=None, stream=None, info=None):
    """y bf16 [m, n_half] = silu(x @ gate.T) * (x @ up.T) over an interleaved prepared gate_up weight."""
    _need(prep_codes, torch.uint8, "prep_codes")
    _need(prep_scales, torch.uint8, "prep_scales")
    k = x.shape[1]
    cb, sb = fp4_prepared_bytes(n_half, k, fmt)
    if prep_codes.numel() < 2 * cb or prep_scales.numel() < 2 * sb:
        raise ValueError("prepared buffers smaller than twice fp4_prepared_bytes(n_half, k, fmt)")
    m, y, workspace, ws_bytes = _linear_common(x, n_half, workspace, fp4_swiglu_workspace_bytes(x.shape[0], n_half,
                                                                                              k, fmt), y)
    _check("fp4_w4a16_gate_up_swiglu", load_library().fp4_w4a16_gate_up_swiglu(
        _ptr(x), m, k, _ptr(prep_codes), _ptr(prep_scales), n_half, float(global_gate), float(global_up), fmt,
        _ptr(y), _ptr(workspace), ws_bytes, _stream(stream), None if info is None else ctypes.byref(info)))
    return y


def fp4_moe_workspace_bytes(pairs, k):
    out = _sz()
    _check("fp4_moe_workspace_bytes", load_library().fp4_moe_workspace_bytes(pairs, k, ctypes.byref(out)))
    return out.value


def fp4_w4a16_moe_decode(x, prep_codes, prep_scales, n, experts, global_scales, fmt, expert_offsets,
                         pair_tokens, y=None, workspace=None, stream=None, info=None):
    """Grouped MoE decode: y[p] = x[pair_tokens[p]] @ w_e.T for every routed pair p (sorted by expert,
    expert e owning pairs expert_offsets[e] .. expert_offsets[e + 1]).  prep_codes / prep_scales hold
    the experts' prepared weights stacked; global_scales is float32 [experts] (NVFP4) or None (MXFP4).
    Returns y bf16 [pairs, n]."""
    return _moe("fp4_w4a16_moe_decode", x, prep_codes, prep_scales, n, experts, global_scales, fmt,
                expert_offsets, pair_tokens, y, workspace, stream, info)


def fp4_w4a16_moe_prefill(x, prep_codes, prep_scales, n, experts, global_scales, fmt, expert_offsets,
                          pair_tokens, y=None, workspace=None, stream=None, info=None):
    """Grouped MoE on the tile GEMM, for routings that give experts many pairs: the same arguments and
    result as fp4_w4a16_moe_decode (no workspace needed)."""
    return _moe("fp4_w4a16_moe_prefill", x, prep_codes, prep_scales, n, experts, global_scales, fmt,
                expert_offsets, pair_tokens, y, workspace, stream, info)


def fp4_w4a16_moe_prefill_swiglu(x, prep_codes, prep_scales, n_half, experts, global_scales, fmt,
                                 expert_offsets, pair_tokens, y=None, stream=None, info=None):
    """Grouped MoE on the tile GEMM with the SwiGLU epilogue: every expert an interleaved gate_up
    weight (fp4_prepare_gate_up_interleaved), y[p] = silu(x[t] @ gate_e.T) * (x[t] @ up_e.T) for
    t = pair_tokens[p].  global_scales is float32 [experts, 2] (gate, up; NVFP4) or None (MXFP4).
    Returns y bf16 [pairs, n_half]."""
    _need(x, torch.bfloat16, "x")
    _need(prep_codes, torch.uint8, "prep_codes")
    _need(prep_scales, torch.uint8, "prep_scales")
    _need(expert_offsets, torch.int32, "expert_offsets")
    _need(pair_tokens, torch.int32, "pair_tokens")
    if global_scales is not None:
        _need(global_scales, torch.float32, "global_scales")
        if global_scales.numel() != 2 * experts:
            raise ValueError("global_scales must hold experts x 2 values (gate, up)")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [tokens, k]")
    tokens, k = x.shape
    pairs = pair_tokens.numel()
    cb, sb = fp4_prepared_bytes(n_half, k, fmt)
    if prep_codes.numel() < experts * 2 * cb or prep_scales.numel() < experts * 2 * sb:
        raise ValueError("stacked prepared buffers smaller than experts x 2 x fp4_prepared_bytes(n_half, k, fmt)")
    if expert_offsets.numel() != experts + 1:
        raise ValueError("expert_offsets must hold experts + 1 values")
    if y is None:
        y = torch.empty((pairs, n_half), dtype=torch.bfloat16, device=x.device)
    _need(y, torch.bfloat16, "y")
    if y.numel() != pairs * n_half:
        raise ValueError("y must hold pairs x n_half values")
    _check("fp4_w4a16_moe_prefill_swiglu", load_library().fp4_w4a16_moe_prefill_swiglu(
        _ptr(x), tokens, k, _ptr(prep_codes), _ptr(prep_scales), n_half, experts, _ptr(global_scales), fmt,
        _ptr(expert_offsets), _ptr(pair_tokens), pairs, _ptr(y), _stream(stream),
        None if info is None else ctypes.byref(info)))
    return y


def _moe(name, x, prep_codes, prep_scales, n, experts, global_scales, fmt, expert_offsets, pair_tokens,
         y, workspace, stream, info):
    _need(x, torch.bfloat16, "x")
    _need(prep_codes, torch.uint8, "prep_codes")
    _need(prep_scales, torch.uint8, "prep_scales")
    _need(expert_offsets, torch.int32, "expert_offsets")
    _need(pair_tokens, torch.int32, "pair_tokens")
    if global_scales is not None:
        _need(global_scales, torch.float32, "global_scales")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [tokens, k]")
    tokens, k = x.shape
    pairs = pair_tokens.numel()
    cb, sb = fp4_prepared_bytes(n, k, fmt)
    if prep_codes.numel() < experts * cb or prep_scales.numel() < experts * sb:
        raise ValueError("stacked prepared buffers smaller than experts x fp4_prepared_bytes(n, k, fmt)")
    if expert_offsets.numel() != experts + 1:
        raise ValueError("expert_offsets must hold experts + 1 values")
    if y is None:
        y = torch.empty((pairs, n), dtype=torch.bfloat16, device=x.device)
    _need(y, torch.bfloat16, "y")
    if y.numel() != pairs * n:
        raise ValueError("y must hold pairs x n values")
    # Both routes read each pair's x row by its token id (the size query
    # reports 0 bytes).
    need = 0 if name == "fp4_w4a16_moe_prefill" else fp4_moe_workspace_bytes(pairs, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(name, getattr(load_library(), name)(
        _ptr(x), tokens, k, _ptr(prep_codes), _ptr(prep_scales), n, experts, _ptr(global_scales), fmt,
        _ptr(expert_offsets), _ptr(pair_tokens), pairs, _ptr(y), _ptr(workspace), ws_bytes, _stream(stream),
        None if info is None else ctypes.byref(info)))
    return y



def fp4_w4a4_act_bytes(m, k):
    """(code_bytes, scale_bytes) of the quantized activations of m rows of k values (W4A4 variant)."""
    cb, sb = _sz(), _sz()
    _check("fp4_w4a4_act_bytes", load_library().fp4_w4a4_act_bytes(m, k, ctypes.byref(cb), ctypes.byref(sb)))
    return cb.value, sb.value


def fp4_quantize_act_mxfp4(x, codes=None, scales=None, stream=None):
    """MXFP4 quantization of bf16 x [m, k] as the W4A4 variant does it; returns (codes, scales)
    uint8 buffers in the documented layout (rows padded to 128, k to 128)."""
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [m, k]")
    m, k = x.shape
    cb, sb = fp4_w4a4_act_bytes(m, k)
    if codes is None:
        codes = torch.empty(max(cb, 16), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(max(sb, 16), dtype=torch.uint8, device=x.device)
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    if codes.numel() < cb or scales.numel() < sb:
        raise ValueError("buffers smaller than fp4_w4a4_act_bytes(m, k)")
    _check("fp4_quantize_act_mxfp4", load_library().fp4_quantize_act_mxfp4(
        _ptr(x), m, k, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def fp4_w4a4_workspace_bytes(m, n, k, projections=1):
    out = _sz()
    _check("fp4_w4a4_workspace_bytes", load_library().fp4_w4a4_workspace_bytes(m, n, k, projections,
                                                                                ctypes.byref(out)))
    return out.value


def fp4_w4a4_linear(x, prep_codes, prep_scales, n, fmt=FMT_MXFP4, y=None, workspace=None, stream=None, info=None):
    """W4A4 variant: y = Q(x) @ w.T, Q the MXFP4 activation quantization, w a prepared MXFP4 weight."""
    _need(prep_codes, torch.uint8, "prep_codes")
    _need(prep_scales, torch.uint8, "prep_scales")
    k = x.shape[1]
    cb, sb = fp4_prepared_bytes(n, k, FMT_MXFP4)
    if prep_codes.numel() < cb or prep_scales.numel() < sb:
        raise ValueError("prepared buffers smaller than fp4_prepared_bytes(n, k, FMT_MXFP4)")
    m, y, workspace, ws_bytes = _linear_common(x, n, workspace, fp4_w4a4_workspace_bytes(x.shape[0], n, k, 1), y)
    _check("fp4_w4a4_linear", load_library().fp4_w4a4_linear(
        _ptr(x), m, k, _ptr(prep_codes), _ptr(prep_scales), n, fmt, _ptr(y), _ptr(workspace), ws_bytes,
        _stream(stream), None if info is None else ctypes.byref(info)))
    return y


def fp4_w4a4_gate_up(x, prep_codes, prep_scales, n_half, fmt=FMT_MXFP4, y=None, workspace=None, stream=None,
                     info=None):
    """W4A4 variant of the fused gate_up: returns bf16 [m, 2*n_half] = [Q(x) @ gate.T | Q(x) @ up.T]."""
    _need(prep_codes, torch.uint8, "prep_codes")
    _need(prep_scales, torch.uint8, "prep_scales")
    k = x.shape[1]
    cb, sb = fp4_prepared_bytes(n_half, k, FMT_MXFP4)
    if prep_codes.numel() < 2 * cb or prep_scales.numel() < 2 * sb:
        raise ValueError("prepared buffers smaller than twice fp4_prepared_bytes(n_half, k, FMT_MXFP4)")
    m, y, workspace, ws_bytes = _linear_common(
        x, 2 * n_half, workspace, fp4_w4a4_workspace_bytes(x.shape[0], n_half, k, 2), y)
    _check("fp4_w4a4_gate_up", load_library().fp4_w4a4_gate_up(
        _ptr(x), m, k, _ptr(prep_codes), _ptr(prep_scales), n_half, fmt, _ptr(y), _ptr(workspace), ws_bytes,
        _stream(stream), None if info is None else ctypes.byref(info)))
    return y


def fp4_quantize_act_nvfp4(x, input_scale, codes=None, scales=None, stream=None):
    """NVFP4 quantization of bf16 x [m, k] with the per-tensor input_scale, as the NVFP4 W4A4 variant
    does it; returns (codes uint8 [m, k/2], scales uint8 [m, k/16])."""
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [m, k]")
    m, k = x.shape
    if codes is None:
        codes = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((m, k // 16), dtype=torch.uint8, device=x.device)
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    if codes.numel() < m * (k // 2) or scales.numel() < m * (k // 16):
        raise ValueError("codes / scales smaller than [m, k/2] / [m, k/16]")
    _check("fp4_quantize_act_nvfp4", load_library().fp4_quantize_act_nvfp4(
        _ptr(x), m, k, float(input_scale), _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def fp4_w4a4_nvfp4_workspace_bytes(m, n, k, projections=1):
    out = _sz()
    _check("fp4_w4a4_nvfp4_workspace_bytes", load_library().fp4_w4a4_nvfp4_workspace_bytes(
        m, n, k, projections, ctypes.byref(out)))
    return out.value


def fp4_w4a4_nvfp4_linear(x, prep_codes, prep_scales, n, global_scale, input_scale, y=None, workspace=None,
                          stream=None, info=None):
    """NVFP4 W4A4 variant: y = alpha * (Q(x) @ w.T), alpha = input_scale * global_scale, w a prepared NVFP4 weight."""
    _need(prep_codes, torch.uint8, "prep_codes")
    _need(prep_scales, torch.uint8, "prep_scales")
    k = x.shape[1]
    cb, sb = fp4_prepared_bytes(n, k, FMT_NVFP4)
    if prep_codes.numel() < cb or prep_scales.numel() < sb:
        raise ValueError("prepared buffers smaller than fp4_prepared_bytes(n, k, FMT_NVFP4)")
    m, y, workspace, ws_bytes = _linear_common(x, n, workspace, fp4_w4a4_nvfp4_workspace_bytes(x.shape[0], n, k, 1),
                                               y)
    _check("fp4_w4a4_nvfp4_linear", load_library().fp4_w4a4_nvfp4_linear(
        _ptr(x), m, k, _ptr(prep_codes), _ptr(prep_scales), n, float(global_scale), float(input_scale), _ptr(y),
        _ptr(workspace), ws_bytes, _stream(stream), None if info is None else ctypes.byref(info)))
    return y


def fp4_w4a4_nvfp4_gate_up(x, prep_codes, prep_scales, n_half, gate_global_scale, up_global_scale, input_scale,
                           y=None, workspace=None, stream=None, info=None):
    """NVFP4 W4A4 fused gate_up: returns bf16 [m, 2*n_half] = [alpha_g Q(x) @ gate.T | alpha_u Q(x) @ up.T]."""
    _need(prep_codes, torch.uint8, "prep_codes")
    _need(prep_scales, torch.uint8, "prep_scales")
    k = x.shape[1]
    cb, sb = fp4_prepared_bytes(n_half, k, FMT_NVFP4)
    if prep_codes.numel() < 2 * cb or prep_scales.numel() < 2 * sb:
        raise ValueError("prepared buffers smaller than twice fp4_prepared_bytes(n_half, k, FMT_NVFP4)")
    m, y, workspace, ws_bytes = _linear_common(
        x, 2 * n_half, workspace, fp4_w4a4_nvfp4_workspace_bytes(x.shape[0], n_half, k, 2), y)
    _check("fp4_w4a4_nvfp4_gate_up", load_library().fp4_w4a4_nvfp4_gate_up(
        _ptr(x), m, k, _ptr(prep_codes), _ptr(prep_scales), n_half, float(gate_global_scale),
        float(up_global_scale), float(input_scale), _ptr(y), _ptr(workspace), ws_bytes, _stream(stream),
        None if info is None else ctypes.byref(info)))
    return y


def fp4_dequantize(prep_codes, prep_scales, n, k, global_scale, fmt, out=None, stream=None):
    """Dequantize a prepared weight to float32 [n, k] with the kernels' decoders."""
    _need(prep_codes, torch.uint8, "prep_codes")
    _need(prep_scales, torch.uint8, "prep_scales")
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=prep_codes.device)
    _need(out, torch.float32, "out")
    _check("fp4_dequantize", load_library().fp4_dequantize(
        _ptr(prep_codes), _ptr(prep_scales), n, k, float(global_scale), fmt, _ptr(out), _stream(stream)))
    return out
