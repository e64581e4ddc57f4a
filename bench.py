"""Benchmark of the W4A16 FP4 linear layer on one MI355X.

Prints ONE JSON line (rank 0, one GPU):
  metric  "W4A16 FP4 linear achieved HBM GB/s at M=1..8; TFLOP/s at M=1024"
  value   whole-job throughput over the timed steps: algorithmic bytes / s in
          GB/s for the decode workloads, 2*m*n*k / s in TFLOP/s for prefill.
A step is one call of the layer at each activation-row count m in the list
(default m = 1, 2, 4, 8 for the decode workloads, 1024 for prefill), on
synthetic activations, with the prepared weights already resident in HBM.

The default run (--workload suite) times every config of the metric in turn:
the MXFP4 fused gate_up (the headline: value, ms_per_step, roofline and
cpu_baseline are its own) at m = 1, 2, 4, 8, then the NVFP4 lm_head, down_proj
and o_proj at m = 1, 2, 4, 8, the NVFP4 and MXFP4 prefill GEMM at m = 1024,
and the two opt-in W4A4 variants at the prefill shape, m = 1024.
Every config's rate, fraction of its roofline peak and time per call per m
also go out as flat scalar keys, e.g. "lm_head_m8_gbs", "lm_head_m8_frac",
"lm_head_m8_us", "prefill_nvfp4_m1024_tflops".
Each m is timed with its own HIP events; by default the timed calls are
replayed from a captured HIP graph so the per-call launch gaps of the host
runtime do not count against the kernels.  Right before the timed region the
same calls are replayed, untimed, for --preroll-ms (default 50 ms): the GPU's
clock ramps up over the first milliseconds of a burst after idle, and 20
timed prefill calls straight after idle measured 214 µs each against 175 µs
under sustained load.
The weights are rotated over enough device copies (>= 1 GiB in total) that
the 256 MB Infinity Cache cannot hold them, so the bytes come from HBM.

Workloads (synthetic weights and activations at the pages' shapes):
  suite          the default: the configs listed above, one after another
  gate_up        MXFP4 fused gate_up, k=4096, n=2x12288          (headline)
  gate_up_swiglu the same weight interleaved, y = silu(gate) * up [m, 12288]
  lm_head        NVFP4 packed lm_head, k=5120, n=248320
  lm_head_argmax the same head with the fused greedy argmax (token ids out,
                 no logits)
  moe_gate_up    grouped MoE decode, NVFP4, 128 experts of n=1536, k=2048,
                 top-8 routing of m tokens (m = 1, 2, 4, 8); bytes counted
                 over the experts the routing activates
  moe_prefill    the same experts and routing recipe at prefill sizes
                 (m = 1024 tokens by default, 8192 pairs) on the grouped
                 MoE tile GEMM; TFLOP/s = 2 * pairs * n * k / s
  moe_prefill_swiglu  the same, each expert's 1536 rows taken as an
                 interleaved gate_up pair of 768, y = silu(gate) * up
  down_proj      NVFP4, k=17408, n=5120
  o_proj         NVFP4, k=6144, n=5120
  prefill_nvfp4  NVFP4, k=5120, n=17408 (m=1024 by default)
  prefill_mxfp4  MXFP4, k=5120, n=17408
  w4a4_gate_up   W4A4 variant (MXFP4 activations quantized per call x MXFP4
                 weights, block-scaled MFMA), the gate_up shape at m=1024
  w4a4_prefill   W4A4 variant, k=5120, n=17408, m=1024
  w4a4_nvfp4_prefill  NVFP4 W4A4 variant (activations quantized to NVFP4 with
                 the batch's calibrated per-tensor scale amax / (6 * 448),
                 contracted as exact bf16 by the W4A16 kernels), the NVFP4
                 prefill weight, m=1024
  tiny           NVFP4, k=256, n=512

Algorithmic bytes per call: packed codes (n*k/2) + scale bytes (n*k/g)
+ global scales (4 B each, NVFP4) + x (2*m*k) + y (2*m*n).  Split-K
partials, padding and rotation copies are not counted.

The roofline object covers the kernel that dominates the step (the longest
per-launch time): its average duration comes from HIP events around its timed
launches on the stream they run on; `traffic` is filled from a committed rocprofv3 counter summary in
profiles/ only when that summary was taken on the current kernel source.

Cross-checks per m (after the timed region, not part of value):
us_per_launch_differenced = (T(N2) - T(N1)) / (N2 - N1) from graphs of
N2 = steps and N1 = steps / 4 calls; for the fused gate_up,
us_split_launches = the same step with the gate and up halves launched as
two separate calls.

cpu_baseline: the oracle (NumPy, float64 sums), as it stands, timed on this
host's cores on a bounded sample of the same workload (a slice of the weight
rows), scaled to the same unit.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A16 FP4 linear achieved HBM GB/s at M=1..8; TFLOP/s at M=1024"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 1 << 30

# name: (workload id, fmt, n per projection, k, projections, default m)
WORKLOADS = {
    "gate_up": (1, 1, 12288, 4096, 2, 8),
    "gate_up_swiglu": (1, 1, 12288, 4096, 2, 8),
    "lm_head": (2, 0, 248320, 5120, 1, 8),
    "lm_head_argmax": (2, 0, 248320, 5120, 1, 8),
    "moe_gate_up": (0, 0, 1536, 2048, 1, 8),
    "moe_prefill": (0, 0, 1536, 2048, 1, 1024),
    "moe_prefill_swiglu": (0, 0, 1536, 2048, 1, 1024),
    "down_proj": (3, 0, 5120, 17408, 1, 8),
    "o_proj": (3, 0, 5120, 6144, 1, 8),
    "prefill_nvfp4": (4, 0, 17408, 5120, 1, 1024),
    "prefill_mxfp4": (4, 1, 17408, 5120, 1, 1024),
    "w4a4_gate_up": (1, 1, 12288, 4096, 2, 1024),
    "w4a4_prefill": (4, 1, 17408, 5120, 1, 1024),
    "w4a4_nvfp4_prefill": (4, 0, 17408, 5120, 1, 1024),
    "tiny": (0, 0, 512, 256, 1, 1),
}
TENSOR = {"o_proj": 1, "prefill_mxfp4": 1, "w4a4_prefill": 1}
# Workloads that run the W4A4 variant (activation quantizer + block-scaled MFMA GEMM).
W4A4 = {"w4a4_gate_up", "w4a4_prefill"}
W4A4_METRIC = "W4A4 MXFP4 linear TFLOP/s at M=1024 (opt-in variant: activations quantized to MXFP4)"
# Workloads that run the NVFP4 W4A4 variant (per-tensor input scale, activations
# quantized to NVFP4 and contracted by the W4A16 kernels as exact bf16 values).
W4A4_NV = {"w4a4_nvfp4_prefill"}
W4A4_NV_METRIC = ("W4A4 NVFP4 linear TFLOP/s at M=1024 (opt-in variant: activations quantized to NVFP4 with a "
                  "per-tensor input scale)")
FP4_MFMA_PEAK_TFLOPS = 10100.0
# Workloads that run the greedy-argmax entry point (no logits written).
ARGMAX = {"lm_head_argmax"}
# Workloads that run the SwiGLU gate_up (interleaved weight, y = silu(gate) * up).
SWIGLU = {"gate_up_swiglu"}
# Grouped MoE decode: 128 experts, top-8 routing per token, each expert a
# gate_up weight of 2 x 768 rows over k = 2048 (an A3B-class MoE block's
# shape; synthetic).  8 distinct expert weights are repeated over the 128.
MOE_EXPERTS, MOE_TOPK, MOE_DISTINCT = 128, 8, 8


def algorithmic_bytes(fmt, n_proj, k, projections, m, argmax=False, swiglu=False):
    """Weights + scales + global scales + x + output: y (2 m n), for the
    greedy argmax the token id and winning logit per row (6 m), for the
    SwiGLU gate_up y of one projection's width (2 m n_proj)."""
    g = 16 if fmt == 0 else 32
    n = n_proj * projections
    w = n * k // 2 + n * k // g + (4 * projections if fmt == 0 else 0)
    out = 6 * m if argmax else 2 * m * (n_proj if swiglu else n)
    return w + 2 * m * k + out


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp4_weight_only_e2m1_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload, m, kernel_hash):
    """Counter-derived HBM bytes per launch from profiles/traffic.json, if taken on this source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    e = data.get("%s_m%d" % (workload, m))
    if not e or e.get("kernel_source") != kernel_hash:
        return None
    return e.get("hbm_bytes_per_launch")


def make_inputs(name, m, torch, fp4, synth):
    wid, fmt, n, k, proj, _ = WORKLOADS[name]
    dev = torch.device("cuda:0")
    import numpy as np

    def upload(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    if proj == 2:
        pg, sg, gg = synth.packed_weight(wid, 0, n, k, fmt)
        pu, su, gu = synth.packed_weight(wid, 1, n, k, fmt)
        prep = fp4.fp4_prepare_gate_up_interleaved if name in SWIGLU else fp4.fp4_prepare_gate_up
        pc, ps = prep(upload(pg), upload(sg), upload(pu), upload(su), n, k, fmt)
        gs = (float(gg), float(gu))
        host = {"packed": (pg, pu), "scales": (sg, su), "g": (gg, gu)}
    else:
        p, s, g = synth.packed_weight(wid, TENSOR.get(name, 0), n, k, fmt)
        pc, ps = fp4.fp4_prepare(upload(p), upload(s), n, k, fmt)
        gs = (float(g),)
        host = {"packed": (p,), "scales": (s,), "g": (g,)}
    xb = synth.activations(wid, m, k)
    x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    torch.cuda.synchronize()
    return pc, ps, gs, x, xb, host


def cpu_baseline(name, xbs, host, budget_s):
    """Time the oracle on a bounded slice of weight rows, one call per m of the step.

    xbs: list of (m, bf16 bits of x).  Returns the cpu_baseline JSON object,
    with the value scaled from the slice to the whole step.
    """
    import numpy as np
    import oracle
    wid, fmt, n, k, proj, _ = WORKLOADS[name]
    xs = [(m, oracle.bf16_bits_to_f32(xb)) for m, xb in xbs]
    packed, scales, g = host["packed"][0], host["scales"][0], host["g"][0]

    def one_step(sl):
        for _, x in xs:
            if name in SWIGLU:
                oracle.gate_up_swiglu(x, host["packed"][0][sl], host["scales"][0][sl], host["packed"][1][sl],
                                      host["scales"][1][sl], k, fmt, host["g"][0], host["g"][1])
                continue
            if name in W4A4:
                oracle.w4a4_linear(x, packed[sl], scales[sl], k)
                continue
            if name in W4A4_NV:
                oracle.w4a4_nvfp4_linear(x, packed[sl], scales[sl], k, g,
                                         np.float32(np.float32(np.max(np.abs(x))) / np.float32(6 * 448)))
                continue
            y = oracle.linear(x, packed[sl], scales[sl], k, fmt, g)
            if name in ARGMAX:
                oracle.greedy_argmax(y)

    rows, spent = 256, 0.0
    # Grow the slice until one step takes a measurable time, then repeat within the budget.
    while True:
        sl = slice(0, min(rows, n))
        t0 = time.perf_counter()
        one_step(sl)
        dt = time.perf_counter() - t0
        spent += dt
        if dt > 0.5 or sl.stop == n or spent > budget_s:
            break
        rows *= 4
    reps = min(50, max(1, int((budget_s - spent) / max(dt, 1e-6))))
    t0 = time.perf_counter()
    for _ in range(reps):
        one_step(sl)
    dt = (time.perf_counter() - t0) / reps
    frac = sl.stop / (n * proj) * (2 if name in SWIGLU else 1)  # SwiGLU: the slice of both projections
    if name.startswith("prefill") or name in W4A4 or name in W4A4_NV:
        value = sum(2.0 * m * sl.stop * k for m, _ in xs) / dt / 1e12
        unit = "TFLOP/s"
    else:
        value = sum(algorithmic_bytes(fmt, n, k, proj, m, name in ARGMAX, name in SWIGLU)
                    for m, _ in xs) * frac / dt / 1e9
        unit = "GB/s"
    # The same slice at m = 1 on one BLAS thread (a second, single-core figure).
    single = None
    x1 = [x for m, x in xs if m == 1]
    if x1:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                t0 = time.perf_counter()
                r1 = 0
                while r1 < 50 and (r1 == 0 or time.perf_counter() - t0 < min(4.0, budget_s / 3)):
                    oracle.linear(x1[0], packed[sl], scales[sl], k, fmt, g)
                    r1 += 1
                d1 = (time.perf_counter() - t0) / r1
            v1 = (2.0 * sl.stop * k / d1 / 1e12 if name.startswith("prefill")
                  else algorithmic_bytes(fmt, n, k, proj, 1, name in ARGMAX) * frac / d1 / 1e9)
            single = {"value": round(v1, 4), "unit": unit, "cores": 1, "m": 1, "repetitions": r1}
        except ImportError:
            single = None
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = cores
    return {"value": round(value, 4), "unit": unit, "cores": int(threads or cores), "kind": "oracle",
            "sample": "%s over weight rows [0, %d) of %d, one call per "
                      "m in %s, %d timed repetitions; value scaled by the row fraction"
                      % ("oracle.w4a4_linear (activation quantization + dequant + float64 matmul)" if name in W4A4
                         else "oracle.w4a4_nvfp4_linear (activation quantization + dequant + float64 matmul)"
                         if name in W4A4_NV else "oracle.linear (dequant + float64 matmul)", sl.stop, n * proj,
                         [m for m, _ in xs],
                         reps),
            "host_cpus": cores, "single_thread": single}


def timed_calls(torch, fn, count, graph, preroll_ms=0.0):
    """Milliseconds for `count` calls fn(0..count-1) on the current stream:
    one replay of a graph that captured them (after an untimed replay, and
    untimed replays for preroll_ms of wall time), or direct launches."""
    stream = torch.cuda.current_stream()
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                fn(i)
        g.replay()
    t_pre = time.perf_counter()
    while preroll_ms > 0:
        if g is not None:
            g.replay()
        else:
            for i in range(count):
                fn(i)
        torch.cuda.synchronize()
        if time.perf_counter() - t_pre >= preroll_ms * 1e-3:
            break
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    if g is not None:
        g.replay()
    else:
        for i in range(count):
            fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def moe_routing(np, tokens, seed):
    """Top-MOE_TOPK distinct experts per token (seeded), pairs sorted by expert."""
    rng = np.random.default_rng(seed)
    pairs = sorted((int(e), t) for t in range(tokens)
                   for e in rng.choice(MOE_EXPERTS, size=MOE_TOPK, replace=False))
    offsets = np.searchsorted([p[0] for p in pairs], np.arange(MOE_EXPERTS + 1)).astype(np.int32)
    return offsets, np.array([p[1] for p in pairs], dtype=np.int32), sorted({p[0] for p in pairs})


def run_moe(args, torch, np, fp4, synth):
    """The grouped MoE workloads: one fp4_w4a16_moe_decode (moe_gate_up) or
    fp4_w4a16_moe_prefill (moe_prefill) call per step and m tokens."""
    name = args.workload
    swiglu = name == "moe_prefill_swiglu"
    prefill = name in ("moe_prefill", "moe_prefill_swiglu")
    wid, fmt, n, k, _, m_default = WORKLOADS[name]
    n_out = n // 2 if swiglu else n
    if args.m is not None:
        ms = [int(v) for v in args.m.split(",")]
    else:
        ms = [m_default] if prefill else [1, 2, 4, 8]
    if swiglu:
        def entry(x, c, s, n_, experts, gsc, fmt_, offsets, ptok, y=None, workspace=None, info=None):
            return fp4.fp4_w4a16_moe_prefill_swiglu(x, c, s, n_ // 2, experts, gsc, fmt_, offsets, ptok, y=y,
                                                    info=info)
    else:
        entry = fp4.fp4_w4a16_moe_prefill if prefill else fp4.fp4_w4a16_moe_decode
    kname = ("moe_gemm_kernel<%s>" if prefill else "moe_decode_kernel<%s>") % (
        ("nvfp4" if fmt == 0 else "mxfp4") + (",swiglu" if swiglu else ""))
    dev = torch.device("cuda:0")
    host, codes, scales, gvals = [], [], [], []
    for e in range(MOE_DISTINCT):
        p, s, g = synth.packed_weight(wid, 200 + e, n, k, fmt)
        if swiglu:
            # Rows [0, n/2) are the gate projection, [n/2, n) the up projection.
            h = n // 2
            pc, ps = fp4.fp4_prepare_gate_up_interleaved(
                *(torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (p[:h], s[:h], p[h:], s[h:])),
                h, k, fmt)
        else:
            pc, ps = fp4.fp4_prepare(torch.from_numpy(p).to(dev), torch.from_numpy(s).to(dev), n, k, fmt)
        host.append((p, s, g))
        codes.append(pc)
        scales.append(ps)
        gvals.append(float(g))
    rep_idx = [e % MOE_DISTINCT for e in range(MOE_EXPERTS)]
    pc_all = torch.cat([codes[i] for i in rep_idx])
    ps_all = torch.cat([scales[i] for i in rep_idx])
    gs = torch.tensor([gvals[i] for i in rep_idx for _ in range(2 if swiglu else 1)], dtype=torch.float32,
                      device=dev)
    footprint = pc_all.numel() + ps_all.numel()
    copies = max(2, math.ceil(ROTATE_BYTES / footprint))
    weights = [(pc_all, ps_all)] + [(pc_all.clone(), ps_all.clone()) for _ in range(copies - 1)]
    cb, sb = fp4.fp4_prepared_bytes(n, k, fmt)
    g_div = 16 if fmt == 0 else 32
    per_expert = n * k // 2 + n * k // g_div + (4 if fmt == 0 else 0)

    per_m = []
    for m in ms:
        offsets, ptok, active = moe_routing(np, m, seed=1000 + m)
        xb = synth.activations(wid, m, k)
        d = {"m": m, "x": torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16), "xb": xb,
             "offsets": torch.from_numpy(offsets).to(dev), "ptok": torch.from_numpy(ptok).to(dev),
             "offsets_h": offsets, "ptok_h": ptok, "active": active, "pairs": len(ptok),
             "y": torch.empty((len(ptok), n_out), dtype=torch.bfloat16, device=dev),
             "ws": torch.empty(fp4.fp4_moe_workspace_bytes(len(ptok), k), dtype=torch.uint8, device=dev),
             "info": fp4.fp4_dispatch_info()}
        d["bytes"] = len(active) * per_expert + 2 * m * k + 2 * len(ptok) * n_out
        d["flops"] = 2.0 * len(ptok) * n * k
        per_m.append(d)

    def call(d, i, fn=entry):
        c, s = weights[i % copies]
        fn(d["x"], c, s, n, MOE_EXPERTS, gs if fmt == 0 else None, fmt, d["offsets"], d["ptok"], y=d["y"],
           workspace=d["ws"], info=d["info"])

    for d in per_m:
        for i in range(args.warmup):
            call(d, i)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for d in per_m:
        d["t_ms"] = timed_calls(torch, lambda i, d=d: call(d, args.warmup + i), args.steps, args.launch == "graph",
                                args.preroll_ms)
    t_wall = time.perf_counter() - t_wall0
    rows, total_ms, total_bytes, total_flops = [], 0.0, 0, 0.0
    for d in per_m:
        us = d["t_ms"] * 1e3 / args.steps
        total_ms += d["t_ms"]
        total_bytes += d["bytes"] * args.steps
        total_flops += d["flops"] * args.steps
        info = d["info"]
        # The decode route runs the wave-split kernel (16-row tiles) for one or two tokens where it serves.
        kw = not prefill and info.grid_x * 16 == (n + 255) // 256 * 256
        row = {"m": d["m"], "kernel": kname.replace("moe_decode_kernel", "moe_decode_kw_kernel") if kw else kname,
               "us_per_launch": round(us, 3),
               "gbs": round(d["bytes"] / (us * 1e-6) / 1e9, 2), "tflops": round(d["flops"] / (us * 1e-6) / 1e12, 3),
               "pairs": d["pairs"], "active_experts": len(d["active"]),
               "grid": [info.grid_x, info.grid_y], "block": info.block, "algorithmic_bytes": d["bytes"],
               "flops": d["flops"]}
        if prefill and not swiglu and not args.no_crosscheck:
            # The same routing through the decode route (8 pairs of an expert per pass over its weight).
            t = timed_calls(torch, lambda i, d=d: call(d, i, fp4.fp4_w4a16_moe_decode), max(args.steps // 4, 5),
                            args.launch == "graph")
            row["us_decode_route"] = round(t * 1e3 / max(args.steps // 4, 5), 3)
        rows.append(row)
    dom = max(rows, key=lambda r: r["us_per_launch"])
    if prefill:
        value, unit = round(total_flops / (total_ms * 1e-3) / 1e12, 3), "TFLOP/s"
        roof = {"bound": "mfma", "achieved": dom["tflops"], "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(dom["tflops"] / BF16_MFMA_PEAK_TFLOPS, 4), "kernel": dom["kernel"], "m": dom["m"],
                "avg_launch_us": dom["us_per_launch"], "units_per_launch": dom["flops"],
                "traffic": read_traffic(name, dom["m"], kernel_source_hash())}
    else:
        value, unit = round(total_bytes / (total_ms * 1e-3) / 1e9, 3), "GB/s"
        roof = {"bound": "hbm", "achieved": dom["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom["gbs"] / HBM_PEAK_GBS, 4), "kernel": dom["kernel"], "m": dom["m"],
                "avg_launch_us": dom["us_per_launch"], "units_per_launch": dom["algorithmic_bytes"],
                "traffic": read_traffic(name, dom["m"], kernel_source_hash())}
    out = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(total_ms / args.steps, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "fmt": "nvfp4" if fmt == 0 else "mxfp4", "m": ms, "n": n, "k": k,
                   "experts": MOE_EXPERTS, "topk": MOE_TOPK, "distinct_expert_weights": MOE_DISTINCT,
                   "launch": args.launch, "rotated_weight_copies": copies,
                   "step": "one grouped call per m (m tokens, top-%d routing)" % MOE_TOPK, "per_m": rows,
                   "wall_s_timed": round(t_wall, 4)},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        d = per_m[0]
        xs = oracle.bf16_bits_to_f32(d["xb"])
        experts = [host[i] for i in rep_idx]
        offsets_h, ptok_h = d["offsets_h"], d["ptok_h"]
        if prefill:
            # Bounded sample: the first 16 pairs of the call (the oracle
            # dequantizes the expert's weight for every pair).
            sp = min(16, len(ptok_h))
            offsets_h = np.minimum(offsets_h, sp)
            ptok_h = ptok_h[:sp]

        def oracle_call():
            if not swiglu:
                return oracle.moe_decode(xs, experts, k, fmt, offsets_h, ptok_h)
            h = n // 2
            for e, (p_, s_, g_) in enumerate(experts):
                for q in range(int(offsets_h[e]), int(offsets_h[e + 1])):
                    t_ = int(ptok_h[q])
                    oracle.gate_up_swiglu(xs[t_:t_ + 1], p_[:h], s_[:h], p_[h:], s_[h:], k, fmt, g_, g_)

        t0 = time.perf_counter()
        reps = 0
        while reps == 0 or (time.perf_counter() - t0 < args.cpu_budget and reps < 20):
            oracle_call()
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        if prefill:
            out["cpu_baseline"] = {"value": round(2.0 * len(ptok_h) * n * k / dt / 1e12, 6), "unit": "TFLOP/s",
                                   "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                                   "sample": "%s of the first %d pairs of the m = %d call, %d repetitions"
                                             % ("oracle.gate_up_swiglu per pair" if swiglu else "oracle.moe_decode",
                                                len(ptok_h), d["m"], reps)}
        else:
            out["cpu_baseline"] = {"value": round(d["bytes"] / dt / 1e9, 4), "unit": "GB/s",
                                   "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                                   "sample": "oracle.moe_decode of the m = %d call (%d pairs over %d experts), %d "
                                             "repetitions" % (d["m"], d["pairs"], len(d["active"]), reps)}
    print(json.dumps(out), flush=True)


def run_dense(args, name, ms, torch, np, fp4, synth, crosscheck, with_cpu):
    """Time one dense workload (every m of `ms`, one call each per step) and
    return its result: per-m rows, totals, the rate, the roofline of the
    dominant kernel and, when asked, the oracle's CPU baseline."""
    wid, fmt, n, k, proj, m_default = WORKLOADS[name]
    dev = torch.device("cuda:0")
    pc, ps, gs, x0, xb0, host = make_inputs(name, ms[0], torch, fp4, synth)

    # Rotate over device copies of the prepared weight so the timed reads come from HBM.
    footprint = pc.numel() + ps.numel()
    copies = max(2, math.ceil(ROTATE_BYTES / footprint))
    weights = [(pc, ps)] + [(pc.clone(), ps.clone()) for _ in range(copies - 1)]
    nout = n * proj

    per_m = []
    for m in ms:
        xb = synth.activations(wid, m, k)
        x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
        y = torch.empty((m, n if name in SWIGLU else nout), dtype=torch.bfloat16, device=dev)
        if name in W4A4:
            ws_bytes = fp4.fp4_w4a4_workspace_bytes(m, n, k, proj)
        elif name in W4A4_NV:
            ws_bytes = fp4.fp4_w4a4_nvfp4_workspace_bytes(m, n, k, proj)
        elif name in SWIGLU:
            ws_bytes = fp4.fp4_swiglu_workspace_bytes(m, n, k, fmt)
        elif name in ARGMAX:
            ws_bytes = fp4.fp4_argmax_workspace_bytes(m, n, k, fmt)
        else:
            ws_bytes = fp4.fp4_workspace_bytes(m, n, k, fmt, proj)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        # NVFP4 W4A4: the per-tensor input scale a calibration over this batch gives, amax / (6 * 448).
        amax = float(np.max(np.abs((xb.astype(np.uint32) << 16).view(np.float32))))
        gx = float(np.float32(np.float32(amax) / np.float32(6 * 448)))
        per_m.append({"m": m, "x": x, "xb": xb, "y": y, "ws": ws, "info": fp4.fp4_dispatch_info(), "gx": gx,
                      "idx": torch.empty(m, dtype=torch.int32, device=dev),
                      "val": torch.empty(m, dtype=torch.bfloat16, device=dev)})

    def call(d, i):
        c, s = weights[i % copies]
        if name in W4A4:
            if proj == 2:
                fp4.fp4_w4a4_gate_up(d["x"], c, s, n, y=d["y"], workspace=d["ws"], info=d["info"])
            else:
                fp4.fp4_w4a4_linear(d["x"], c, s, n, y=d["y"], workspace=d["ws"], info=d["info"])
        elif name in W4A4_NV:
            fp4.fp4_w4a4_nvfp4_linear(d["x"], c, s, n, gs[0], d["gx"], y=d["y"], workspace=d["ws"], info=d["info"])
        elif name in SWIGLU:
            fp4.fp4_w4a16_gate_up_swiglu(d["x"], c, s, n, gs[0], gs[1], fmt, y=d["y"], workspace=d["ws"],
                                         info=d["info"])
        elif proj == 2:
            fp4.fp4_w4a16_gate_up(d["x"], c, s, n, gs[0], gs[1], fmt, y=d["y"], workspace=d["ws"], info=d["info"])
        elif name in ARGMAX:
            fp4.fp4_w4a16_linear_argmax(d["x"], c, s, n, gs[0], fmt, idx=d["idx"], val=d["val"],
                                        workspace=d["ws"], info=d["info"])
        else:
            fp4.fp4_w4a16_linear(d["x"], c, s, n, gs[0], fmt, y=d["y"], workspace=d["ws"], info=d["info"])

    for d in per_m:
        for i in range(args.warmup):
            call(d, i)
    torch.cuda.synchronize()

    graphs = []
    if args.launch == "graph":
        for d in per_m:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(args.steps):
                    call(d, args.warmup + i)
            graphs.append(g)
        for g in graphs:   # one untimed replay each
            g.replay()
        torch.cuda.synchronize()

    # Untimed pre-roll right before the timed region: the same calls for at
    # least --preroll-ms of wall time, so the timed calls run at the clock the
    # GPU holds under sustained load rather than on its ramp up from idle.
    t_pre = time.perf_counter()
    while True:
        for j, d in enumerate(per_m):
            if graphs:
                graphs[j].replay()
            else:
                for i in range(args.steps):
                    call(d, args.warmup + i)
        torch.cuda.synchronize()
        if time.perf_counter() - t_pre >= args.preroll_ms * 1e-3:
            break

    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in per_m]
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for j, d in enumerate(per_m):
        evs[j][0].record(stream)
        if graphs:
            graphs[j].replay()
        else:
            for i in range(args.steps):
                call(d, args.warmup + i)
        evs[j][1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0

    total_ms = 0.0
    total_bytes = 0
    total_flops = 0.0
    rows = []
    for j, d in enumerate(per_m):
        ms_m = evs[j][0].elapsed_time(evs[j][1])
        d["t_ms"] = ms_m
        m = d["m"]
        b = algorithmic_bytes(fmt, n, k, proj, m, name in ARGMAX, name in SWIGLU)
        f = 2.0 * m * nout * k
        total_ms += ms_m
        total_bytes += b * args.steps
        total_flops += f * args.steps
        info = d["info"]
        kern = {0: "gemv_kernel", 2: "decode_mfma_kernel", 1: "gemm_kernel", 4: "w4a4_gemm_kernel",
                6: "decode_kw_kernel"}[info.kernel]
        us = ms_m * 1e3 / args.steps
        if info.kernel == 4:
            kname = "act_quant_kernel + w4a4_gemm_kernel" + (" + tail_reduce_kernel" if info.splits > 1 else "")
        else:
            kname = ("%s<%d,%s>" % (kern, m, "nvfp4" if fmt == 0 else "mxfp4") if info.kernel != 1
                     else "%s<%s>" % (kern, "nvfp4" if fmt == 0 else "mxfp4"))
        if name in ARGMAX:
            kname += " + argmax_reduce_kernel"
        if name in W4A4_NV:
            kname = "act_nvfp4_kernel + " + kname
        if name in SWIGLU:
            kname += " swiglu" if info.kernel != 1 else " + tail_reduce_kernel swiglu"
        rows.append({"m": m, "kernel": kname,
                     "us_per_launch": round(us, 3), "gbs": round(b / (us * 1e-6) / 1e9, 2),
                     "tflops": round(f / (us * 1e-6) / 1e12, 3), "splits": info.splits,
                     "grid": [info.grid_x, info.grid_y], "block": info.block,
                     "algorithmic_bytes": b, "flops": f})

    # Cross-checks, after (and not part of) the timed region:
    # * two-length differencing: the per-call time from graphs of N1 and N2
    #   calls, (T2 - T1) / (N2 - N1), which cancels any fixed cost per replay;
    # * fused gate_up only: the same step with the gate and up halves launched
    #   separately (two calls per step, the halves of the same prepared weight).
    n1 = max(1, args.steps // 4)
    for j, d in enumerate(per_m if crosscheck else []):
        t1 = timed_calls(torch, lambda i, d=d: call(d, args.warmup + i), n1, args.launch == "graph")
        if args.steps > n1:
            rows[j]["us_per_launch_differenced"] = round((d["t_ms"] - t1) * 1e3 / (args.steps - n1), 3)
        if name in W4A4:
            # The activation quantizer alone (the first launch of each call).
            qc, qs = fp4.fp4_w4a4_act_bytes(d["m"], k)
            qct = torch.empty(qc, dtype=torch.uint8, device=dev)
            qst = torch.empty(qs, dtype=torch.uint8, device=dev)
            tq = timed_calls(torch, lambda i, d=d: fp4.fp4_quantize_act_mxfp4(d["x"], qct, qst), args.steps,
                             args.launch == "graph")
            rows[j]["us_act_quant"] = round(tq * 1e3 / args.steps, 3)
            rows[j]["us_gemm_and_reduce"] = round(rows[j]["us_per_launch"] - rows[j]["us_act_quant"], 3)
        if name in W4A4_NV:
            # The same W4A16 call on x alone (the launches after the quantizer).
            wsb = fp4.fp4_workspace_bytes(d["m"], n, k, fmt, 1)
            wsl = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)

            def w4a16_call(i, d=d, wsl=wsl):
                c, s = weights[(args.warmup + i) % copies]
                fp4.fp4_w4a16_linear(d["x"], c, s, n, gs[0], fmt, y=d["y"], workspace=wsl)

            tw = timed_calls(torch, w4a16_call, args.steps, args.launch == "graph")
            rows[j]["us_w4a16_call"] = round(tw * 1e3 / args.steps, 3)
            rows[j]["us_quantizer"] = round(rows[j]["us_per_launch"] - rows[j]["us_w4a16_call"], 3)
        if proj == 2 and name not in SWIGLU and name not in W4A4:
            cb, sb = fp4.fp4_prepared_bytes(n, k, fmt)
            yg = torch.empty((d["m"], n), dtype=torch.bfloat16, device=dev)
            yu = torch.empty((d["m"], n), dtype=torch.bfloat16, device=dev)
            wsb = fp4.fp4_workspace_bytes(d["m"], n, k, fmt, 1)
            wsg = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
            wsu = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)

            def split_call(i, d=d, yg=yg, yu=yu, wsg=wsg, wsu=wsu, cb=cb, sb=sb):
                c, s = weights[(args.warmup + i) % copies]
                fp4.fp4_w4a16_linear(d["x"], c[:cb], s[:sb], n, gs[0], fmt, y=yg, workspace=wsg)
                fp4.fp4_w4a16_linear(d["x"], c[cb:], s[sb:], n, gs[1], fmt, y=yu, workspace=wsu)

            for i in range(args.warmup):
                split_call(i)
            ts = timed_calls(torch, split_call, args.steps, args.launch == "graph")
            rows[j]["us_split_launches"] = round(ts * 1e3 / args.steps, 3)

    # Rates follow the kernel that ran: the decode kernels (m <= 32) stream
    # the weights (GB/s against HBM), the tile GEMMs contract (TFLOP/s).
    prefill = any(d["info"].kernel in (1, 4) for d in per_m)
    if prefill:
        value = total_flops / (total_ms * 1e-3) / 1e12
        unit = "TFLOP/s"
    else:
        value = total_bytes / (total_ms * 1e-3) / 1e9
        unit = "GB/s"
    dom = max(rows, key=lambda r: r["us_per_launch"])
    if prefill:
        peak = FP4_MFMA_PEAK_TFLOPS if name in W4A4 else BF16_MFMA_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": dom["tflops"], "peak": peak, "unit": "TFLOP/s",
                "frac": round(dom["tflops"] / peak, 4)}
    else:
        roof = {"bound": "hbm", "achieved": dom["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom["gbs"] / HBM_PEAK_GBS, 4)}
    roof.update({"kernel": dom["kernel"], "m": dom["m"], "avg_launch_us": dom["us_per_launch"],
                 "units_per_launch": dom["flops"] if prefill else dom["algorithmic_bytes"],
                 "traffic": read_traffic(name, dom["m"], kernel_source_hash())})

    res = {"name": name, "fmt": fmt, "n": nout, "k": k, "proj": proj, "ms": ms, "rows": rows,
           "total_ms": total_ms, "value": value, "unit": unit, "roofline": roof, "copies": copies,
           "t_wall": t_wall, "cpu_baseline": None}
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline(name, [(d["m"], d["xb"]) for d in per_m], host, args.cpu_budget)
    del weights, per_m, graphs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


# The default run: the headline workload (the metric's M = 1..8 decode
# config) with its cross-checks and CPU baseline, then every other config of
# the metric at its own m values.  Each config's rates also go out as flat
# scalar keys of the JSON line (see suite_keys).
SUITE = [("gate_up", [1, 2, 4, 8]), ("lm_head", [1, 2, 4, 8]), ("down_proj", [1, 2, 4, 8]),
         ("o_proj", [1, 2, 4, 8]), ("prefill_nvfp4", [1024]), ("prefill_mxfp4", [1024]),
         ("w4a4_nvfp4_prefill", [1024]), ("w4a4_prefill", [1024])]


def suite_keys(res):
    """Flat scalar keys of one config's result: per m, the rate (GB/s for the
    decode kernels, TFLOP/s for the tile GEMMs), its fraction of the roofline
    peak and the time per call."""
    out = {}
    for r in res["rows"]:
        tile = "gemm_kernel" in r["kernel"]
        key = "%s_m%d" % (res["name"], r["m"])
        if tile:
            peak = FP4_MFMA_PEAK_TFLOPS if res["name"] in W4A4 else BF16_MFMA_PEAK_TFLOPS
            out[key + "_tflops"] = r["tflops"]
            out[key + "_frac"] = round(r["tflops"] / peak, 4)
        else:
            out[key + "_gbs"] = r["gbs"]
            out[key + "_frac"] = round(r["gbs"] / HBM_PEAK_GBS, 4)
        out[key + "_us"] = r["us_per_launch"]
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="suite", choices=["suite"] + sorted(WORKLOADS),
                    help="suite (default): every config of the metric, headline gate_up first")
    ap.add_argument("--m", default=None,
                    help="activation rows, comma separated (default: 1,2,4,8 for decode, 1024 for prefill)")
    ap.add_argument("--launch", default="graph", choices=["graph", "eager"],
                    help="replay the timed calls from a captured HIP graph, or launch them one by one")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle timing")
    ap.add_argument("--preroll-ms", type=float, default=50.0,
                    help="untimed replays of the timed calls right before the timed region, in ms of wall time "
                         "(the GPU clock ramps up over the first milliseconds of a burst)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-crosscheck", action="store_true",
                    help="skip the differencing and split-launch cross-checks (e.g. under a counter "
                         "profiler, where their launches would mix with the timed ones)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 10 plain device-to-device copies of MIB MiB (reference for the HBM "
                         "byte counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the layer's kernels run on a single MI355X and no "
              "multi-GPU path is built (the layer would shard over its output rows, each GPU running the same "
              "kernels on its share of the weight).", file=sys.stderr)
        sys.exit(2)

    import torch
    import numpy as np
    import fp4_weight_only_e2m1_amd as fp4
    import synth

    if args.calibrate_copy:
        nbytes = args.calibrate_copy << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": nbytes, "copies": 10}), flush=True)
        return

    name = args.workload
    if name in ("moe_gate_up", "moe_prefill", "moe_prefill_swiglu"):
        return run_moe(args, torch, np, fp4, synth)
    if name == "suite":
        results = [run_dense(args, w, wms, torch, np, fp4, synth, crosscheck=(j == 0 and not args.no_crosscheck),
                             with_cpu=(j == 0 and not args.no_cpu_baseline))
                   for j, (w, wms) in enumerate(SUITE)]
    else:
        wid, fmt, n, k, proj, m_default = WORKLOADS[name]
        if args.m is None:
            ms = [1, 2, 4, 8] if m_default <= 8 else [m_default]
        else:
            ms = [int(v) for v in args.m.split(",")]
        results = [run_dense(args, name, ms, torch, np, fp4, synth, crosscheck=not args.no_crosscheck,
                             with_cpu=not args.no_cpu_baseline)]
    head = results[0]
    out = {
        "metric": (W4A4_METRIC if head["name"] in W4A4 else W4A4_NV_METRIC if head["name"] in W4A4_NV else METRIC),
        "value": round(head["value"], 3),
        "unit": head["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["total_ms"] / args.steps, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4" if head["name"] in W4A4 else "bf16", "data": "synthetic",
        "config": {"workload": head["name"], "fmt": "nvfp4" if head["fmt"] == 0 else "mxfp4", "m": head["ms"],
                   "n": head["n"], "k": head["k"], "projections": head["proj"], "launch": args.launch,
                   "rotated_weight_copies": head["copies"], "step": "one call at each m in the list",
                   "per_m": head["rows"], "wall_s_timed": round(head["t_wall"], 4),
                   "suite": [{"workload": r["name"], "m": r["ms"], "n": r["n"], "k": r["k"],
                              "value": round(r["value"], 3), "unit": r["unit"], "per_m": r["rows"]}
                             for r in results[1:]]},
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
    }
    for r in results:
        out.update(suite_keys(r))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
