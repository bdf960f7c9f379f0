"""Benchmark of the MoE FFN layer on one MI355X.

One step = one full forward of the layer (router, dispatch, gate/up GEMM,
down GEMM, combine) over one batch of synthetic tokens whose inputs and weights
are already resident in HBM. The headline workload is the Mixtral-8x7B-shaped
prefill layer (T=4096, d_model=4096, E=8, top-2, d_ff=14336, bf16); by default
the other four layer shapes (fine-grained 128 experts top-4, decode T=32,
skewed 64 experts with two hot ones, and the same with 20 masked experts) are
timed in the same run and reported under "workloads".

Prints one JSON line: the headline's throughput (tokens/s), the roofline
position of its dominant kernel (the gate/up GEMM, its average duration
measured live with the library's HIP events on the layer's stream), the layer's
MFMA and HBM fractions, one sub-record per workload, and the CPU oracle timed on
a bounded sample of the headline workload.

    python bench.py [--steps K] [--warmup W] [--workloads all|NAME[,NAME...]]
                    [--fp8-weights] [--fp8-activations] [--no-cpu-baseline]

The timed loop runs on a handle without per-stage events; kernel durations come
from a second handle with COLIBRI_MOE_FLAG_STAGE_TIMING over the same number of
steps. --fp8-weights builds the layers with 8-bit expert weights (E4M3 codes,
one power-of-two scale per weight row, converted to bf16 in registers).
--fp8-activations (implies --fp8-weights) also quantizes the token rows and
runs the gate/up GEMM on the fp8 MFMA; its roofline peak is then the fp8 one.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at 1 GPU; % of peak MFMA (prefill) / HBM GB/s (decode)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (vector and matrix)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
WORKLOAD_NAMES = {
    "mixtral": "mixtral-8x7b-prefill",
    "fine-grained": "fine-grained-128e-top4",
    "decode": "mixtral-8x7b-decode",
    "skewed": "skewed-64e-top2",
    "skewed-masked": "skewed-64e-top2-20-empty",
    "tiny-f32": "tiny-f32",
    "dense": "dense-single-expert",
    "square": "square-gemm-8192",
}
DEFAULT_WORKLOADS = ("mixtral", "fine-grained", "decode", "skewed", "skewed-masked")
HEADLINE = "mixtral"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workloads", default="all",
                    help="'all' (the five layer shapes, headline mixtral) or a comma-separated list; "
                         "the first one listed is the headline")
    ap.add_argument("--fp8-weights", action="store_true",
                    help="8-bit expert weights (bf16 workloads only)")
    ap.add_argument("--fp8-activations", action="store_true",
                    help="8-bit expert weights and token rows, fp8 MFMA gate/up GEMM (bf16 workloads only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens of the oracle sample (0 = sized to ~15 s of CPU work)")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure attainable rates (the library's stream copy, its grouped GEMM on one expert "
                         "at square and dense shapes, torch.matmul beside it for reference) and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (to scale HBM counters) and exit")
    return ap.parse_args()


def copy_calibration(mib: int):
    """A device-to-device copy of known size with the library's own streaming
    copy kernel: its FETCH_SIZE / WRITE_SIZE readings give the factor between
    those counters and bytes moved, and its rate (bytes read + written per
    second) is the attainable HBM figure stated next to the 8 TB/s nominal
    one. torch's own copy is timed beside it."""
    import torch
    import sparse_moe_gemm_amd as cm

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)

    def rate(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(10):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / 10

    ms = rate(lambda: cm.stream_copy(src, dst))
    ms_torch = rate(lambda: dst.copy_(src))
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 13, "kernel": "stream_copy_kernel",
                      "copy_gbs_read_plus_write": 2 * n * 4 / (ms * 1e-3) / 1e9, "copy_ms": ms,
                      "torch_copy_gbs_read_plus_write": 2 * n * 4 / (ms_torch * 1e-3) / 1e9}), flush=True)


def peaks(args):
    """Attainable rates on this GPU next to the nominal peaks: the library's
    streaming copy (bytes read + written per second, 2 GiB), and its grouped
    GEMM with every token on one expert, so that the gate/up GEMM is one
    plain dense product, at M = N = K = 8192 and at 8192 x 28672 x 4096 (the
    Mixtral gate/up shape with all 8192 rows on one expert). torch.matmul on
    the same bf16 shapes (a vendor library GEMM, not part of this library) is
    timed beside it for reference, and, on the mixtral, fine-grained and
    skewed layers' own routing, one torch.matmul per active expert beside the
    library's grouped gate/up and down GEMMs. Kernel times are the layer's own stage
    events (median of K forwards)."""
    import torch

    import synth
    import sparse_moe_gemm_amd as cm

    out = {"nominal": {"bf16_mfma_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS}}
    n = (2 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)

    def timed(fn, reps=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out["stream_copy_gbs"] = 2 * n * 4 / (timed(lambda: cm.stream_copy(src, dst)) * 1e-3) / 1e9
    out["torch_copy_gbs"] = 2 * n * 4 / (timed(lambda: dst.copy_(src)) * 1e-3) / 1e9
    del src, dst
    gemms = {}
    for name in ("square", "dense"):
        cfg = synth.CONFIGS[name]
        inp = synth.make_inputs(cfg)
        wts = [to_dev(inp[k]) for k in ("w_router", "b_router", "w_gate", "w_up", "w_down")]
        x = to_dev(inp["x"])
        y = torch.empty_like(x)
        layer = cm.MoELayer(*wts, cfg.k, max_tokens=cfg.T, flags=cm.FLAG_ASYNC | cm.FLAG_STAGE_TIMING)
        for _ in range(args.warmup):
            layer.forward(x, y)
        ts = []
        for _ in range(args.steps):
            layer.forward(x, y)
            ts.append(layer.stage_times()["gate_up_gemm"])
        layer.close()
        M, N, K = cfg.T, 2 * cfg.f, cfg.d
        flop = 2.0 * M * N * K
        ours = float(np.median(ts))
        a = torch.randn(M, K, device="cuda").to(torch.bfloat16)
        b = torch.randn(K, N, device="cuda").to(torch.bfloat16)
        ref = timed(lambda: torch.matmul(a, b))
        gemms[f"{M}x{N}x{K}"] = {"library_gate_up_ms": ours, "library_tflops": flop / (ours * 1e-3) / 1e12,
                                 "torch_matmul_ms": ref, "torch_matmul_tflops": flop / (ref * 1e-3) / 1e12}
        del a, b, x, y, wts
        torch.cuda.empty_cache()
    out["gemm_bf16"] = gemms
    out["grouped_gate_up"] = {name: grouped_reference(name, args, timed) for name in ("mixtral", "fine-grained", "skewed")}
    print(json.dumps(out), flush=True)


def grouped_reference(name, args, timed):
    """The expert GEMMs of a layer shape on its own routing: the library's
    grouped kernels (stage events; gate/up also gathers the token rows through
    perm and applies SiLU(g)*u) against one torch.matmul (hipBLASLt) per
    active expert on rows already in expert order (a vendor library reference,
    not part of this library; gathering and weight transposes are outside its
    timed region, and the down products take random bf16 rows of h)."""
    import torch

    import synth
    import sparse_moe_gemm_amd as cm

    cfg = synth.CONFIGS[name]
    inp = synth.make_inputs(cfg)
    wts = [to_dev(inp[k]) for k in ("w_router", "b_router", "w_gate", "w_up", "w_down")]
    x = to_dev(inp["x"])
    y = torch.empty_like(x)
    layer = cm.MoELayer(*wts, cfg.k, max_tokens=cfg.T, flags=cm.FLAG_ASYNC | cm.FLAG_STAGE_TIMING)
    rt = layer.routing_buffers(cfg.T)
    for _ in range(args.warmup):
        layer.forward(x, y, routing=rt)
    ts, td = [], []
    for _ in range(args.steps):
        layer.forward(x, y, routing=rt)
        st = layer.stage_times()
        ts.append(st["gate_up_gemm"])
        td.append(st["down_gemm"])
    layer.close()
    torch.cuda.synchronize()
    ours, ours_dn = float(np.median(ts)), float(np.median(td))
    counts = rt["expert_counts"].cpu().tolist()
    offs = rt["expert_offsets"].cpu().tolist()
    a_sorted = x[rt["perm"].long()].contiguous()
    # [E][d][2f] contiguous right operands (gate rows then up rows of each expert)
    w_gu = torch.cat([wts[2], wts[3]], dim=1).transpose(1, 2).contiguous()
    w_dn = wts[4].transpose(1, 2).contiguous()  # [E][f][d]
    h_sorted = torch.randn(cfg.T * cfg.k, cfg.f, device="cuda").to(torch.bfloat16)
    del wts, x, y, rt
    active = [e for e in range(cfg.E) if counts[e] > 0]
    outs = {e: torch.empty(counts[e], 2 * cfg.f, dtype=torch.bfloat16, device="cuda") for e in active}
    outs_dn = {e: torch.empty(counts[e], cfg.d, dtype=torch.bfloat16, device="cuda") for e in active}

    def per_expert():
        for e in active:
            torch.matmul(a_sorted[offs[e]:offs[e + 1]], w_gu[e], out=outs[e])

    def per_expert_dn():
        for e in active:
            torch.matmul(h_sorted[offs[e]:offs[e + 1]], w_dn[e], out=outs_dn[e])

    ref = timed(per_expert)
    ref_dn = timed(per_expert_dn)
    flop = 4.0 * cfg.d * cfg.f * cfg.T * cfg.k
    del a_sorted, w_gu, outs, h_sorted, w_dn, outs_dn
    torch.cuda.empty_cache()
    return {"workload": WORKLOAD_NAMES.get(name, name), "active_experts": len(active),
            "library_gate_up_ms": ours, "library_tflops": flop / (ours * 1e-3) / 1e12,
            "torch_matmul_per_expert_ms": ref, "torch_matmul_per_expert_tflops": flop / (ref * 1e-3) / 1e12,
            "library_down_ms": ours_dn, "torch_matmul_per_expert_down_ms": ref_dn}


def to_dev(a):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to("cuda")


def gemm_flops_per_assignment(cfg):
    """Algorithmic flops per (token, slot) assignment of each expert GEMM."""
    return {"gate_up_gemm": 4.0 * cfg.d * cfg.f, "down_gemm": 2.0 * cfg.d * cfg.f}


def active_weight_bytes(cfg, counts, stage, fp8=False):
    """Bytes of the active experts' weights of one GEMM (fp8: codes plus one
    fp32 scale per weight row)."""
    n_active = int((counts > 0).sum())
    if fp8:
        per = {"gate_up_gemm": 2 * cfg.f * (cfg.d + 4), "down_gemm": cfg.d * (cfg.f + 4)}[stage]
    else:
        es = cfg.elem_bytes()
        per = {"gate_up_gemm": 2 * cfg.d * cfg.f * es, "down_gemm": cfg.d * cfg.f * es}[stage]
    return n_active * per


def layer_bytes(cfg, counts, fp8=False):
    """Algorithmic HBM bytes of one forward: the active experts' weights (read
    once), the router weights and bias, x and y."""
    es = cfg.elem_bytes()
    w = active_weight_bytes(cfg, counts, "gate_up_gemm", fp8) + active_weight_bytes(cfg, counts, "down_gemm", fp8)
    return w + cfg.d * cfg.E * es + cfg.E * 4 + 2 * cfg.T * cfg.d * es


def source_digest() -> str:
    """sha256 over every file of the library's sources (names and contents):
    a profile taken on other sources says nothing about these kernels."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_moe_gemm_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        h.update(fn.encode())
        h.update(open(os.path.join(csrc, fn), "rb").read())
    return h.hexdigest()


def profile_fields(workload: str, kernel: str) -> dict:
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_rocprof.md")
    if not os.path.exists(path):
        return {}
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("|"):
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    return fields


def gate_up_kernel_name(cfg, A: int, fp8: bool, q8: bool) -> str:
    """The tiled gate/up kernel the library picks for a call (the rule in
    api.cpp): 64-wide K stages for bf16 weights when the layer has at least
    768 rows per expert on average, or at most CMOE_M_ORDER_ROWS (384; the
    layers in m-tile order) (CMOE_K64 bit 0; bit 2 drops the row condition),
    else the 32-wide kernel."""
    k64 = int(os.environ.get("CMOE_K64", "1"))
    order_m = A <= int(os.environ.get("CMOE_M_ORDER_ROWS", "384")) * cfg.E
    if not fp8 and not q8 and (k64 & 1) and ((k64 & 4) or order_m or A >= 768 * cfg.E):
        return "grouped_gemm64_kernel<true, false> (gate/up, 64-wide K stages)"
    return "grouped_gemm_kernel (gate/up" + (", fp8 MFMA" if q8 else "") + ")"


def profiled_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` ("gate_up_gemm") from the committed
    rocprofv3 summary of this workload (FETCH_SIZE and WRITE_SIZE, scaled by a
    plain copy's readings), or None when that summary is missing or was taken
    on library sources other than the current ones (sha256 of the whole csrc
    directory, which also covers launch decisions such as tile order and K
    splits)."""
    fields = profile_fields(workload, kernel)
    if fields.get("csrc_sha256") != source_digest():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.partition(":")[2].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, sample_tokens: int, fp8: bool = False, q8: bool = False):
    import oracle

    gomp = ctypes.CDLL("libgomp.so.1")
    threads = int(gomp.omp_get_max_threads())
    # fp8: the oracle's 8-bit layer is its ordinary layer on the dequantized
    # weights (quantized here, outside the timed part, as the library does at
    # init); q8 adds its 8-bit activation mode
    L = oracle.Layer.from_inputs(oracle.quantized_expert_weights(inp) if fp8 else inp, cfg.k)
    x = inp["x"]
    per_tok_macs = cfg.d * cfg.E + 3 * cfg.d * cfg.f * cfg.k
    if sample_tokens <= 0:
        # About 15 s of wall time at ~2 GMAC/s per thread for this scalar code.
        sample_tokens = int(15.0 * threads * 2.0e9 / per_tok_macs)
        sample_tokens = min(cfg.T, max(threads, sample_tokens))
    toks = np.arange(sample_tokens, dtype=np.int32)
    # When the sample is the whole (small) workload, repeat it until about
    # 10 s of CPU work have been timed.
    reps, dt = 0, 0.0
    while reps == 0 or (sample_tokens == cfg.T and dt < 10.0 and reps < 1000):
        t0 = time.perf_counter()
        L.forward(x, tokens=toks, act_fp8=q8)
        dt += time.perf_counter() - t0
        reps += 1
    what = f"first {sample_tokens} tokens of the workload" if reps == 1 else \
        f"all {sample_tokens} tokens of the workload, {reps} times"
    return {"value": reps * sample_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{what} (router, top-k and their {cfg.k} experts' SwiGLU FFN + combine in double), "
                      f"wall {dt:.2f} s"}


def run_workload(name: str, args, fp8: bool, q8: bool) -> dict:
    """Time one workload: K forwards on a handle without stage events (the
    step time), then K more on a handle with them (per-kernel durations)."""
    import torch

    import synth
    import sparse_moe_gemm_amd as cm

    cfg = synth.CONFIGS[name]
    if fp8 and cfg.dtype != "bf16":
        raise SystemExit("--fp8-weights / --fp8-activations need bf16 workloads")
    t_gen = time.perf_counter()
    inp = synth.make_inputs(cfg)
    t_gen = time.perf_counter() - t_gen
    wts = [to_dev(inp[n]) for n in ("w_router", "b_router", "w_gate", "w_up", "w_down")]
    flags = (cm.FLAG_FP8_WEIGHTS if fp8 else 0) | (cm.FLAG_FP8_ACTIVATIONS if q8 else 0)
    x = to_dev(inp["x"])
    y = torch.empty_like(x)

    # 1) step time: K back-to-back forwards, HIP events on the layer's stream
    layer = cm.MoELayer(*wts, cfg.k, max_tokens=cfg.T, flags=cm.FLAG_ASYNC | flags)
    rt = layer.routing_buffers(cfg.T)
    keep = {"expert_counts": rt["expert_counts"]}
    stream = layer.stream
    for _ in range(args.warmup):
        layer.forward(x, y, keep)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    t_wall = time.perf_counter()
    for _ in range(args.steps):
        layer.forward(x, y, keep)
    t_enq = time.perf_counter() - t_wall  # host time to enqueue the K forwards
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    counts = keep["expert_counts"].cpu().numpy()
    layer.close()

    # 1b) the same forward captured once into a HIP graph and replayed K
    # times (small batches, where launch gaps matter): the handle runs on the
    # capturing stream
    graph_ms = None
    if cfg.T * cfg.k <= 256 and cfg.dtype == "bf16":
        gs = torch.cuda.Stream()
        glayer = cm.MoELayer(*wts, cfg.k, max_tokens=cfg.T, flags=cm.FLAG_ASYNC | flags, stream=gs)
        with torch.cuda.stream(gs):
            for _ in range(2):
                glayer.forward(x, y)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gs):
            glayer.forward(x, y)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        with torch.cuda.stream(gs):
            ev0.record(gs)
            for _ in range(args.steps):
                graph.replay()
            ev1.record(gs)
        torch.cuda.synchronize()
        graph_ms = ev0.elapsed_time(ev1) / args.steps
        del graph
        glayer.close()

    # 1c) layers back to back (small batches): NB handles (each with its own
    # copy of the weights in its arena, so every layer streams its weights
    # from HBM) chained on one stream, x -> y0 -> y1 -> ..., as consecutive
    # MoE layers of a decode step would run; per-layer time of the chain
    chain_ms = None
    NB = 4
    if cfg.T * cfg.k <= 256 and cfg.dtype == "bf16":
        layers = [cm.MoELayer(*wts, cfg.k, max_tokens=cfg.T, flags=cm.FLAG_ASYNC | flags) for _ in range(NB)]
        cs = layers[0].stream
        ys = [torch.empty_like(x) for _ in range(NB)]

        def chain():
            src = x
            for L, dst in zip(layers, ys):
                L.forward(src, dst)
                src = dst

        for _ in range(args.warmup):
            chain()
        torch.cuda.synchronize()
        ev0.record(cs)
        for _ in range(args.steps):
            chain()
        ev1.record(cs)
        torch.cuda.synchronize()
        chain_ms = ev0.elapsed_time(ev1) / args.steps / NB
        for L in layers:
            L.close()
        del layers, ys

    # 2) per-kernel durations: the library's per-stage events (recorded on
    # the same stream as the kernels), averaged over K forwards
    layer = cm.MoELayer(*wts, cfg.k, max_tokens=cfg.T, flags=cm.FLAG_ASYNC | cm.FLAG_STAGE_TIMING | flags)
    for _ in range(max(1, args.warmup // 2)):
        layer.forward(x, y)
    stage_sum = {s: 0.0 for s in cm.STAGES}
    for _ in range(args.steps):
        layer.forward(x, y)
        for s, v in layer.stage_times().items():
            stage_sum[s] += v
    stage_ms = {s: v / args.steps for s, v in stage_sum.items()}
    layer.close()
    del wts, x, y
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    A = cfg.T * cfg.k
    t = ms_per_step * 1e-3
    peak_mm = PEAK_FP8_TFLOPS if q8 else PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    layer_tflops = cfg.flops() / t / 1e12
    layer_gbs = layer_bytes(cfg, counts, fp8) / t / 1e9
    # The library takes its small-batch (weight streaming) path for bf16 calls
    # with at most CMOE_DECODE_MAX_A (default 2048) assignments when no expert
    # holds more than CMOE_DECODE_MAX_ROWS rows (default 48, 32 with 8-bit
    # weights; 0: no such test): HBM-bound.
    max_rows = int(os.environ.get("CMOE_DECODE_MAX_ROWS", "32" if fp8 else "48"))
    small_batch = (cfg.dtype == "bf16" and A <= int(os.environ.get("CMOE_DECODE_MAX_A", "2048"))
                   and (max_rows == 0 or int(np.max(counts)) <= max_rows))
    dom = "gate_up_gemm"  # carries 2/3 of the flops and of the weight bytes
    prof_key = name + ("-w8a8" if q8 else "-fp8" if fp8 else "")
    traffic = profiled_traffic(prof_key, dom)
    if small_batch:
        achieved = active_weight_bytes(cfg, counts, dom, fp8) / (stage_ms[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                "kernel": ("decode_gemm_q8_kernel<true>" if q8 else "decode_gemm_f8_kernel<true>" if fp8
                           else f"decode_gemm_kernel<true, {1 if cfg.T <= 32 else 2}>") + " (gate/up)"}
    else:
        achieved = gemm_flops_per_assignment(cfg)[dom] * A / (stage_ms[dom] * 1e-3) / 1e12
        gu_peak = PEAK_FP8_TFLOPS if q8 else peak_mm
        roof = {"bound": "mfma", "achieved": achieved, "peak": gu_peak, "unit": "TFLOP/s",
                "frac": achieved / gu_peak, "traffic": traffic,
                "kernel": gate_up_kernel_name(cfg, A, fp8, q8)}
    return {
        "cfg": cfg,
        "inp": inp,
        "record": {
            "workload": WORKLOAD_NAMES[name] + ("-w8a8" if q8 else "-fp8-weights" if fp8 else ""),
            "T": cfg.T, "d_model": cfg.d, "n_experts": cfg.E, "top_k": cfg.k, "d_ff": cfg.f,
            "ms_per_step": ms_per_step,
            "tokens_per_s": cfg.T / t,
            "bound": "hbm" if small_batch else "mfma",
            "layer_tflops": layer_tflops,
            "layer_mfma_frac": layer_tflops / peak_mm,
            "layer_gbs": layer_gbs,
            "layer_hbm_frac": layer_gbs / PEAK_HBM_GBS,
            "kernel_roofline": roof,
            "stage_ms": stage_ms,
            "empty_experts": int((counts == 0).sum()),
            "active_experts": int((counts > 0).sum()),
            "host_enqueue_us_per_step": t_enq / args.steps * 1e6,
            "graph_replay_ms_per_step": graph_ms,
            "back_to_back_layers": NB if chain_ms is not None else None,
            "back_to_back_ms_per_layer": chain_ms,
            "wall_s_timed": t_wall,
            "input_gen_s": t_gen,
        },
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer build has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch  # noqa: F401

    import synth  # noqa: F401
    import sparse_moe_gemm_amd  # noqa: F401  (fails loudly without the built library)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.peaks:
        peaks(args)
        return
    names = list(DEFAULT_WORKLOADS) if args.workloads == "all" else args.workloads.split(",")
    for n in names:
        if n not in WORKLOAD_NAMES:
            raise SystemExit(f"unknown workload {n}; known: {', '.join(WORKLOAD_NAMES)}")
    q8 = bool(args.fp8_activations)
    fp8 = bool(args.fp8_weights) or q8

    results = {}
    for n in names:
        r = run_workload(n, args, fp8, q8)
        results[n] = r
        rec = r["record"]
        print(f"# {rec['workload']}: {rec['ms_per_step']:.3f} ms/step, {rec['tokens_per_s']:.4g} tokens/s, "
              f"layer MFMA {rec['layer_mfma_frac']:.3f} HBM {rec['layer_hbm_frac']:.3f}", file=sys.stderr,
              flush=True)
        if n != names[0]:
            del r["inp"]
    head = results[names[0]]
    cfg, rec = head["cfg"], head["record"]
    out = {
        "metric": METRIC,
        "value": rec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if q8 else cfg.dtype,
        "data": "synthetic (seeded SplitMix64 + Box-Muller, bf16 RNE; no trained weights)",
        "config": {"workload": rec["workload"], "T": cfg.T, "d_model": cfg.d, "n_experts": cfg.E,
                   "top_k": cfg.k, "d_ff": cfg.f, "router_bias": cfg.bias or None,
                   "expert_weights": "fp8-e4m3, per-row power-of-two scale" if fp8 else cfg.dtype,
                   "token_rows_for_gate_up": "fp8-e4m3, per-row power-of-two scale" if q8 else cfg.dtype},
        "roofline": rec["kernel_roofline"],
        "layer": {"tflops": rec["layer_tflops"], "mfma_frac": rec["layer_mfma_frac"], "gbs": rec["layer_gbs"],
                  "hbm_frac": rec["layer_hbm_frac"]},
        "stage_ms": rec["stage_ms"],
        "workloads": {results[n]["record"]["workload"]: results[n]["record"] for n in names},
        "csrc_sha256": source_digest(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, head["inp"], args.cpu_sample_tokens, fp8, q8)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
