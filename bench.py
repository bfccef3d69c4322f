"""Throughput of the MoE layer (route -> permute -> forward) on one MI355X.

A step is one pass of the whole layer over one batch, with every input already
resident in HBM.  The default workload is the Qwen3-MoE-30B-A3B-shaped decode
layer (hidden 2048, 128 experts, top-8, expert ffn 768, Q4_0 experts, bf16
router and activations) on a batch of 16 tokens.  Consecutive steps use
different copies of the expert weights, like consecutive layers of a model, so
no step finds its weights in the 256 MB Infinity Cache.

Prints one JSON line: tokens/s, ms per step, the dominant kernel's roofline
(its algorithmic bytes over its own duration, timed with HIP events on the
launch stream) and the CPU oracle's throughput on a bounded sample."""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moegen  # noqa: E402
from sparse_moe_block_amd import fwmoe as fw  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0
MFMA_FP8_PEAK_TFLOPS = 5000.0    # dense fp8 (E4M3 x E2M1 runs at the fp8 rate)
MFMA_INT8_PEAK_TOPS = 5000.0     # dense int8
METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA TFLOP/s (prefill)"
CSRC = os.path.join(ROOT, "sparse_moe_block_amd", "csrc")
# sources that decide each dominant kernel's memory traffic (a change to any
# voids its counter figures)
TRAFFIC_SOURCES = {"gemv_kernel<gate/up>": ["common.h", "abi.hip", "forward.hip", "stages.h",
                                            "gemv.hip"],
                   "gemm_mx_kernel<gate/up>": ["common.h", "abi.hip", "forward.hip", "stages.h",
                                               "gemm_mx.hip"],
                   "gemm_kernel<gate/up>": ["common.h", "abi.hip", "forward.hip", "stages.h",
                                            "gemm_frag.h", "gemm.hip"],
                   "gemm_i8_kernel<gate/up>": ["common.h", "abi.hip", "forward.hip", "stages.h",
                                               "gemm_i8.hip"]}

N_STAGES = fw.FW_N_STAGE_EVENTS - 1   # front/staging, gate/up routed, shared, down, combine
HEADLINE = "deepseek4096"   # the largest configuration, MFMA-bound (grouped GEMM)
DECODE_EXTRA = "decode16"   # the metric's HBM-bound decode point, carried as "decode"

WORKLOADS = {
    # name: (config, T, weight copies)
    "decode16": (moegen.QWEN3_DECODE, 16, 16),
    "decode4": (moegen.QWEN3_DECODE, 4, 16),
    "decode1": (moegen.QWEN3_DECODE, 1, 16),
    "deepseek1": (moegen.DEEPSEEK, 1, 2),
    "deepseek32": (moegen.DEEPSEEK, 32, 2),
    "prefill2048": (moegen.QWEN3_PREFILL, 2048, 4),
    "deepseek4096": (moegen.DEEPSEEK, 4096, 1),
    # the same shapes on Q4_K experts (GGUF K-quant super-blocks)
    "decode16_q4k": (moegen.QWEN3_DECODE.with_(expert_q=moegen.Q4_K), 16, 16),
    "prefill2048_q4k": (moegen.QWEN3_PREFILL.with_(expert_q=moegen.Q4_K), 2048, 4),
    # and on Q6_K experts (210-byte super-blocks)
    "decode16_q6k": (moegen.QWEN3_DECODE.with_(expert_q=moegen.Q6_K), 16, 16),
    "prefill2048_q6k": (moegen.QWEN3_PREFILL.with_(expert_q=moegen.Q6_K), 2048, 4),
    # and on MXFP4 experts (MLX packing, group 32)
    "decode16_mxfp4": (moegen.QWEN3_DECODE.with_(expert_q=moegen.MXFP4), 16, 16),
    "prefill2048_mxfp4": (moegen.QWEN3_PREFILL.with_(expert_q=moegen.MXFP4), 2048, 4),
    # MXFP4 experts with MXFP8 activations on the block-scaled MFMA
    "prefill2048_mx8": (moegen.QWEN3_PREFILL.with_(expert_q=moegen.MXFP4, act_quant="mxfp8"),
                        2048, 4),
    "deepseek4096_mx8": (moegen.DEEPSEEK.with_(expert_q=moegen.MXFP4, shared_q=moegen.MXFP4,
                                               act_quant="mxfp8"), 4096, 1),
    # int8 activations (Q8_1-style blocks) on the int8 MFMA
    "prefill2048_int8": (moegen.QWEN3_PREFILL.with_(act_quant="int8"), 2048, 4),
    "deepseek4096_int8": (moegen.DEEPSEEK.with_(act_quant="int8"), 4096, 1),
    # and on Q8_0 experts (the sweep's other format)
    "decode16_q8": (moegen.QWEN3_DECODE.with_(expert_q=moegen.Q8_0), 16, 8),
    "prefill2048_q8": (moegen.QWEN3_PREFILL.with_(expert_q=moegen.Q8_0), 2048, 2),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="deepseek4096", choices=sorted(WORKLOADS))
    ap.add_argument("--no-decode-extra", dest="decode_extra", action="store_false",
                    help="skip the decode T=16 figures the default line carries under "
                         "'decode' (the metric's HBM-bound point)")
    ap.add_argument("--peaks", action="store_true",
                    help="instead of the layer: measure the fp16 MFMA and streaming-read "
                         "peaks of this GPU and the price of a grid-wide rendezvous inside "
                         "one kernel, with the microbenchmarks of libfwpeak.so")
    ap.add_argument("--path", default="auto", choices=["auto", "gemv", "gemm"])
    ap.add_argument("--three-calls", action="store_true",
                    help="time the layer as fw_moe_route + fw_moe_permute + fw_moe_forward "
                         "instead of the one fw_moe_layer call")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time direct launches only (value from the direct loop)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--reduce-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="instead of benchmarking: turn two rocprofv3 --pmc output "
                         "directories (FETCH_SIZE, WRITE_SIZE) of this workload run "
                         "with --copy-mib into profiles/traffic_<kernel>_<workload>.json")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the one-line benchmark: the hidden-4096 / 64-expert "
                         "top-4 sweep layer over T = 1..8192 with Q8_0 and Q4_0 experts "
                         "and uniform or Zipf(1.3) routing, both kernel families timed "
                         "at each T; one JSON line per point, then the decode-to-prefill "
                         "crossover of each variant")
    ap.add_argument("--sweep-layer", default="sweep", choices=["sweep", "qwen3", "deepseek"],
                    help="layer of --sweep: the hidden-4096 sweep layer (default), the "
                         "Qwen3-MoE-30B-A3B-shaped layer, or the DeepSeek-shaped layer "
                         "(their own formats; T = 1..4096)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a negation "
                         "kernel, the reference that scales hardware byte counters)")
    return ap.parse_args()


def main():
    a = parse()
    if a.reduce_counters:
        reduce_counters(a)
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {a.gpus} is not supported "
              f"(the layer is measured on one MI355X)", file=sys.stderr)
        sys.exit(2)
    if a.sweep:
        sweep(a)
        return
    if a.peaks:
        peaks(a)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    line, ctx = measure(a, a.workload, a.steps, a.warmup)
    if a.decode_extra and a.workload == HEADLINE:
        # the decode point of the metric (HBM-bound GEMV family), same timing rules
        free(ctx)
        ctx = None
        dline, dctx = measure(a, DECODE_EXTRA, max(a.steps, 50), max(a.warmup, 10))
        free(dctx)
        line["decode"] = {k: dline[k] for k in ("value", "unit", "ms_per_step", "config",
                                                "direct_ms_per_step", "stage_us", "roofline")}
    if not a.no_cpu_baseline:
        if ctx is None:
            ctx = measure(a, a.workload, 0, 0, setup_only=True)[1]
        line["cpu_baseline"] = cpu_baseline(ctx["cfg"], ctx["L"], ctx["x"], ctx["T"],
                                            a.cpu_seconds)
    print(json.dumps(line), flush=True)


def free(ctx):
    if ctx is not None:
        ctx.clear()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def measure(a, workload, steps, warmup, setup_only=False):
    """One workload: K timed steps of the layer (HIP-graph replays; the same K
    steps as direct launches with per-stage events), the dominant kernel's
    roofline.  Returns the JSON fields and the layer (for the CPU baseline)."""
    cfg, T, copies = WORKLOADS[workload]
    dev = torch.device("cuda:0")
    L = moegen.make_layer(cfg, device=dev)
    x = moegen.make_x(cfg, T, device=dev)
    ctx = {"cfg": cfg, "L": L, "x": x, "T": T}
    if setup_only:
        return None, ctx
    layers = [L]
    for _ in range(copies - 1):
        layers.append(moegen.Layer(cfg, L.router, L.bias, L.w_gate.clone(), L.w_up.clone(),
                                   L.w_down.clone(),
                                   *(None if t is None else t.clone()
                                     for t in (L.s_gate, L.s_up, L.s_down))))
    ctx["layers"] = layers
    desc = fw.make_desc(cfg.hidden, cfg.n_experts, cfg.top_k, cfg.ffn, cfg.shared_ffn,
                        cfg.act_dtype, cfg.router_dtype, cfg.expert_q, cfg.shared_q,
                        cfg.score, a.path, cfg.act_quant)
    E, k, H = cfg.n_experts, cfg.top_k, cfg.hidden
    P = T * k
    logits = torch.empty(T, E, device=dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(P, dtype=torch.int32, device=dev)
    inv = torch.empty(P, dtype=torch.int32, device=dev)
    out = torch.empty(T, H, device=dev)
    ws = torch.empty(fw.fw_moe_workspace_size(desc, T), dtype=torch.uint8, device=dev)
    ctx["bufs"] = (logits, ids, w, off, sp, inv, out, ws)
    fw.fw_moe_clear_status(ws)
    stream = torch.cuda.current_stream()

    def step(i, s=stream, events=None):
        Li = layers[i % copies]
        if a.three_calls:
            fw.fw_moe_route(desc, T, x, Li.router, Li.bias, None, logits, ids, w, s)
            fw.fw_moe_permute(desc, T, ids, off, sp, inv, ws, stream=s)
            fw.fw_moe_forward(desc, T, x, Li.w_gate, Li.w_up, Li.w_down, Li.s_gate, Li.s_up,
                              Li.s_down, w, off, sp, inv, out, ws, stream=s)
        elif events is not None:
            fw.fw_moe_layer_timed(desc, T, x, Li.router, Li.bias, Li.w_gate, Li.w_up,
                                  Li.w_down, Li.s_gate, Li.s_up, Li.s_down, logits, ids, w,
                                  off, sp, inv, out, ws, events, stream=s)
        else:
            fw.fw_moe_layer(desc, T, x, Li.router, Li.bias, Li.w_gate, Li.w_up, Li.w_down,
                            Li.s_gate, Li.s_up, Li.s_down, logits, ids, w, off, sp, inv, out,
                            ws, stream=s)

    if a.copy_mib:
        # reads and writes exactly copy_mib MiB in one elementwise kernel
        src = torch.ones((a.copy_mib << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    status = fw.fw_moe_read_status(ws)
    assert status == 0, f"device status {status}"
    n_active = int((torch.diff(off) > 0).sum())

    # the K steps launched directly, each with its own stage events (HIP events
    # the library records on `stream` around the forward's stages); the
    # three-call form has no stage events and its stages are not timed
    timed = not a.three_calls
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(fw.FW_N_STAGE_EVENTS)]
           for _ in range(steps)] if timed else None
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        step(warmup + i, events=evs[i] if timed else None)
    t1.record(stream)
    torch.cuda.synchronize()
    direct_ms = t0.elapsed_time(t1) / steps
    if timed:
        stage_ms = np.array([[e[s].elapsed_time(e[s + 1]) for s in range(N_STAGES)]
                             for e in evs])
        stage_avg = stage_ms.mean(axis=0)
    else:
        stage_avg = np.full(N_STAGES, np.nan)

    # the same K steps as HIP-graph replays (one captured step per weight copy;
    # decode runtimes replay the layer as a graph).  Every ABI call is
    # asynchronous and allocation-free, so the library captures as is.
    graph_ms = None
    if not a.no_graph:
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c, torch.cuda.current_stream())
            graphs.append(g)
        # a replay gives the eager result bit for bit
        step(0)
        torch.cuda.synchronize()
        eager = out.clone()
        out.fill_(float("nan"))
        graphs[0].replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "graph replay differs from the eager step"
        del eager
        for i in range(warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record()
        for i in range(steps):
            graphs[(warmup + i) % copies].replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / steps
        del graphs
    ms = graph_ms if graph_ms is not None else direct_ms
    status = fw.fw_moe_read_status(ws)
    assert status == 0, f"device status {status}"

    # dominant kernel: the routed experts' gate/up launch (2/3 of the routed
    # expert bytes and flops); the shared expert's launch is timed apart
    path = fw.fw_moe_forward_path(desc, T)
    gu_ms = float(stage_avg[1])
    if path == fw.FW_PATH_GEMV:
        # bytes: the active experts' gate and up rows, x in (fp16), a out
        gu_alg = (n_active * 2 * cfg.ffn * moegen.row_bytes(cfg.expert_q, H) + T * H * 2 +
                  P * cfg.ffn * 2)
        achieved = gu_alg / (gu_ms * 1e-3) / 1e9
        roof = {"kernel": "gemv_kernel<gate/up>", "bound": "hbm", "achieved": achieved,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                "traffic": None, "algorithmic_bytes": gu_alg}
    else:
        # flops: 2 projections x 2 flops x P x H x F
        gu_alg = 4 * P * H * cfg.ffn
        achieved = gu_alg / (gu_ms * 1e-3) / 1e12
        kernel, peak, unit = {
            "none": ("gemm_kernel<gate/up>", MFMA_FP16_PEAK_TFLOPS, "TFLOP/s"),
            "mxfp8": ("gemm_mx_kernel<gate/up>", MFMA_FP8_PEAK_TFLOPS, "TFLOP/s"),
            "int8": ("gemm_i8_kernel<gate/up>", MFMA_INT8_PEAK_TOPS, "TOP/s")}[cfg.act_quant]
        roof = {"kernel": kernel, "bound": "mfma", "achieved": achieved, "peak": peak,
                "unit": unit, "frac": achieved / peak, "traffic": None,
                "algorithmic_flops": gu_alg}
    roof["duration_us"] = gu_ms * 1e3
    layer_bytes = (n_active * cfg.expert_bytes + cfg.shared_bytes + cfg.router_bytes +
                   cfg.act_bytes(T) + T * H * 4)
    fused = (not a.three_calls and path == fw.FW_PATH_GEMV and P <= 2048)
    stage0 = "front (top-k + permute + staging)" if fused else "prepare"
    layer_flops = 6 * P * H * cfg.ffn + 6 * T * H * cfg.shared_ffn + 2 * T * H * E

    roof["traffic"] = traffic(workload, roof)
    line = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"none": "f16", "mxfp8": "e4m3 x e2m1", "int8": "i8"}[cfg.act_quant],
        "data": "synthetic (seeded N(0,0.02) weights quantized to GGUF blocks, N(0,1) bf16 tokens)",
        "config": {"workload": f"{cfg.name}, T={T}", "hidden": H, "experts": E, "top_k": k,
                   "ffn": cfg.ffn, "expert_format": cfg.expert_q, "shared_ffn": cfg.shared_ffn,
                   "activations": {"none": "fp16"}.get(cfg.act_quant, cfg.act_quant),
                   "tokens": T, "active_experts": n_active, "weight_copies": copies,
                   "path": "gemv" if path == fw.FW_PATH_GEMV else "gemm"},
        "timing": "hip-graph replay per step" if graph_ms is not None else "direct launches",
        "entry": "three calls" if a.three_calls else "fw_moe_layer",
        "direct_ms_per_step": direct_ms,
        "layer_GBps": layer_bytes / (ms * 1e-3) / 1e9,
        "layer_TFLOPs": layer_flops / (ms * 1e-3) / 1e12,
        "stage_us": {n: round(float(v) * 1e3, 2) for n, v in
                     zip([stage0, "gate_up", "gate_up_shared", "down", "combine"], stage_avg)
                     if cfg.shared_ffn or n != "gate_up_shared"},
        "roofline": roof,
    }
    return line, ctx


def sweep(a):
    """Step time of a layer with each kernel family forced, over T = 1, 2, 3,
    4, 6, 8, 12, ... (powers of two and the points halfway between, to 8192
    for the sweep layer, 4096 for the others).  Each step is a
    HIP-graph replay of one fw_moe_layer call on one of 8 weight copies (2 for
    the DeepSeek-shaped layer; cold Infinity Cache either way, as in the main
    benchmark).  The GEMV family is timed while it is at most three
    times slower than the grouped GEMM; the crossover of a variant is the
    smallest T from which the GEMM step is faster at every larger T."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    copies = 8
    steps, warm = min(a.steps, 30), min(a.warmup, 5)
    summary = []
    if a.sweep_layer == "sweep":
        variants = [b.with_(zipf=z) for b in (moegen.SWEEP_Q8, moegen.SWEEP_Q4)
                    for z in (None, 1.3)]
        t_max = 8192
    elif a.sweep_layer == "qwen3":
        variants = [moegen.QWEN3_DECODE, moegen.QWEN3_PREFILL]
        t_max = 4096
    else:
        variants = [moegen.DEEPSEEK]
        t_max = 4096
        copies = 2
    for cfg in variants:
        zipf = cfg.zipf
        L = moegen.make_layer(cfg, device=dev)
        layers = [L] + [moegen.Layer(cfg, L.router, L.bias, L.w_gate.clone(),
                                     L.w_up.clone(), L.w_down.clone(),
                                     *(None if t is None else t.clone()
                                       for t in (L.s_gate, L.s_up, L.s_down)))
                        for _ in range(copies - 1)]
        E, k, H = cfg.n_experts, cfg.top_k, cfg.hidden
        times = {}
        gemv_on = True
        # powers of two and the points halfway between them (3 * 2^i)
        for T in sorted({2 ** i for i in range(14)} | {3 << i for i in range(13)}):
            if T > t_max:
                continue
            x = moegen.make_x(cfg, T, device=dev)
            P = T * k
            bufs = dict(logits=torch.empty(T, E, device=dev),
                        ids=torch.empty(T, k, dtype=torch.int32, device=dev),
                        w=torch.empty(T, k, device=dev),
                        off=torch.empty(E + 1, dtype=torch.int32, device=dev),
                        sp=torch.empty(P, dtype=torch.int32, device=dev),
                        inv=torch.empty(P, dtype=torch.int32, device=dev),
                        out=torch.empty(T, H, device=dev))
            row = {"variant": f"{cfg.name}, {cfg.expert_q}, "
                              f"{'zipf' + str(zipf) if zipf else 'uniform'}", "T": T}
            for path in ("gemv", "gemm"):
                if path == "gemv" and not gemv_on:
                    continue
                desc = fw.make_desc(H, E, k, cfg.ffn, cfg.shared_ffn, cfg.act_dtype,
                                    cfg.router_dtype, cfg.expert_q, cfg.shared_q, cfg.score,
                                    path)
                ws = torch.empty(fw.fw_moe_workspace_size(desc, T), dtype=torch.uint8,
                                 device=dev)
                fw.fw_moe_clear_status(ws)
                b = bufs

                def step(i, s):
                    Li = layers[i % copies]
                    fw.fw_moe_layer(desc, T, x, Li.router, Li.bias, Li.w_gate, Li.w_up,
                                    Li.w_down, Li.s_gate, Li.s_up, Li.s_down, b["logits"],
                                    b["ids"],
                                    b["w"], b["off"], b["sp"], b["inv"], b["out"], ws,
                                    stream=s)

                step(0, torch.cuda.current_stream())
                torch.cuda.synchronize()
                assert fw.fw_moe_read_status(ws) == 0
                graphs = []
                for c in range(copies):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        step(c, torch.cuda.current_stream())
                    graphs.append(g)
                for i in range(warm):
                    graphs[i % copies].replay()
                torch.cuda.synchronize()
                g0 = torch.cuda.Event(enable_timing=True)
                g1 = torch.cuda.Event(enable_timing=True)
                g0.record()
                for i in range(steps):
                    graphs[(warm + i) % copies].replay()
                g1.record()
                torch.cuda.synchronize()
                ms = g0.elapsed_time(g1) / steps
                row[f"{path}_us"] = round(ms * 1e3, 1)
                row[f"{path}_tok_s"] = round(T / (ms * 1e-3))
                del graphs, ws
            times[T] = row
            if "gemv_us" in row and row["gemv_us"] > 3 * row["gemm_us"]:
                gemv_on = False
            row["auto"] = "gemv" if fw.fw_moe_forward_path(
                fw.make_desc(H, E, k, cfg.ffn, cfg.shared_ffn, cfg.act_dtype,
                             cfg.router_dtype, cfg.expert_q, cfg.shared_q, cfg.score,
                             "auto"), T) == fw.FW_PATH_GEMV else "gemm"
            print(json.dumps(row), flush=True)
        cross = None
        for T in sorted(times, reverse=True):
            r = times[T]
            if "gemv_us" in r and r["gemv_us"] <= r["gemm_us"]:
                break
            cross = T
        summary.append({"variant": row["variant"], "crossover_T": cross})
        del layers, L
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": a.sweep_layer, "crossover": summary}), flush=True)


def peaks(a):
    """The two ceilings, measured on this GPU with libfwpeak.so: dense fp16
    MFMA throughput (16x16x32 and 32x32x16, every SIMD busy, eight independent
    accumulators per wavefront) and HBM streaming bandwidth (a 4 GiB read with
    16-byte loads; a 2 GiB copy); and the price of a grid-wide rendezvous
    inside one kernel.  One JSON line per figure, each the best of five timed
    launches after a warm-up."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_moe_block_amd", "libfwpeak.so"))
    lib.fw_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p]
    lib.fw_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p]
    lib.fw_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count

    def best(launch, n=5):
        launch()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts)

    # 4 or 8 wavefronts per CU (one or two per SIMD), several accumulator chains
    out = torch.empty(cus * 8 * 256, dtype=torch.float32, device=dev)
    for shape, flops, chain_set in ((16, 16384, (4, 8, 16)), (32, 32768, (2, 4, 8))):
        for per_simd in (1, 2):
            blocks = cus * per_simd
            for ch in chain_set:
                iters = 32000 // ch
                t = best(lambda: lib.fw_peak_mfma(shape, ch, blocks, iters,
                                                  ctypes.c_void_p(out.data_ptr()),
                                                  ctypes.c_void_p(stream.cuda_stream)))
                total = blocks * 4 * iters * ch * flops
                print(json.dumps({"peak": f"fp16 mfma {shape}x{shape}x{512 // shape}",
                                  "waves_per_simd": per_simd, "chains": ch, "seconds": t,
                                  "TFLOP/s": total / t / 1e12}), flush=True)
    nbytes = 4 << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    for blocks in (cus * 4, cus * 8, cus * 16):
        o = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
        t = best(lambda: lib.fw_peak_read(ctypes.c_void_p(src.data_ptr()), nbytes, blocks,
                                          ctypes.c_void_p(o.data_ptr()),
                                          ctypes.c_void_p(stream.cuda_stream)))
        print(json.dumps({"peak": "hbm streaming read", "bytes": nbytes, "workgroups": blocks,
                          "seconds": t, "GB/s": nbytes / t / 1e9}), flush=True)
    half = nbytes // 2
    dst = torch.empty(half // 4, dtype=torch.int32, device=dev)
    for blocks in (cus * 4, cus * 8):
        t = best(lambda: lib.fw_peak_copy(ctypes.c_void_p(src.data_ptr()),
                                          ctypes.c_void_p(dst.data_ptr()), half, blocks,
                                          ctypes.c_void_p(stream.cuda_stream)))
        print(json.dumps({"peak": "hbm copy (read + write)", "bytes_moved": 2 * half,
                          "workgroups": blocks, "seconds": t,
                          "GB/s": 2 * half / t / 1e9}), flush=True)
    del src, dst
    # one grid-wide rendezvous inside a kernel: (101 rounds - 1 round) / 100
    lib.fw_peak_grid_barrier.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 4
    for blocks in (cus // 2, cus, 2 * cus):
        for fence in (0, 1):
            per = {}
            for rounds in (1, 101):
                flags = torch.zeros(blocks * 16, dtype=torch.int32, device=dev)
                data = torch.zeros(blocks * 256, dtype=torch.float32, device=dev)
                err = torch.zeros(1, dtype=torch.int32, device=dev)

                def launch():
                    flags.zero_()
                    err.zero_()
                    lib.fw_peak_grid_barrier(blocks, rounds, 200000, fence,
                                             ctypes.c_void_p(flags.data_ptr()),
                                             ctypes.c_void_p(data.data_ptr()),
                                             ctypes.c_void_p(err.data_ptr()),
                                             ctypes.c_void_p(stream.cuda_stream))
                per[rounds] = best(launch)
                if int(err.item()):
                    sys.exit("grid barrier: a poll gave up (grid not co-resident)")
            print(json.dumps({"peak": "grid-wide rendezvous in one kernel", "workgroups": blocks,
                              "device_fence": bool(fence),
                              "us_per_round": (per[101] - per[1]) / 100 * 1e6}), flush=True)


def source_hash(kernel):
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# dominant kernel: label in the JSON line, mangled-name fragment in counter files
KERNELS = {"gemv_kernel<gate/up>": ("gemv_gate_up", "gemv_kernelILi"),
           "gemm_mx_kernel<gate/up>": ("gemm_mx_gate_up", "gemm_mx_kernelILb1E"),
           "gemm_kernel<gate/up>": ("gemm_gate_up", "gemm_kernelILi"),
           "gemm_i8_kernel<gate/up>": ("gemm_i8_gate_up", "gemm_i8_kernelILi")}


def traffic_path(workload, kernel):
    return os.path.join(ROOT, "profiles", f"traffic_{KERNELS[kernel][0]}_{workload}.json")


def traffic(workload, roof):
    """HBM bytes per launch of the dominant kernel, from the committed
    FETCH_SIZE / WRITE_SIZE counter summary of this workload (scaled by the
    counters' reading of a plain copy of known size), or None when there is
    none or the kernel sources changed since it was taken."""
    p = traffic_path(workload, roof["kernel"])
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        t = json.load(fh)
    if t.get("source_sha") != source_hash(roof["kernel"]):
        return None
    return t["bytes_per_launch"]


def reduce_counters(a):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the dominant kernel (the
    routed experts' gate/up launch), averaged over its dispatches, each scaled
    by what the counter read for the --copy-mib negation kernel (which reads
    and writes exactly that many bytes).  Where the shared expert's gate/up
    launch is the same kernel (same weight format), every step dispatches the
    routed launch first and the shared one right after it, so the routed ones
    are every other dispatch in dispatch order."""
    import csv
    import glob
    cfg, T, _ = WORKLOADS[a.workload]
    desc = fw.make_desc(cfg.hidden, cfg.n_experts, cfg.top_k, cfg.ffn, cfg.shared_ffn,
                        cfg.act_dtype, cfg.router_dtype, cfg.expert_q, cfg.shared_q,
                        cfg.score, a.path, cfg.act_quant)
    path_gemv = fw.fw_moe_forward_path(desc, T) == fw.FW_PATH_GEMV
    kernel = "gemv_kernel<gate/up>" if path_gemv else "gemm_kernel<gate/up>"
    qi = {"q8_0": "0", "q4_0": "1", "q4_k": "2", "q6_k": "3", "mxfp4": "4"}[cfg.expert_q]
    # the profiler writes kernel names mangled or demangled: match either
    frags = (KERNELS[kernel][1] + qi + "ELb1E",
             KERNELS[kernel][1].replace("ILi", "<") + qi + ", true")
    if cfg.act_quant == "mxfp8":
        kernel = "gemm_mx_kernel<gate/up>"
        frags = (KERNELS[kernel][1], "gemm_mx_kernel<true>")
    if cfg.act_quant == "int8":
        kernel = "gemm_i8_kernel<gate/up>"
        frags = (KERNELS[kernel][1] + qi + "ELb1E", "gemm_i8_kernel<" + qi + ", true")

    both = cfg.shared_ffn > 0 and cfg.shared_q == cfg.expert_q

    def per_dispatch(d, counter, sub, routed_only=False):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r["Counter_Name"] == counter and any(f in r["Kernel_Name"] for f in sub):
                        key = (f, int(r["Dispatch_Id"]))
                        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        v = [vals[k] for k in sorted(vals)]
        return v[0::2] if routed_only and both else v

    fd, wd = a.reduce_counters
    kf = per_dispatch(fd, "FETCH_SIZE", frags, routed_only=True)
    kw = per_dispatch(wd, "WRITE_SIZE", frags, routed_only=True)
    cf = per_dispatch(fd, "FETCH_SIZE", ("neg_kernel",))
    cw = per_dispatch(wd, "WRITE_SIZE", ("neg_kernel",))
    if not (kf and kw and cf and cw):
        sys.exit("counter files lack the kernel or the calibration copy")
    copy_bytes = a.copy_mib << 20
    ff, wf = copy_bytes / (max(cf) * 1024), copy_bytes / (max(cw) * 1024)
    fetch = sum(kf) / len(kf) * 1024 * ff
    write = sum(kw) / len(kw) * 1024 * wf
    res = {"workload": a.workload, "kernel": kernel, "source_sha": source_hash(kernel),
           "dispatches": [len(kf), len(kw)], "fetch_kib_per_dispatch": sum(kf) / len(kf),
           "write_kib_per_dispatch": sum(kw) / len(kw), "copy_mib": a.copy_mib,
           "copy_fetch_kib": max(cf), "copy_write_kib": max(cw), "fetch_factor": ff,
           "write_factor": wf, "fetch_bytes_per_launch": fetch,
           "write_bytes_per_launch": write, "bytes_per_launch": fetch + write}
    with open(traffic_path(a.workload, kernel), "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, L, x, T, seconds):
    """The CPU oracle (route + forward) on a bounded sample of the batch's
    tokens: consecutive 16-token slices of the same batch, routed and run
    through the layer, for about `seconds` on all host cores; then a few
    tokens on one core.  Tokens are independent, so tokens/s of the sample is
    the oracle's rate on the workload."""
    from oracle import fwref
    h = moegen.as_numpy_bits
    xh, wr, bias = h(x), h(L.router), h(L.bias)
    wg, wu, wd = h(L.w_gate), h(L.w_up), h(L.w_down)
    sg, su, sd = h(L.s_gate), h(L.s_up), h(L.s_down)

    def run(tok, threads):
        xs = np.ascontiguousarray(xh[tok])
        _, ids, w = fwref.route(xs, wr, bias, k=cfg.top_k, act_dtype=cfg.act_dtype,
                                router_dtype=cfg.router_dtype, score=cfg.score)
        fwref.forward(xs, wg, wu, wd, ids, w, n_experts=cfg.n_experts, ffn=cfg.ffn,
                      qtype=cfg.expert_q, act_dtype=cfg.act_dtype, s_gate=sg, s_up=su,
                      s_down=sd, shared_ffn=cfg.shared_ffn, shared_q=cfg.shared_q,
                      n_threads=threads, act_quant=cfg.act_quant)

    threads = fwref.threads(0)
    chunk = min(T, 16)
    n = 0
    t0 = time.perf_counter()
    while True:
        lo = (n * chunk) % T
        run(np.arange(lo, min(lo + chunk, T)), 0)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    tokens = n * chunk if T >= chunk else n * T
    one = min(T, 2)
    t1 = time.perf_counter()
    run(np.arange(one), 1)
    el1 = time.perf_counter() - t1
    return {"value": tokens / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} slices of {chunk} consecutive tokens of the {T}-token batch "
                      f"({tokens} tokens, route + forward, {el:.1f} s)",
            "cpu_model": cpu_model(),
            "one_core": {"value": one / el1, "unit": "tokens/s",
                         "sample": f"tokens 0..{one - 1}, route + forward ({el1:.1f} s)"}}


if __name__ == "__main__":
    main()
