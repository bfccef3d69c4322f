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

WORKLOADS = {
    # name: (config, T, weight copies)
    "decode16": (moegen.QWEN3_DECODE, 16, 16),
    "decode4": (moegen.QWEN3_DECODE, 4, 16),
    "decode1": (moegen.QWEN3_DECODE, 1, 16),
    "deepseek1": (moegen.DEEPSEEK, 1, 2),
    "deepseek32": (moegen.DEEPSEEK, 32, 2),
    "prefill2048": (moegen.QWEN3_PREFILL, 2048, 4),
    "deepseek4096": (moegen.DEEPSEEK, 4096, 1),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode16", choices=sorted(WORKLOADS))
    ap.add_argument("--path", default="auto", choices=["auto", "gemv", "gemm"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (the "
                         "reference kernel that scales hardware byte counters)")
    return ap.parse_args()


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {a.gpus} is not supported "
              f"(the layer is measured on one MI355X)", file=sys.stderr)
        sys.exit(2)
    cfg, T, copies = WORKLOADS[a.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = moegen.make_layer(cfg, device=dev)
    x = moegen.make_x(cfg, T, device=dev)
    layers = [L]
    for _ in range(copies - 1):
        layers.append(moegen.Layer(cfg, L.router, L.bias, L.w_gate.clone(), L.w_up.clone(),
                                   L.w_down.clone(),
                                   *(None if t is None else t.clone()
                                     for t in (L.s_gate, L.s_up, L.s_down))))
    desc = fw.make_desc(cfg.hidden, cfg.n_experts, cfg.top_k, cfg.ffn, cfg.shared_ffn,
                        cfg.act_dtype, cfg.router_dtype, cfg.expert_q, cfg.shared_q,
                        cfg.score, a.path)
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
    fw.fw_moe_clear_status(ws)
    stream = torch.cuda.current_stream()

    def step(i):
        Li = layers[i % copies]
        fw.fw_moe_route(desc, T, x, Li.router, Li.bias, None, logits, ids, w, stream)
        fw.fw_moe_permute(desc, T, ids, off, sp, inv, ws, stream=stream)
        fw.fw_moe_forward(desc, T, x, Li.w_gate, Li.w_up, Li.w_down, Li.s_gate, Li.s_up,
                          Li.s_down, w, off, sp, inv, out, ws, stream=stream)

    if a.copy_mib:
        src = torch.empty(a.copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    assert fw.fw_moe_read_status(ws) == 0
    n_active = int((torch.diff(off) > 0).sum())

    # per-step stage events (HIP events recorded by the library on `stream`)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(fw.FW_N_STAGE_EVENTS)]
           for _ in range(a.steps)]
    for e in evs:
        fw.fw_moe_set_stage_events(e)   # creates the events
    fw.fw_moe_set_stage_events(None)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(a.steps):
        fw.fw_moe_set_stage_events(evs[i])
        step(a.warmup + i)
    t1.record(stream)
    torch.cuda.synchronize()
    fw.fw_moe_set_stage_events(None)
    ms = t0.elapsed_time(t1) / a.steps
    stage_ms = np.array([[e[s].elapsed_time(e[s + 1]) for s in range(4)] for e in evs])
    stage_avg = stage_ms.mean(axis=0)

    # dominant kernel: the gate/up projection (2/3 of the expert bytes and flops)
    path = fw.fw_moe_forward_path(desc, T)
    gu_ms = float(stage_avg[1])
    bq = moegen.BLOCK_BYTES[cfg.expert_q]
    if path == fw.FW_PATH_GEMV:
        # bytes: the active experts' gate and up rows, x in (bf16), a out
        gu_alg = n_active * 2 * cfg.ffn * (H // 32) * bq + T * H * 2 + P * cfg.ffn * 2
        if cfg.shared_ffn:
            gu_alg += 2 * cfg.shared_ffn * (H // 32) * moegen.BLOCK_BYTES[cfg.shared_q]
            gu_alg += T * cfg.shared_ffn * 2
        achieved = gu_alg / (gu_ms * 1e-3) / 1e9
        roof = {"kernel": "gemv_kernel<gate/up>", "bound": "hbm", "achieved": achieved,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                "traffic": None, "algorithmic_bytes": gu_alg}
    else:
        # flops: 2 projections x 2 flops x P x H x F (+ the shared expert on T rows)
        gu_alg = 4 * P * H * cfg.ffn + 4 * T * H * cfg.shared_ffn
        achieved = gu_alg / (gu_ms * 1e-3) / 1e12
        roof = {"kernel": "gemm_kernel<gate/up>", "bound": "mfma", "achieved": achieved,
                "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_FP16_PEAK_TFLOPS, "traffic": None,
                "algorithmic_flops": gu_alg}
    layer_bytes = (n_active * cfg.expert_bytes + cfg.shared_bytes + cfg.router_bytes +
                   cfg.act_bytes(T) + T * H * 4)
    layer_flops = 6 * P * H * cfg.ffn + 6 * T * H * cfg.shared_ffn + 2 * T * H * E

    line = {
        "metric": "MoE-layer tokens/s (" + ("decode; HBM-bound" if path == fw.FW_PATH_GEMV
                                             else "prefill; MFMA-bound") + ")",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4_0 weights, fp32 accumulate" if cfg.expert_q == "q4_0" else "q8_0 weights, fp32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights quantized to GGUF blocks, N(0,1) bf16 tokens)",
        "config": {"workload": f"{cfg.name}, T={T}", "hidden": H, "experts": E, "top_k": k,
                   "ffn": cfg.ffn, "expert_format": cfg.expert_q, "shared_ffn": cfg.shared_ffn,
                   "tokens": T, "active_experts": n_active, "weight_copies": copies,
                   "path": "gemv" if path == fw.FW_PATH_GEMV else "gemm"},
        "layer_GBps": layer_bytes / (ms * 1e-3) / 1e9,
        "layer_TFLOPs": layer_flops / (ms * 1e-3) / 1e12,
        "stage_us": {n: round(float(v) * 1e3, 2) for n, v in
                     zip(["prepare", "gate_up", "down", "combine"], stage_avg)},
        "roofline": roof,
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, L, x, T, a.cpu_seconds)
    print(json.dumps(line), flush=True)


def cpu_baseline(cfg, L, x, T, seconds):
    """The CPU oracle (route + forward) on the same batch, repeated for about
    `seconds`, on all host cores."""
    from oracle import fwref
    h = moegen.as_numpy_bits
    xh, wr, bias = h(x), h(L.router), h(L.bias)
    wg, wu, wd = h(L.w_gate), h(L.w_up), h(L.w_down)
    sg, su, sd = h(L.s_gate), h(L.s_up), h(L.s_down)
    threads = fwref.threads(0)
    n = 0
    t0 = time.perf_counter()
    while True:
        _, ids, w = fwref.route(xh, wr, bias, k=cfg.top_k, act_dtype=cfg.act_dtype,
                                router_dtype=cfg.router_dtype, score=cfg.score)
        fwref.forward(xh, wg, wu, wd, ids, w, n_experts=cfg.n_experts, ffn=cfg.ffn,
                      qtype=cfg.expert_q, act_dtype=cfg.act_dtype, s_gate=sg, s_up=su,
                      s_down=sd, shared_ffn=cfg.shared_ffn, shared_q=cfg.shared_q)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": n * T / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} passes of route+forward over the same {T}-token batch "
                      f"({el:.1f} s)"}


if __name__ == "__main__":
    main()
