"""fw_moe_layer -- the whole layer in one call, with the fused decode front end
(top-k + permutation + staging in one kernel) wherever the forward runs the
GEMV family -- against the three separate calls, bit for bit, and against the
CPU oracle."""

import numpy as np
import pytest
import torch

import moegen
from sparse_moe_block_amd import fwmoe as fw
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

C = moegen
CASES = [
    (C.TINY, 4, "auto"),
    (C.QWEN3_DECODE, 1, "auto"),
    (C.QWEN3_DECODE, 4, "auto"),
    (C.QWEN3_DECODE, 16, "auto"),
    (C.QWEN3_DECODE.with_(expert_q=C.Q4_K), 16, "auto"),   # staged block sums too
    (C.QWEN3_DECODE, 33, "auto"),      # just above the crossover: GEMM, unfused
    (C.QWEN3_DECODE, 256, "gemv"),     # 2048 pairs: the largest fused batch
    (C.QWEN3_DECODE, 257, "gemv"),     # 2056 pairs: multi-kernel permutation, unfused
    (C.SWEEP_Q8, 32, "auto"),
    (C.DEEPSEEK, 1, "auto"),           # shared expert; 256 experts (4 per lane)
    (C.DEEPSEEK, 32, "auto"),          # 7 staging blocks beside the front block
    (C.QWEN3_PREFILL, 2048, "auto"),   # the GEMM path through the one call
    (C.DEEPSEEK, 64, "auto"),          # 2 rows per expert: the last GEMV batch
    (C.DEEPSEEK, 65, "auto"),          # the first GEMM batch
    (C.DEEPSEEK, 4096, "auto"),
    # every expert format at the benchmark's decode and prefill shapes
    (C.QWEN3_DECODE.with_(expert_q=C.Q8_0), 16, "auto"),
    (C.QWEN3_PREFILL.with_(expert_q=C.Q8_0), 2048, "auto"),
    (C.QWEN3_PREFILL.with_(expert_q=C.Q4_K), 2048, "auto"),
    (C.QWEN3_DECODE.with_(expert_q=C.Q6_K), 16, "auto"),
    (C.QWEN3_PREFILL.with_(expert_q=C.Q6_K), 2048, "auto"),
    (C.QWEN3_DECODE.with_(expert_q=C.MXFP4), 16, "auto"),
    (C.QWEN3_PREFILL.with_(expert_q=C.MXFP4), 2048, "auto"),
    # MXFP8 activations on the block-scaled MFMA (the GEMM family at every T)
    (C.QWEN3_DECODE.with_(expert_q=C.MXFP4, act_quant="mxfp8"), 1, "auto"),
    (C.QWEN3_PREFILL.with_(expert_q=C.MXFP4, act_quant="mxfp8"), 2048, "auto"),
    (C.DEEPSEEK.with_(expert_q=C.MXFP4, shared_q=C.MXFP4, act_quant="mxfp8"), 64, "auto"),
    # int8 activations on the int8 MFMA (the GEMM family at every T)
    (C.QWEN3_DECODE.with_(act_quant="int8"), 4, "auto"),
    (C.QWEN3_PREFILL.with_(act_quant="int8"), 2048, "auto"),
    (C.DEEPSEEK.with_(act_quant="int8"), 64, "auto"),
]
AQ = {"none": "", "mxfp8": "-mx8", "int8": "-int8"}
IDS = [f"c{c.cid}-{c.expert_q}{AQ[c.act_quant]}-T{T}-{p}" for c, T, p in CASES]


def _three_calls(desc, cfg, dl, x):
    logits, ids, w = G.route(desc, cfg, dl, x)
    ws = G.workspace(desc, x.shape[0])
    off, sp, inv = G.permute(desc, cfg, ids, ws)
    out = G.forward(desc, cfg, dl, x, w, off, sp, inv, ws)
    assert fw.fw_moe_read_status(ws) == 0
    return logits, ids, w, off, sp, inv, out


def _one_call(desc, cfg, dl, x):
    T, E, k, P = x.shape[0], cfg.n_experts, cfg.top_k, x.shape[0] * cfg.top_k
    logits = torch.full((T, E), float("nan"), device=G.DEV)
    ids = torch.full((T, k), -7, dtype=torch.int32, device=G.DEV)
    w = torch.full((T, k), float("nan"), device=G.DEV)
    off = torch.full((E + 1,), -7, dtype=torch.int32, device=G.DEV)
    sp = torch.full((P,), -7, dtype=torch.int32, device=G.DEV)
    inv = torch.full((P,), -7, dtype=torch.int32, device=G.DEV)
    out = torch.full((T, cfg.hidden), float("nan"), device=G.DEV)
    ws = G.workspace(desc, T)
    L = dl.L
    fw.fw_moe_layer(desc, T, x, L.router, L.bias, L.w_gate, L.w_up, L.w_down, L.s_gate,
                    L.s_up, L.s_down, logits, ids, w, off, sp, inv, out, ws)
    assert fw.fw_moe_read_status(ws) == 0
    return logits, ids, w, off, sp, inv, out, ws


@pytest.mark.parametrize("cfg,T,path", CASES, ids=IDS)
def test_layer_matches_three_calls_and_oracle(ref, cfg, T, path):
    print(f"fw_moe_layer {cfg.name} q={cfg.expert_q} T={T} path={path}", flush=True)
    dl = G.layer(cfg)
    desc = G.desc_of(cfg, path=path)
    x = moegen.make_x(cfg, T, device=G.DEV)
    xh = moegen.as_numpy_bits(x)
    sep = _three_calls(desc, cfg, dl, x)
    one = _one_call(desc, cfg, dl, x)
    for name, a, b in zip(["logits", "ids", "w", "offsets", "sorted", "inv", "out"], sep, one):
        assert torch.equal(a, b), f"{name} differs from the three calls"
    # against the oracle: tokens without a near tie were routed as the oracle
    # routes them, and their outputs agree within the layer tolerance
    logits, ids, w, _, _, _, out = (t.cpu().numpy() for t in one[:7])
    rl, rids, rw = G.oracle_route(ref, cfg, dl, xh)
    assert np.abs(logits - rl).max() <= G.LOGIT_MAX_ABS
    ok = ~G.small_gaps(rl, cfg.top_k)
    assert np.array_equal(ids[ok], rids[ok])
    assert np.abs(w[ok] - rw[ok]).max() <= G.W_MAX_ABS
    tok = np.intersect1d(G.compare_tokens(T, rids, cfg.n_experts), np.nonzero(ok)[0])
    assert tok.size > 0
    want = G.oracle_forward(ref, cfg, dl, np.ascontiguousarray(xh[tok]), rids[tok], rw[tok])
    if cfg.act_quant == "mxfp8":
        from tests.test_gpu_mx8 import check_mx8
        check_mx8(out[tok], want)
    elif cfg.act_quant == "int8":
        from tests.test_gpu_int8 import check_int8, down_max_abs, h_step_max
        check_int8(out[tok], want, h_step_max(desc, cfg, one[7], T) * down_max_abs(cfg, dl))
    else:
        G.check_out(out[tok], want)
