"""Graph capture: route -> permute -> forward (three calls, or the one
fw_moe_layer call) captured once in a HIP graph and
replayed several times, with eager work and synchronisations between the
replays; every replay must equal the eager result bit for bit.  (The library
issues no memset and no allocation, so it captures as is; split-K counters and
the status word are cleared by kernels.)"""

import pytest
import torch

import moegen
from sparse_moe_block_amd import fwmoe as fw
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

C = moegen
MX8 = dict(expert_q=C.MXFP4, act_quant="mxfp8")
CASES = [(C.QWEN3_DECODE, 16, "auto"), (C.DEEPSEEK, 1, "auto"), (C.DEEPSEEK, 32, "auto"),
         (C.QWEN3_PREFILL, 256, "gemm"), (C.QWEN3_DECODE.with_(**MX8), 16, "auto"),
         (C.DEEPSEEK.with_(shared_q=C.MXFP4, **MX8), 32, "auto"),
         (C.QWEN3_DECODE.with_(act_quant="int8"), 16, "auto"),
         (C.DEEPSEEK.with_(act_quant="int8"), 32, "auto")]


@pytest.mark.parametrize("one_call", [False, True], ids=["three-calls", "fw_moe_layer"])
@pytest.mark.parametrize("cfg,T,path", CASES, ids=["c1-T16", "c3-T1", "c3-T32", "c2-T256-gemm",
                                                  "c1-mx8-T16", "c3-mx8-T32", "c1-int8-T16",
                                                  "c3-int8-T32"])
def test_graph_replays_equal_eager(cfg, T, path, one_call):
    print(f"graph {cfg.name} T={T} {path} one_call={one_call}", flush=True)
    dl = G.layer(cfg)
    L = dl.L
    desc = G.desc_of(cfg, path=path)
    E, k, H = cfg.n_experts, cfg.top_k, cfg.hidden
    x = moegen.make_x(cfg, T, device=G.DEV)
    x2 = moegen.make_x(cfg, T, device=G.DEV, variant=1)
    logits = torch.empty(T, E, device=G.DEV)
    ids = torch.empty(T, k, dtype=torch.int32, device=G.DEV)
    w = torch.empty(T, k, device=G.DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=G.DEV)
    sp = torch.empty(T * k, dtype=torch.int32, device=G.DEV)
    inv = torch.empty(T * k, dtype=torch.int32, device=G.DEV)
    out = torch.empty(T, H, device=G.DEV)
    ws = G.workspace(desc, T)

    def step(xin, s=None):
        if one_call:
            fw.fw_moe_layer(desc, T, xin, L.router, L.bias, L.w_gate, L.w_up, L.w_down,
                            L.s_gate, L.s_up, L.s_down, logits, ids, w, off, sp, inv, out, ws,
                            stream=s)
            return
        fw.fw_moe_route(desc, T, xin, L.router, L.bias, None, logits, ids, w, s)
        fw.fw_moe_permute(desc, T, ids, off, sp, inv, ws, stream=s)
        fw.fw_moe_forward(desc, T, xin, L.w_gate, L.w_up, L.w_down, L.s_gate, L.s_up,
                          L.s_down, w, off, sp, inv, out, ws, stream=s)

    step(x2)                      # warm (first launches set up per-device state)
    step(x)
    torch.cuda.synchronize()
    eager = out.clone()
    assert torch.isfinite(eager).all()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(x, torch.cuda.current_stream())
    for rep in range(3):
        step(x2)                  # eager work on other inputs between the replays
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager result"
    assert fw.fw_moe_read_status(ws) == 0
