"""fw_moe_layer_noalloc -- the layer with its workspace in the library's own
static device array, for callers that cannot allocate -- against fw_moe_layer
on the same inputs, bit for bit, on two calls in a row, the second with a
smaller batch (the array keeps the first call's contents)."""

import ctypes

import pytest
import torch

import moegen
from sparse_moe_block_amd import fwmoe as fw
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

C = moegen


def _bufs(cfg, T):
    E, k, P = cfg.n_experts, cfg.top_k, T * cfg.top_k
    return dict(logits=torch.full((T, E), float("nan"), device=G.DEV),
                ids=torch.full((T, k), -7, dtype=torch.int32, device=G.DEV),
                w=torch.full((T, k), float("nan"), device=G.DEV),
                off=torch.full((E + 1,), -7, dtype=torch.int32, device=G.DEV),
                sp=torch.full((P,), -7, dtype=torch.int32, device=G.DEV),
                inv=torch.full((P,), -7, dtype=torch.int32, device=G.DEV),
                out=torch.full((T, cfg.hidden), float("nan"), device=G.DEV))


def _with_workspace(desc, cfg, L, x):
    T = x.shape[0]
    b = _bufs(cfg, T)
    ws = G.workspace(desc, T)
    fw.fw_moe_layer(desc, T, x, L.router, L.bias, L.w_gate, L.w_up, L.w_down, L.s_gate, L.s_up,
                    L.s_down, b["logits"], b["ids"], b["w"], b["off"], b["sp"], b["inv"],
                    b["out"], ws)
    torch.cuda.synchronize()
    assert fw.fw_moe_read_status(ws) == 0
    return b


def _no_alloc(desc, cfg, L, x):
    T = x.shape[0]
    b = _bufs(cfg, T)
    status = torch.full((1,), -1, dtype=torch.int32, device=G.DEV)
    fw.fw_moe_layer_noalloc(desc, T, x, L.router, L.bias, L.w_gate, L.w_up, L.w_down,
                            L.s_gate, L.s_up, L.s_down, b["logits"], b["ids"], b["w"], b["off"],
                            b["sp"], b["inv"], b["out"], status)
    torch.cuda.synchronize()
    b["status"] = int(status.item())
    return b


# (config, first T, second T): decode batches of the DeepSeek-shaped layer
# (GEMV family, fused front end, shared expert, split-K at T = 1), a
# Qwen3-shaped batch on the grouped GEMM followed by a decode batch, and the
# MXFP8-activation mode (block-scaled GEMMs at every T), and the int8 one
MX8 = C.QWEN3_DECODE.with_(expert_q=C.MXFP4, act_quant="mxfp8")
I8 = C.QWEN3_DECODE.with_(act_quant="int8")


@pytest.mark.parametrize("cfg,T1,T2", [(C.DEEPSEEK, 32, 1), (C.QWEN3_DECODE, 256, 16),
                                       (MX8, 64, 4), (I8, 64, 4)],
                         ids=["deepseek-32-then-1", "qwen3-256-then-16", "qwen3-mx8-64-then-4",
                              "qwen3-int8-64-then-4"])
def test_noalloc_matches_workspace_call(cfg, T1, T2):
    print(f"no-alloc {cfg.name} T={T1} then T={T2}", flush=True)
    dl = G.layer(cfg)
    desc = G.desc_of(cfg)
    for T, v in ((T1, 1), (T2, 2)):
        x = moegen.make_x(cfg, T, device=G.DEV, variant=v)
        want = _with_workspace(desc, cfg, dl.L, x)
        got = _no_alloc(desc, cfg, dl.L, x)
        assert got["status"] == 0
        for name in ("logits", "ids", "w", "off", "sp", "inv", "out"):
            assert torch.equal(got[name], want[name]), f"T={T}: {name} differs"


def test_noalloc_refuses_oversized_batches():
    """A batch whose workspace exceeds the static array is refused before
    anything is enqueued."""
    cfg = C.DEEPSEEK
    desc = G.desc_of(cfg)
    T = 4096
    assert fw.fw_moe_workspace_size(desc, T) > fw.FW_NOALLOC_SCRATCH_BYTES
    rc = fw.lib().fw_moe_layer_noalloc(ctypes.byref(desc), T, 16, 16, None, 16, 16, 16, 16, 16,
                                       16, 16, 16, 16, 16, 16, 16, 16, None, None)
    assert rc == fw.FW_EWORKSPACE
