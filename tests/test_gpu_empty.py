"""An empty batch (T = 0) through every entry point of the C ABI, for the
default, MXFP8-activation and int8-activation descriptors: every call returns
FW_OK; fw_moe_permute writes E + 1 zero offsets and nothing else; route,
forward and fw_moe_layer write nothing (sentinel buffers keep their fill);
the workspace status stays clear."""

import pytest
import torch

import moegen
from sparse_moe_block_amd import fwmoe as fw
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

C = moegen
CFGS = [C.QWEN3_DECODE, C.DEEPSEEK,
        C.QWEN3_DECODE.with_(expert_q=C.MXFP4, act_quant="mxfp8"),
        C.DEEPSEEK.with_(act_quant="int8")]
IDS = ["c1", "c3", "c1-mx8", "c3-int8"]


@pytest.mark.parametrize("cfg", CFGS, ids=IDS)
def test_empty_batch(cfg):
    print(f"empty batch {cfg.name} act_quant={cfg.act_quant}", flush=True)
    desc = G.desc_of(cfg)
    H, E, k = cfg.hidden, cfg.n_experts, cfg.top_k
    dev = G.DEV
    # the calls read nothing at T = 0: small stand-ins for x and the weights
    x = torch.zeros(16, H, dtype=torch.bfloat16, device=dev)
    wbuf = torch.zeros(4096, dtype=torch.uint8, device=dev)
    router = torch.zeros(E, H, dtype=torch.bfloat16, device=dev)
    sentinel = lambda *shape, dt=torch.float32: torch.full(shape, -7, dtype=dt, device=dev)
    logits, w, out = sentinel(1, E), sentinel(1, k), sentinel(1, H)
    ids, sp, inv = (sentinel(1, k, dt=torch.int32), sentinel(1, dt=torch.int32),
                    sentinel(1, dt=torch.int32))
    off = sentinel(E + 1, dt=torch.int32)
    ws = G.workspace(desc, 0)

    fw.fw_moe_route(desc, 0, x, router, None, None, logits, ids, w)
    fw.fw_moe_permute(desc, 0, ids, off, sp, inv, ws)
    torch.cuda.synchronize()
    assert torch.equal(off, torch.zeros_like(off)), "offsets of an empty batch"
    off_after_permute = off.clone()
    fw.fw_moe_forward(desc, 0, x, wbuf, wbuf, wbuf, wbuf, wbuf, wbuf, w, off, sp, inv, out, ws)
    fw.fw_moe_layer(desc, 0, x, router, None, wbuf, wbuf, wbuf, wbuf, wbuf, wbuf, logits, ids,
                    w, off, sp, inv, out, ws)
    torch.cuda.synchronize()
    for name, t in (("logits", logits), ("w", w), ("out", out), ("ids", ids), ("sorted", sp),
                    ("inv", inv)):
        assert bool((t == -7).all()), f"{name} was written"
    assert torch.equal(off, off_after_permute)
    assert fw.fw_moe_read_status(ws) == 0
