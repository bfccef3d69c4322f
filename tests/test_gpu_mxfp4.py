"""GPU parity of the layer on MXFP4 experts (MLX packing, group 32: E2M1
codes, then E8M0 scales) against
the CPU oracle: both kernel families, the decode and prefill shapes, the
DeepSeek shape with a Q8_0 and with an MXFP4 shared expert, and a skewed sweep.
Scale rows of 24 bytes (Qwen3 down, K = 768) put half the units' scales 8 bytes
into their 16-byte piece."""

import numpy as np
import pytest
import torch

import moegen
from sparse_moe_block_amd import fwmoe as fw
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

C = moegen
DS_K = C.DEEPSEEK.with_(shared_q=C.MXFP4)
SWEEP_KZ = C.SWEEP_Q8.with_(zipf=1.3)
CASES = [(C.QWEN3_DECODE, 1, "gemv"), (C.QWEN3_DECODE, 16, "gemv"),
         (C.QWEN3_DECODE, 16, "gemm"), (C.QWEN3_PREFILL, 2048, "auto"),
         (C.DEEPSEEK, 32, "gemv"), (C.DEEPSEEK, 32, "gemm"), (DS_K, 1, "gemv"),
         (DS_K, 300, "gemm"), (SWEEP_KZ, 64, "gemv"), (SWEEP_KZ, 1000, "gemm")]
IDS = [f"c{c.cid}{'-sk' if c.shared_q == C.MXFP4 and c.shared_ffn else ''}"
       f"{'z' if c.cid == 4 else ''}-T{T}-{p}" for c, T, p in CASES]


@pytest.mark.parametrize("cfg,T,path", CASES, ids=IDS)
def test_forward_mxfp4(ref, cfg, T, path):
    print(f"forward mxfp4 {cfg.name} T={T} {path}", flush=True)
    dl = G.layer(cfg, C.MXFP4)
    desc = G.desc_of(cfg, path=path, qtype=C.MXFP4)
    x = moegen.make_x(cfg, T, device=G.DEV)
    xh = moegen.as_numpy_bits(x)
    _, rids, rw = G.oracle_route(ref, cfg, dl, xh)
    ws = G.workspace(desc, T)
    ids_d = torch.from_numpy(rids).to(G.DEV)
    w_d = torch.from_numpy(rw).to(G.DEV)
    off, sp, inv = G.permute(desc, cfg, ids_d, ws)
    out = G.forward(desc, cfg, dl, x, w_d, off, sp, inv, ws).cpu().numpy()
    assert fw.fw_moe_read_status(ws) == 0
    tok = G.compare_tokens(T, rids, cfg.n_experts, n_random=24)
    want = G.oracle_forward(ref, cfg, dl, np.ascontiguousarray(xh[tok]), rids[tok], rw[tok])
    err, rel = G.check_out(out[tok], want)
    print(f"  max-abs {err:.2e} rel-L2 {rel:.2e}", flush=True)


def test_mxfp4_families_agree(ref):
    """The two kernel families on the same MXFP4 batch stay within the
    tolerance of each other (they round the weights differently)."""
    cfg, T = C.QWEN3_DECODE, 16
    dl = G.layer(cfg, C.MXFP4)
    x = moegen.make_x(cfg, T, device=G.DEV)
    xh = moegen.as_numpy_bits(x)
    _, rids, rw = G.oracle_route(ref, cfg, dl, xh)
    outs = []
    for path in ("gemv", "gemm"):
        desc = G.desc_of(cfg, path=path, qtype=C.MXFP4)
        ws = G.workspace(desc, T)
        off, sp, inv = G.permute(desc, cfg, torch.from_numpy(rids).to(G.DEV), ws)
        outs.append(G.forward(desc, cfg, dl, x, torch.from_numpy(rw).to(G.DEV), off, sp, inv,
                              ws).cpu().numpy())
    G.check_out(outs[0], outs[1].astype(np.float64))
