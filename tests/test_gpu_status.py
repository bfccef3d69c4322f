"""Data-dependent errors of fw_moe_forward are reported, never faulted on:
host-written corrupt expert_offsets, sorted_pairs and inv_pos set the sticky
FW_STATUS_BAD_OFFSETS / FW_STATUS_BAD_PAIR bits, and nothing is written outside
the workspace (guard bytes on both sides stay intact).

Every index the kernels derive from these inputs stays in range by
construction: the schedule clamps each expert's segment to [0, P] and writes at
most max_tiles row tiles; the GEMV clamps the device-written chunk count to the
bound its launch (split-K slices, counters, partials) was sized for; the GEMM
clamps its tile count to its grid; a pair id outside [0, P) is replaced by row
0 and an inv_pos entry outside [0, P) is skipped."""

import numpy as np
import pytest
import torch

import moegen
from sparse_moe_block_amd import fwmoe as fw
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

C = moegen
GUARD = 1 << 16    # bytes on each side of the workspace (keeps 256-byte alignment)


def _guarded_workspace(desc, T):
    need = fw.fw_moe_workspace_size(desc, T)
    buf = torch.full((need + 2 * GUARD,), 0xA5, dtype=torch.uint8, device=G.DEV)
    ws = buf[GUARD:GUARD + need]
    assert ws.data_ptr() % 256 == 0
    fw.fw_moe_clear_status(ws)
    return buf, ws


def _guards_intact(buf, need):
    g = buf.cpu().numpy()
    return bool(np.all(g[:GUARD] == 0xA5) and np.all(g[GUARD + need:] == 0xA5))


def _run_forward(desc, cfg, dl, x, w, off, sp, inv):
    T = x.shape[0]
    buf, ws = _guarded_workspace(desc, T)
    out = torch.zeros((T, cfg.hidden), device=G.DEV)
    L = dl.L
    fw.fw_moe_forward(desc, T, x, L.w_gate, L.w_up, L.w_down, L.s_gate, L.s_up, L.s_down, w,
                      off, sp, inv, out, ws)
    torch.cuda.synchronize()
    status = fw.fw_moe_read_status(ws)
    return status, _guards_intact(buf, ws.numel()), out


def _routing(cfg, T, seed=1):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(cfg.n_experts, cfg.top_k, replace=False) for _ in range(T)])
    w = np.full((T, cfg.top_k), 1.0 / cfg.top_k, np.float32)
    return ids.astype(np.int32), w


# DeepSeek-shaped layer (7168 hidden, 256 experts).  Top-1 at T = 1: one
# routed pair, 32 GEMV items, so the GEMV splits the reduction (7 slices) and
# sizes its arrival counters and partials for one row chunk, while the
# corrupt offsets below make the device schedule 128 chunks.  Top-8 at T = 8
# and 32 on the GEMV and at T = 32 on the grouped GEMM.
TOP1 = C.DEEPSEEK.with_(top_k=1, shared_ffn=0)


@pytest.mark.parametrize("cfg,T,path", [(TOP1, 1, "gemv"), (C.DEEPSEEK, 8, "gemv"),
                                        (C.DEEPSEEK, 32, "gemv"), (C.DEEPSEEK, 32, "gemm")],
                         ids=["top1-T1-gemv", "T8-gemv", "T32-gemv", "T32-gemm"])
def test_bad_offsets_flagged_and_contained(ref, cfg, T, path):
    print(f"bad offsets {cfg.name} k={cfg.top_k} T={T} {path}", flush=True)
    dl = G.layer(cfg)
    desc = G.desc_of(cfg, path=path)
    x = moegen.make_x(cfg, T, device=G.DEV)
    ids, w = _routing(cfg, T)
    P = T * cfg.top_k
    roff, rsp, rinv = ref.permute(ids, cfg.n_experts)
    # non-monotone offsets: every even expert claims [0, 1), every odd one
    # [1, 0) -- many more row tiles than P pairs can make
    off = np.array([0 if e % 2 == 0 else 1 for e in range(cfg.n_experts + 1)], np.int32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(G.DEV)
    status, intact, out = _run_forward(desc, cfg, dl, x, d(w), d(off), d(rsp), d(rinv))
    assert status & fw.FW_STATUS_BAD_OFFSETS
    assert intact, "bytes outside the workspace were written"
    # offsets past P and a negative start
    off2 = roff.copy()
    off2[1] = -5
    off2[cfg.n_experts // 2] = P + 100
    status, intact, _ = _run_forward(desc, cfg, dl, x, d(w), d(off2), d(rsp), d(rinv))
    assert status & fw.FW_STATUS_BAD_OFFSETS
    assert intact
    # the same call with the valid offsets is clean
    status, intact, _ = _run_forward(desc, cfg, dl, x, d(w), d(roff), d(rsp), d(rinv))
    assert status == 0 and intact


@pytest.mark.parametrize("path", ["gemv", "gemm"])
def test_bad_pairs_flagged_and_contained(ref, path):
    print(f"bad pairs qwen3 T=16 {path}", flush=True)
    cfg, T = C.QWEN3_DECODE, 16
    dl = G.layer(cfg)
    desc = G.desc_of(cfg, path=path)
    x = moegen.make_x(cfg, T, device=G.DEV)
    xh = moegen.as_numpy_bits(x)
    ids, w = _routing(cfg, T, seed=2)
    P = T * cfg.top_k
    roff, rsp, rinv = ref.permute(ids, cfg.n_experts)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(G.DEV)
    sp = rsp.copy()
    sp[3], sp[P - 1] = -3, P + 5        # pair ids outside [0, P)
    status, intact, _ = _run_forward(desc, cfg, dl, x, d(w), d(roff), d(sp), d(rinv))
    assert status & fw.FW_STATUS_BAD_PAIR
    assert (status & fw.FW_STATUS_BAD_OFFSETS) == 0
    assert intact
    inv = rinv.copy()
    bad_t = 5
    inv[bad_t * cfg.top_k + 1] = P + 7  # a slot that points nowhere: skipped in the combine
    status, intact, out = _run_forward(desc, cfg, dl, x, d(w), d(roff), d(rsp), d(inv))
    assert status & fw.FW_STATUS_BAD_PAIR
    assert intact
    # the other tokens are untouched by the bad slot
    ok = np.array([t for t in range(T) if t != bad_t])
    want = G.oracle_forward(ref, cfg, dl, np.ascontiguousarray(xh[ok]), ids[ok], w[ok])
    G.check_out(out.cpu().numpy()[ok], want)


MX8 = C.QWEN3_DECODE.with_(expert_q=C.MXFP4, act_quant="mxfp8")


def test_mx8_bad_offsets_and_pairs_flagged_and_contained(ref):
    """The block-scaled kernels share the grouped GEMM's tile list and its
    clamps: corrupt offsets and pair ids are flagged and contained."""
    cfg, T = MX8, 16
    print(f"bad offsets and pairs, mxfp8 mode, T={T}", flush=True)
    dl = G.layer(cfg, C.MXFP4)
    desc = G.desc_of(cfg)
    x = moegen.make_x(cfg, T, device=G.DEV)
    ids, w = _routing(cfg, T, seed=3)
    P = T * cfg.top_k
    roff, rsp, rinv = ref.permute(ids, cfg.n_experts)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(G.DEV)
    off = np.array([0 if e % 2 == 0 else 1 for e in range(cfg.n_experts + 1)], np.int32)
    status, intact, _ = _run_forward(desc, cfg, dl, x, d(w), d(off), d(rsp), d(rinv))
    assert status & fw.FW_STATUS_BAD_OFFSETS
    assert intact, "bytes outside the workspace were written"
    sp = rsp.copy()
    sp[3], sp[P - 1] = -3, P + 5
    status, intact, _ = _run_forward(desc, cfg, dl, x, d(w), d(roff), d(sp), d(rinv))
    assert status & fw.FW_STATUS_BAD_PAIR
    assert (status & fw.FW_STATUS_BAD_OFFSETS) == 0
    assert intact
    status, intact, _ = _run_forward(desc, cfg, dl, x, d(w), d(roff), d(rsp), d(rinv))
    assert status == 0 and intact


I8 = C.QWEN3_DECODE.with_(act_quant="int8")


def test_int8_bad_offsets_and_pairs_flagged_and_contained(ref):
    """The int8 kernels share the grouped GEMM's tile list and its clamps:
    corrupt offsets and pair ids are flagged and contained."""
    cfg, T = I8, 16
    print(f"bad offsets and pairs, int8 mode, T={T}", flush=True)
    dl = G.layer(cfg)
    desc = G.desc_of(cfg)
    x = moegen.make_x(cfg, T, device=G.DEV)
    ids, w = _routing(cfg, T, seed=5)
    P = T * cfg.top_k
    roff, rsp, rinv = ref.permute(ids, cfg.n_experts)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(G.DEV)
    off = np.array([0 if e % 2 == 0 else 1 for e in range(cfg.n_experts + 1)], np.int32)
    status, intact, _ = _run_forward(desc, cfg, dl, x, d(w), d(off), d(rsp), d(rinv))
    assert status & fw.FW_STATUS_BAD_OFFSETS
    assert intact, "bytes outside the workspace were written"
    sp = rsp.copy()
    sp[3], sp[P - 1] = -3, P + 5
    status, intact, _ = _run_forward(desc, cfg, dl, x, d(w), d(roff), d(sp), d(rinv))
    assert status & fw.FW_STATUS_BAD_PAIR
    assert (status & fw.FW_STATUS_BAD_OFFSETS) == 0
    assert intact
    status, intact, _ = _run_forward(desc, cfg, dl, x, d(w), d(roff), d(rsp), d(rinv))
    assert status == 0 and intact
