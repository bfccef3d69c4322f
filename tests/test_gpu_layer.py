"""GPU parity of the three C-ABI calls against the CPU oracle, on the seeded
workloads (all five, at their full sizes).  Outputs are compared on every row
up to 2048 tokens; larger batches compare a sample that holds both ends, 48
random tokens and, for every expert, the token of its last routed row (its
last, partial GEMM tile), which the oracle computes one by one."""

import numpy as np
import pytest
import torch

import moegen
from sparse_moe_block_amd import fwmoe as fw
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

C = moegen
SWEEP_Z = C.SWEEP_Q8.with_(zipf=1.3)
SWEEP_Q4_Z = C.SWEEP_Q4.with_(zipf=1.3)
# (config, T): every batch size each workload names; the sweep layer (Q8_0 and
# Q4_0 experts, uniform and Zipf(1.3) routing) at a spread of T around its
# decode-to-prefill crossover (32 / 48 tokens) and at both ends of its range
CASES = [(C.TINY, 4), (C.QWEN3_DECODE, 1), (C.QWEN3_DECODE, 4), (C.QWEN3_DECODE, 16),
         (C.QWEN3_PREFILL, 2048), (C.DEEPSEEK, 1), (C.DEEPSEEK, 32), (C.DEEPSEEK, 4096),
         (C.SWEEP_Q8, 1), (C.SWEEP_Q8, 64), (C.SWEEP_Q8, 1024), (C.SWEEP_Q8, 8192),
         (SWEEP_Z, 8192)]
CASES += [(cfg, T) for cfg in (C.SWEEP_Q4, SWEEP_Q4_Z) for T in (1, 32, 48, 1024, 8192)]
IDS = [f"c{c.cid}{'' if c.cid != 4 else '-' + c.expert_q}{'z' if c.zipf and c.cid == 4 else ''}"
       f"-T{T}" for c, T in CASES]


def _x(cfg, T):
    x = moegen.make_x(cfg, T, device=G.DEV)
    return x, moegen.as_numpy_bits(x)


@pytest.mark.parametrize("cfg,T", CASES, ids=IDS)
def test_route(ref, cfg, T):
    print(f"route {cfg.name} T={T}", flush=True)
    dl = G.layer(cfg)
    desc = G.desc_of(cfg)
    x, xh = _x(cfg, T)
    logits, ids, w = G.route(desc, cfg, dl, x)
    rl, rids, rw = G.oracle_route(ref, cfg, dl, xh)
    gl = logits.cpu().numpy()
    assert np.abs(gl - rl).max() <= G.LOGIT_MAX_ABS
    # near ties: the oracle's logits are fed in for those tokens, then ids must
    # agree exactly everywhere
    near = G.small_gaps(rl, cfg.top_k)
    lin = gl.copy()
    lin[near] = rl[near]
    lin_d = torch.from_numpy(lin).to(G.DEV)
    _, ids2, w2 = G.route(desc, cfg, dl, x, logits_in=lin_d)
    assert np.array_equal(ids2.cpu().numpy(), rids)
    _, rids2, rw2 = G.oracle_route(ref, cfg, dl, xh, logits_in=lin)
    assert np.array_equal(rids2, rids)
    assert np.abs(w2.cpu().numpy() - rw2).max() <= G.W_MAX_ABS
    s = w2.double().sum(dim=1).cpu().numpy()
    assert np.abs(s - 1).max() <= 1e-5
    # tokens without near ties were routed identically from the GPU's own logits
    assert np.array_equal(ids.cpu().numpy()[~near], rids[~near])


@pytest.mark.parametrize("cfg,T", CASES, ids=IDS)
def test_permute(ref, cfg, T):
    print(f"permute {cfg.name} T={T}", flush=True)
    dl = G.layer(cfg)
    desc = G.desc_of(cfg)
    x, xh = _x(cfg, T)
    _, rids, _ = G.oracle_route(ref, cfg, dl, xh)
    ws = G.workspace(desc, T)
    off, sp, inv = G.permute(desc, cfg, torch.from_numpy(rids).to(G.DEV), ws)
    roff, rsp, rinv = ref.permute(rids, cfg.n_experts)
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(sp.cpu().numpy(), rsp)
    assert np.array_equal(inv.cpu().numpy(), rinv)
    assert fw.fw_moe_read_status(ws) == 0


@pytest.mark.parametrize("path", ["gemv", "gemm"])
@pytest.mark.parametrize("cfg,T", CASES, ids=IDS)
def test_forward(ref, cfg, T, path):
    """Oracle routing in, GPU permutation + expert FFNs + combine out."""
    print(f"forward {cfg.name} T={T} {path}", flush=True)
    dl = G.layer(cfg)
    desc = G.desc_of(cfg, path=path)
    x, xh = _x(cfg, T)
    _, rids, rw = G.oracle_route(ref, cfg, dl, xh)
    ws = G.workspace(desc, T)
    ids_d = torch.from_numpy(rids).to(G.DEV)
    w_d = torch.from_numpy(rw).to(G.DEV)
    off, sp, inv = G.permute(desc, cfg, ids_d, ws)
    out = G.forward(desc, cfg, dl, x, w_d, off, sp, inv, ws).cpu().numpy()
    assert fw.fw_moe_read_status(ws) == 0
    tok = G.compare_tokens(T, rids, cfg.n_experts)
    want = G.oracle_forward(ref, cfg, dl, np.ascontiguousarray(xh[tok]), rids[tok], rw[tok])
    G.check_out(out[tok], want)


@pytest.mark.parametrize("cfg,T", [(C.QWEN3_DECODE, 16), (C.DEEPSEEK, 32), (C.TINY, 4),
                                   (C.QWEN3_PREFILL, 2048)],
                         ids=["c1-T16", "c3-T32", "c0-T4", "c2-T2048"])
def test_end_to_end(ref, cfg, T):
    """route -> permute -> forward on the GPU against the oracle's route +
    forward (near-tie tokens take the oracle's logits)."""
    dl = G.layer(cfg)
    desc = G.desc_of(cfg)
    x, xh = _x(cfg, T)
    logits, _, _ = G.route(desc, cfg, dl, x)
    rl, rids, rw = G.oracle_route(ref, cfg, dl, xh)
    near = G.small_gaps(rl, cfg.top_k)
    lin = logits.cpu().numpy()
    lin[near] = rl[near]
    _, ids, w = G.route(desc, cfg, dl, x, logits_in=torch.from_numpy(lin).to(G.DEV))
    ws = G.workspace(desc, T)
    off, sp, inv = G.permute(desc, cfg, ids, ws)
    out = G.forward(desc, cfg, dl, x, w, off, sp, inv, ws).cpu().numpy()
    assert fw.fw_moe_read_status(ws) == 0
    tok = G.compare_tokens(T, rids, cfg.n_experts)
    want = G.oracle_forward(ref, cfg, dl, np.ascontiguousarray(xh[tok]), rids[tok], rw[tok])
    G.check_out(out[tok], want)


@pytest.mark.parametrize("path", ["gemv", "gemm"])
def test_repeat_is_bitwise_identical(path):
    cfg, T = C.DEEPSEEK, 32
    dl = G.layer(cfg)
    desc = G.desc_of(cfg, path=path)
    x, _ = _x(cfg, T)
    outs = []
    for _ in range(3):
        _, ids, w = G.route(desc, cfg, dl, x)
        ws = G.workspace(desc, T)
        off, sp, inv = G.permute(desc, cfg, ids, ws)
        outs.append(G.forward(desc, cfg, dl, x, w, off, sp, inv, ws).cpu())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("E,k", [(8, 2), (64, 4), (128, 8), (256, 8), (512, 16), (100, 16)])
def test_route_ties_and_signed_zeros(ref, E, k):
    """Selection from logits with many exact ties (a handful of distinct values,
    +0 and -0 among them): ids must equal the oracle's (descending, ties to the
    lower index, -0 == +0) and the weights must agree."""
    T = 37
    rng = np.random.default_rng(E * 100 + k)
    vals = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 1.0, 2.0, -3.0],
                    dtype=np.float32)
    lin = vals[rng.integers(0, len(vals), size=(T, E))]
    lin[0] = 0.0
    lin[1] = -0.0
    lin[2, ::2] = -0.0        # alternate signed zeros
    for score in ("softmax", "sigmoid"):
        desc = fw.make_desc(256, E, k, 256, score=score)
        ids = torch.full((T, k), -7, dtype=torch.int32, device=G.DEV)
        w = torch.full((T, k), float("nan"), device=G.DEV)
        fw.fw_moe_route(desc, T, None, None, None, torch.from_numpy(lin).to(G.DEV), None, ids, w)
        x_dummy = np.zeros((T, 256), np.uint16)
        r_dummy = np.zeros((E, 256), np.uint16)
        _, rids, rw = ref.route(x_dummy, r_dummy, None, k=k, act_dtype="bf16",
                                router_dtype="bf16", score=score, logits_in=lin)
        assert np.array_equal(ids.cpu().numpy(), rids), score
        assert np.abs(w.cpu().numpy() - rw).max() <= G.W_MAX_ABS, score
