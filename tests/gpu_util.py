"""Helpers of the GPU parity tests: seeded layers on the device with host copies
for the oracle, and the three C-ABI calls with their buffers."""

import functools

import numpy as np
import torch

import moegen
from sparse_moe_block_amd import fwmoe as fw

DEV = torch.device("cuda:0")

# tolerances of the layer output against the oracle (max-abs, relative L2)
OUT_MAX_ABS = 2e-3
OUT_REL_L2 = 1e-3
LOGIT_MAX_ABS = 1e-4   # router logits (fp32 sums of exact bf16 products)
W_MAX_ABS = 1e-5       # renormalised gate weights
GAP = 1e-3             # below this k-th/(k+1)-th logit gap the oracle's logits are fed in


def desc_of(cfg, path="auto", qtype=None):
    return fw.make_desc(cfg.hidden, cfg.n_experts, cfg.top_k, cfg.ffn, cfg.shared_ffn,
                        cfg.act_dtype, cfg.router_dtype, qtype or cfg.expert_q, cfg.shared_q,
                        cfg.score, path, cfg.act_quant)


class DevLayer:
    """A generated layer on the GPU plus lazily made host copies."""

    def __init__(self, cfg, qtype=None):
        self.cfg = cfg
        self.qtype = qtype or cfg.expert_q
        self.L = moegen.make_layer(cfg, device=DEV, qtype=self.qtype)
        torch.cuda.synchronize()

    @functools.cached_property
    def host(self):
        h = moegen.as_numpy_bits
        L = self.L
        return dict(router=h(L.router), bias=h(L.bias), w_gate=h(L.w_gate), w_up=h(L.w_up),
                    w_down=h(L.w_down), s_gate=h(L.s_gate), s_up=h(L.s_up),
                    s_down=h(L.s_down))


@functools.lru_cache(maxsize=2)
def layer(cfg, qtype=None):
    return DevLayer(cfg, qtype)


def route(desc, cfg, dl, x, logits_in=None):
    T = x.shape[0]
    E, k = cfg.n_experts, cfg.top_k
    logits = torch.full((T, E), float("nan"), device=DEV)
    ids = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, k), float("nan"), device=DEV)
    fw.fw_moe_route(desc, T, x, dl.L.router, dl.L.bias, logits_in,
                    None if logits_in is not None else logits, ids, w)
    return logits, ids, w


def workspace(desc, T):
    n = fw.fw_moe_workspace_size(desc, T)
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    fw.fw_moe_clear_status(ws)
    return ws


def permute(desc, cfg, ids, ws):
    T = ids.shape[0]
    P = T * cfg.top_k
    off = torch.full((cfg.n_experts + 1,), -7, dtype=torch.int32, device=DEV)
    sp = torch.full((max(P, 1),), -7, dtype=torch.int32, device=DEV)
    inv = torch.full((max(P, 1),), -7, dtype=torch.int32, device=DEV)
    fw.fw_moe_permute(desc, T, ids, off, sp, inv, ws)
    return off, sp, inv


def forward(desc, cfg, dl, x, w, off, sp, inv, ws):
    T = x.shape[0]
    out = torch.full((T, cfg.hidden), float("nan"), device=DEV)
    L = dl.L
    fw.fw_moe_forward(desc, T, x, L.w_gate, L.w_up, L.w_down, L.s_gate, L.s_up, L.s_down, w,
                      off, sp, inv, out, ws)
    return out


def oracle_route(ref, cfg, dl, x_host, logits_in=None):
    hh = dl.host
    return ref.route(x_host, hh["router"], hh["bias"], k=cfg.top_k, act_dtype=cfg.act_dtype,
                     router_dtype=cfg.router_dtype, score=cfg.score, logits_in=logits_in)


def oracle_forward(ref, cfg, dl, x_host, ids, w):
    hh = dl.host
    return ref.forward(x_host, hh["w_gate"], hh["w_up"], hh["w_down"], ids, w,
                       n_experts=cfg.n_experts, ffn=cfg.ffn, qtype=dl.qtype,
                       act_dtype=cfg.act_dtype, s_gate=hh["s_gate"], s_up=hh["s_up"],
                       s_down=hh["s_down"], shared_ffn=cfg.shared_ffn, shared_q=cfg.shared_q,
                       act_quant=cfg.act_quant)


def small_gaps(logits, k):
    """Tokens whose k-th and (k+1)-th largest logits are closer than GAP."""
    if logits.shape[1] <= k:
        return np.zeros(logits.shape[0], bool)
    srt = -np.sort(-logits.astype(np.float64), axis=1)
    return (srt[:, k - 1] - srt[:, k]) < GAP


# Batches up to this many tokens are compared with the oracle on every row.
FULL_COMPARE_MAX_T = 2048


def compare_tokens(T, ids, n_experts, n_random=48, seed=0):
    """The tokens whose output rows are compared with the oracle: every token
    up to FULL_COMPARE_MAX_T; above that, both ends, n_random tokens drawn at
    random, and, for every expert, the token of its last routed row in the
    expert-sorted pair order -- a row of the expert's last (usually partial)
    row tile of the grouped GEMM and of its last GEMV row chunk.  Relative L2 is then
    computed over the rows of this sample."""
    if T <= FULL_COMPARE_MAX_T:
        return np.arange(T)
    k = ids.shape[1]
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")          # expert-major, ascending pair id
    counts = np.bincount(flat, minlength=n_experts)
    ends = np.cumsum(counts)
    last = [order[ends[e] - 1] // k for e in range(n_experts) if counts[e] > 0]
    rng = np.random.default_rng(seed + T)
    tok = np.concatenate([[0, T - 1], rng.choice(T, n_random, replace=False), last])
    return np.unique(tok)


def check_out(got, want):
    err = float(np.abs(got - want).max())
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    assert np.all(np.isfinite(got)), "non-finite output"
    assert err <= OUT_MAX_ABS and rel <= OUT_REL_L2, f"max-abs {err:.3e} rel-L2 {rel:.3e}"
    return err, rel
