"""GPU parity of the int8-activation mode (Q8_0 / Q4_0 experts on the int8
MFMA) against the oracle's int8 mode: the staged int8 codes and fp32 scales of
x bit for bit, the SwiGLU output's codes (a code may sit one step off where
the exact value is within rounding distance of a half-integer, since the two
sides accumulate g and u in a different order), and the layer output at the
layer's tolerances on every config's shapes, ragged tiles and the DeepSeek
batch that bench.py times.  The mode's refusals are CPU tests (test_abi.py)."""

import numpy as np
import pytest
import torch

import moegen
from sparse_moe_block_amd import fwmoe as fw
from tests import gpu_util as G
from tests import np_ref

pytestmark = pytest.mark.gpu

C = moegen
I8 = dict(act_quant="int8")
TINY = C.TINY.with_(**I8)
Q_DEC = C.QWEN3_DECODE.with_(**I8)
Q_PRE = C.QWEN3_PREFILL.with_(**I8)
DS = C.DEEPSEEK.with_(**I8)
SW8 = C.SWEEP_Q8.with_(zipf=1.3, **I8)
SW4 = C.SWEEP_Q4.with_(**I8)
CASES = [(TINY, 4), (Q_DEC, 1), (Q_DEC, 16), (Q_DEC, 33), (Q_PRE, 2048), (DS, 1), (DS, 300),
         (DS, 4096), (SW8, 1000), (SW4, 4096)]
IDS = [f"c{c.cid}-{c.expert_q}-T{T}" for c, T in CASES]


# Output tolerances of the mode.  The two sides reach the SwiGLU output by
# different accumulation orders (fp32 fma over int32 block sums against the
# oracle's fp64), so an element that lies on an int8 rounding boundary of its
# block can take the neighbouring code (test_h_codes_valid checks that every
# differing code sits on a boundary).  One such flip moves h by one step d_h
# (the block's amax / 127) and the token's output row by d_h times a column of
# down weights times the slot's gate weight (at most 1): up to d_h * max |Wd|
# per element, a few 1e-3 on the sweep layer.  The criteria: relative L2 over
# the compared rows within the layer's 1e-3, and no element beyond the
# layer's 2e-3 plus two such steps (a wrong scale or code moves whole rows and
# blocks, far beyond both).
def down_max_abs(cfg, dl):
    """Largest |weight| of the routed and shared down matrices, from their
    fp16 block scales (|code| <= 127 for Q8_0, <= 8 for Q4_0)."""
    hh, m = dl.host, 0.0
    for q, raw in ((cfg.expert_q, hh["w_down"]), (cfg.shared_q, hh["s_down"])):
        if raw is None or raw.size == 0 or (raw is hh["s_down"] and cfg.shared_ffn == 0):
            continue
        bb = 34 if q == C.Q8_0 else 18
        d = raw.reshape(-1)[: raw.size // bb * bb].reshape(-1, bb)[:, :2].copy()
        d = np.abs(d.view(np.float16).astype(np.float64)).max()
        m = max(m, d * (127 if q == C.Q8_0 else 8))
    return m


def h_step_max(desc, cfg, ws, T):
    """Largest int8 step of the staged SwiGLU output (its fp32 block scales)."""
    P = T * cfg.top_k
    _, ho = fw.fw_moe_workspace_offsets(desc, T)
    n = P * cfg.ffn + T * cfg.shared_ffn
    raw = ws.cpu().numpy()
    return float(raw[ho + n:ho + n + n // 8].view(np.float32).max())


def check_int8(got, want, step):
    d = np.abs(got - want)
    err = float(d.max())
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    assert np.all(np.isfinite(got)), "non-finite output"
    bound = G.OUT_MAX_ABS + 2 * step
    assert rel <= G.OUT_REL_L2 and err <= bound, \
        f"max-abs {err:.3e} (bound {bound:.3e}) rel-L2 {rel:.3e}"
    return err, rel, int((d > G.OUT_MAX_ABS).sum())


def run(ref, cfg, T, seed_variant=0):
    dl = G.layer(cfg)
    desc = G.desc_of(cfg)
    assert fw.fw_moe_forward_path(desc, T) == fw.FW_PATH_GEMM
    x = moegen.make_x(cfg, T, device=G.DEV, variant=seed_variant)
    xh = moegen.as_numpy_bits(x)
    _, rids, rw = G.oracle_route(ref, cfg, dl, xh)
    ws = G.workspace(desc, T)
    off, sp, inv = G.permute(desc, cfg, torch.from_numpy(rids).to(G.DEV), ws)
    out = G.forward(desc, cfg, dl, x, torch.from_numpy(rw).to(G.DEV), off, sp, inv, ws)
    torch.cuda.synchronize()
    return dl, desc, x, xh, rids, rw, ws, out.cpu().numpy(), sp.cpu().numpy()


@pytest.mark.parametrize("cfg,T", CASES, ids=IDS)
def test_forward_int8(ref, cfg, T):
    print(f"forward int8 {cfg.name} {cfg.expert_q} T={T}", flush=True)
    dl, desc, x, xh, rids, rw, ws, out, _ = run(ref, cfg, T)
    assert fw.fw_moe_read_status(ws) == 0
    tok = G.compare_tokens(T, rids, cfg.n_experts, n_random=24)
    want = G.oracle_forward(ref, cfg, dl, np.ascontiguousarray(xh[tok]), rids[tok], rw[tok])
    step = h_step_max(desc, cfg, ws, T) * down_max_abs(cfg, dl)
    err, rel, n_big = check_int8(out[tok], want, step)
    print(f"  max-abs {err:.2e} rel-L2 {rel:.2e}; one h step moves y by up to {step:.2e}; "
          f"elements above {G.OUT_MAX_ABS}: {n_big}", flush=True)


@pytest.mark.parametrize("cfg,T", [(TINY, 4), (Q_PRE, 2048), (DS, 300)],
                         ids=["c0-T4", "c2-T2048", "c3-T300"])
def test_staged_x_bit_exact(ref, cfg, T):
    """The staging kernel's int8 codes and fp32 scales of every token row
    equal the oracle's quantiser on the same fp32 values."""
    dl, desc, x, xh, rids, rw, ws, out, _ = run(ref, cfg, T)
    xo, _ = fw.fw_moe_workspace_offsets(desc, T)
    H = cfg.hidden
    raw = ws.cpu().numpy()
    codes = raw[xo:xo + T * H].view(np.int8).reshape(T, H)
    scales = raw[xo + T * H:xo + T * H + T * H // 8].view(np.float32).reshape(T, H // 32)
    xf = np_ref.act(xh).astype(np.float32)
    for t in range(T):
        c, s = ref.q8a_quantize(xf[t])
        assert np.array_equal(scales[t], s), f"token {t}: scales"
        assert np.array_equal(codes[t], c), f"token {t}: codes"


# Bound on |g_gpu - g| relative to sum |w x|: per block the fp32 product of the
# two scales and the fma into the accumulator each round once (2^-24), over at
# most a few hundred blocks.
ACC_REL = 2.0 ** -14


@pytest.mark.parametrize("cfg,T", [(Q_DEC, 16), (DS, 8), (SW8, 64)],
                         ids=["c1-T16", "c3-T8", "c4-T64"])
def test_h_codes_valid(ref, cfg, T):
    """The gate/up kernel's int8 SwiGLU output against a float64 evaluation
    (x through the oracle's quantiser, g and u in float64, a rounded to fp32
    and quantised by the oracle's quantiser) on the routed rows.  With dg =
    ACC_REL * sum |w x| (du alike) the kernel's a may differ from the exact
    one by da = |silu'(g) u| dg + |silu(g)| du + dg du, so: a block's scale
    d (its largest |a| over 127, which moves in its last bits with the sums)
    must be within da / 127 of the exact one; with that d, a code may differ
    from the oracle's rounding of a / d only by one, with the exact a / d
    within da / d of the half-integer between the two codes; and under 1 % of
    the codes differ."""
    dl, desc, x, xh, rids, rw, ws, out, sp = run(ref, cfg, T)
    _, ho = fw.fw_moe_workspace_offsets(desc, T)
    H, F, k, E = cfg.hidden, cfg.ffn, cfg.top_k, cfg.n_experts
    P = T * k
    raw = ws.cpu().numpy()
    h8 = raw[ho:ho + P * F].view(np.int8).reshape(P, F)
    # the scales follow all codes (routed rows, then the shared expert's T rows)
    so = ho + P * F + T * cfg.shared_ffn
    hs = raw[so:so + P * F // 8].view(np.float32).reshape(P, F // 32)
    hh = dl.host
    cache = {}

    def gate_up(e):   # expert e's gate and up rows, decoded once
        if e not in cache:
            cache[e] = tuple(np_ref.matrix_rows(cfg.expert_q, hh[m], E * F, H, e * F, (e + 1) * F)
                             for m in ("w_gate", "w_up"))
        return cache[e]
    xf = np_ref.act(xh).astype(np.float32)
    n_diff = n_scale = 0
    for row in range(P):
        q = int(sp[row])                  # the pair at this expert-sorted row
        t, e = q // k, int(rids.reshape(-1)[q])
        xc, xs = ref.q8a_quantize(xf[t])
        xq = xc.astype(np.float64) * np.repeat(xs.astype(np.float64), 32)
        Wge, Wue = gate_up(e)
        g, u = Wge @ xq, Wue @ xq
        dg = ACC_REL * (np.abs(Wge) @ np.abs(xq))
        du = ACC_REL * (np.abs(Wue) @ np.abs(xq))
        sg = 1.0 / (1.0 + np.exp(-g))
        a64 = g * sg * u
        da = np.abs((sg + g * sg * (1 - sg)) * u) * dg + np.abs(g * sg) * du + dg * du
        c, sc = ref.q8a_quantize(a64.astype(np.float32))
        a32 = a64.astype(np.float32)
        for b in range(F // 32):
            blk = slice(32 * b, 32 * b + 32)
            i = int(np.argmax(np.abs(a64[blk])))
            amax = abs(float(a64[blk][i]))
            d = float(hs[row, b])
            # the kernel's scale is its own block maximum / 127: within the
            # accumulation bound of the exact one
            assert abs(d * 127 - amax) <= da[blk][i] + 2.0 ** -20 * amax, \
                f"row {row} block {b}: scale {d} vs exact amax {amax}"
            n_scale += int(hs[row, b] != sc[b])
            if d == 0.0:
                assert not h8[row, blk].any()
                continue
            # the codes: the oracle's rounding rule with the kernel's scale
            t = (a32[blk] / np.float32(d)).astype(np.float64)
            cref = np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -127, 127).astype(np.int64)
            got = h8[row, blk].astype(np.int64)
            bad = got != cref
            for j in np.where(bad)[0]:
                f = 32 * b + j
                lo, hi = sorted((int(got[j]), int(cref[j])))
                assert hi - lo == 1, f"row {row} feature {f}: codes {got[j]} vs {cref[j]}"
                y = float(a64[f]) / d
                assert abs(abs(y) - abs(lo + hi) / 2) <= da[f] / d + 2.0 ** -20 * abs(y), \
                    f"row {row} feature {f}: {y} is not at the boundary of {lo} and {hi}"
            n_diff += int(bad.sum())
    print(f"  h codes differing at a rounding boundary: {n_diff} of {P * F}; "
          f"blocks whose scale differs in its last bits: {n_scale} of {P * F // 32}", flush=True)
    assert n_diff <= P * F // 100


# Descriptor extremes (the edge-shape configs): the smallest hidden and ffn
# with 512 experts and top-16, the largest hidden with top-1 sigmoid routing,
# uneven step counts with k = E and a Q4_0 shared expert, one expert with
# fp32 activations.
def _edge_cases():
    from tests.test_gpu_edge_shapes import EDGE_MIN, EDGE_ONE, EDGE_RAGGED, EDGE_WIDE
    return [(c.with_(**I8), T) for c, Ts in [(EDGE_MIN, (1, 33)), (EDGE_WIDE, (1, 40)),
                                             (EDGE_RAGGED, (9, 70)), (EDGE_ONE, (3, 100))]
            for T in Ts]


EDGE = _edge_cases()


@pytest.mark.parametrize("cfg,T", EDGE, ids=[f"c{c.cid}-T{T}" for c, T in EDGE])
def test_edge_shapes_int8(ref, cfg, T):
    print(f"edge int8 {cfg.name} T={T}", flush=True)
    dl, desc, x, xh, rids, rw, ws, out, _ = run(ref, cfg, T)
    assert fw.fw_moe_read_status(ws) == 0
    want = G.oracle_forward(ref, cfg, dl, xh, rids, rw)
    step = h_step_max(desc, cfg, ws, T) * down_max_abs(cfg, dl)
    err, rel, n_big = check_int8(out, want, step)
    print(f"  max-abs {err:.2e} rel-L2 {rel:.2e}; elements above {G.OUT_MAX_ABS}: {n_big}",
          flush=True)
