"""GPU parity of the MXFP8-activation mode (MXFP4 experts on the block-scaled
MFMA) against the oracle's MXFP8 mode: the staged E4M3 codes and E8M0 scales
of x bit for bit, the SwiGLU output's codes (a code may sit one step off where
the fp32 value is within rounding distance of a decision boundary, since the
two sides accumulate g and u in a different order), and the layer output at
the layer's tolerances on the decode, prefill and DeepSeek shapes (with an
MXFP4 shared expert) and ragged tiles.  The mode's refusals are CPU tests
(test_abi.py)."""

import numpy as np
import pytest
import torch

import moegen
from sparse_moe_block_amd import fwmoe as fw
from tests import gpu_util as G
from tests import np_ref

pytestmark = pytest.mark.gpu

C = moegen
MX = dict(expert_q=C.MXFP4, act_quant="mxfp8")
Q_DEC = C.QWEN3_DECODE.with_(**MX)
Q_PRE = C.QWEN3_PREFILL.with_(**MX)
DS = C.DEEPSEEK.with_(shared_q=C.MXFP4, **MX)
SW = C.SWEEP_Q8.with_(zipf=1.3, **MX)
CASES = [(Q_DEC, 1), (Q_DEC, 16), (Q_DEC, 33), (Q_PRE, 2048), (DS, 1), (DS, 300),
         (SW, 1000), (SW, 4096)]
IDS = [f"c{c.cid}-T{T}" for c, T in CASES]


# Output tolerances of the mode.  The two sides reach the SwiGLU output by
# different accumulation orders (fp32 MFMA sums against the oracle's fp64), so
# an element that lies on an E4M3 rounding boundary can take the neighbouring
# code (test_h_codes_valid checks that every differing element sits on a
# boundary).  One such flip moves one h element by one E4M3 step (up to 2^-3
# of its magnitude, several units on the DeepSeek shape) and so the token's
# whole output row by that step times a column of down weights, ~1e-2 per
# element there; with H = 7168 most tokens have one.  The criteria: relative
# L2 over the compared rows within the layer's 1e-3, and no element beyond
# 5e-2 (a wrong scale or code moves whole blocks by orders of magnitude more).
MX8_OUT_REL_L2 = G.OUT_REL_L2
MX8_OUT_MAX_ABS = 5e-2


def check_mx8(got, want):
    d = np.abs(got - want)
    err = float(d.max())
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    assert np.all(np.isfinite(got)), "non-finite output"
    assert rel <= MX8_OUT_REL_L2 and err <= MX8_OUT_MAX_ABS, \
        f"max-abs {err:.3e} rel-L2 {rel:.3e}"
    return err, rel


def run(ref, cfg, T, seed_variant=0):
    dl = G.layer(cfg, C.MXFP4)
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
def test_forward_mx8(ref, cfg, T):
    print(f"forward mx8 {cfg.name} T={T}", flush=True)
    dl, desc, x, xh, rids, rw, ws, out, _ = run(ref, cfg, T)
    assert fw.fw_moe_read_status(ws) == 0
    tok = G.compare_tokens(T, rids, cfg.n_experts, n_random=24)
    want = G.oracle_forward(ref, cfg, dl, np.ascontiguousarray(xh[tok]), rids[tok], rw[tok])
    err, rel = check_mx8(out[tok], want)
    n_big = int((np.abs(out[tok] - want) > G.OUT_MAX_ABS).sum())
    print(f"  max-abs {err:.2e} rel-L2 {rel:.2e}; elements above {G.OUT_MAX_ABS}: {n_big}",
          flush=True)


def _same_codes(a, b):
    """E4M3 codes equal, +0 and -0 counted the same."""
    a, b = a.astype(np.int64), b.astype(np.int64)
    return (a == b) | (((a & 0x7F) == 0) & ((b & 0x7F) == 0))


@pytest.mark.parametrize("cfg,T", [(Q_DEC, 16), (Q_PRE, 2048), (DS, 300)],
                         ids=["c1-T16", "c2-T2048", "c3-T300"])
def test_staged_x_bit_exact(ref, cfg, T):
    """The staging kernel's E4M3 codes and E8M0 scales of every token row
    equal the oracle's quantiser on the same fp32 values."""
    dl, desc, x, xh, rids, rw, ws, out, _ = run(ref, cfg, T)
    xo, _ = fw.fw_moe_workspace_offsets(desc, T)
    H = cfg.hidden
    raw = ws.cpu().numpy()
    codes = raw[xo:xo + T * H].reshape(T, H)
    scales = raw[xo + T * H:xo + T * H + T * H // 32].reshape(T, H // 32)
    xf = np_ref.act(xh).astype(np.float32)
    for t in range(T):
        c, s = ref.mxfp8_quantize(xf[t])
        assert np.array_equal(scales[t], s), f"token {t}: scales"
        assert np.all(_same_codes(codes[t], c)), f"token {t}: codes"


# The block-scaled MFMA does not sum a 64-product slice exactly in fp32: on
# random E4M3 x E2M1 operands its error reaches ~1e-4 of the slice's sum of
# |products| (median ~3e-6).  The bound the checks below allow for g and u:
MFMA_REL = 2.0 ** -12


@pytest.mark.parametrize("cfg,T", [(Q_DEC, 16), (DS, 8)], ids=["c1-T16", "c3-T8"])
def test_h_codes_valid(ref, cfg, T):
    """The gate/up kernel's MXFP8 SwiGLU output against a float64 evaluation
    (x quantised by the exhaustive quantiser, g and u in float64, a rounded to
    fp32 and quantised by the oracle's quantiser) on the routed rows.  With
    dg = MFMA_REL * sum |w x| (du alike) the kernel's a may differ from the
    exact one by da = |silu'(g) u| dg + |silu(g)| du + dg du, so: a block's
    scale may differ only where its largest |a| is within da of a power of two
    (those blocks are skipped, and must be rare); a code may differ only by one
    E4M3 step, with the exact value within da of the boundary between the two
    codes; and under 1 % of the codes differ."""
    dl, desc, x, xh, rids, rw, ws, out, sp = run(ref, cfg, T)
    _, ho = fw.fw_moe_workspace_offsets(desc, T)
    H, F, k, E = cfg.hidden, cfg.ffn, cfg.top_k, cfg.n_experts
    P = T * k
    raw = ws.cpu().numpy()
    h8 = raw[ho:ho + P * F].reshape(P, F)
    # the scales follow all codes (routed rows, then the shared expert's T rows)
    so = ho + P * F + T * cfg.shared_ffn
    hs = raw[so:so + P * F // 32].reshape(P, F // 32)
    hh = dl.host
    cache = {}

    def gate_up(e):   # expert e's gate and up rows, decoded once
        if e not in cache:
            cache[e] = tuple(np_ref.matrix_rows("mxfp4", hh[m], E * F, H, e * F, (e + 1) * F)
                             for m in ("w_gate", "w_up"))
        return cache[e]
    xf = np_ref.act(xh).astype(np.float32)
    tab = np_ref.e4m3_table()
    finite = np.unique(tab[~np.isnan(tab)])   # sorted, +0 and -0 once
    n_diff = n_scale = 0
    for row in range(P):
        q = int(sp[row])                  # the pair at this expert-sorted row
        t, e = q // k, int(rids.reshape(-1)[q])
        xq = np_ref.mxfp8_round_trip(xf[t])
        Wge, Wue = gate_up(e)
        g, u = Wge @ xq, Wue @ xq
        dg = MFMA_REL * (np.abs(Wge) @ np.abs(xq))
        du = MFMA_REL * (np.abs(Wue) @ np.abs(xq))
        sg = 1.0 / (1.0 + np.exp(-g))
        a64 = g * sg * u
        da = np.abs((sg + g * sg * (1 - sg)) * u) * dg + np.abs(g * sg) * du + dg * du
        a = a64.astype(np.float32)
        c, sc = ref.mxfp8_quantize(a)
        for b in range(F // 32):
            blk = slice(32 * b, 32 * b + 32)
            if hs[row, b] != sc[b]:
                i = int(np.argmax(np.abs(a64[blk])))
                amax, tol = abs(a64[blk][i]), da[blk][i]
                edge = 2.0 ** np.round(np.log2(amax))
                assert abs(int(hs[row, b]) - int(sc[b])) == 1 and abs(amax - edge) <= tol, \
                    f"row {row} block {b}: scale {hs[row, b]} vs {sc[b]}, amax {amax}"
                n_scale += 1
                continue
            X = 2.0 ** (int(sc[b]) - 127)
            bad = ~_same_codes(h8[row, blk], c[blk])
            for j in np.where(bad)[0]:
                f = 32 * b + j
                v1, v2 = tab[h8[row, f]], tab[c[f]]
                lo, hi = min(v1, v2), max(v1, v2)
                assert np.searchsorted(finite, hi) - np.searchsorted(finite, lo) == 1, \
                    f"row {row} feature {f}: codes {h8[row, f]:#x} vs {c[f]:#x} not adjacent"
                y = float(a64[f]) / X
                assert abs(y - (lo + hi) / 2) <= da[f] / X + 2.0 ** -20 * abs(y), \
                    f"row {row} feature {f}: {y} is {abs(y - (lo + hi) / 2)} from the " \
                    f"boundary, beyond {da[f] / X}"
            n_diff += int(bad.sum())
    print(f"  h codes differing at a rounding boundary: {n_diff} of {P * F}; "
          f"blocks with a scale at a power-of-two edge: {n_scale} of {P * F // 32}", flush=True)
    assert n_diff <= P * F // 100 and n_scale <= P * F // 32 // 100
