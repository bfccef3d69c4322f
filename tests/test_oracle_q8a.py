"""Pins of the oracle's int8-activation mode (Q8_0 / Q4_0 experts, the pages'
MMQ path): the quantiser against hand-computed blocks (golden/q8a_blocks.txt),
against an exact nearest-code search and its round-trip bound, and the whole
int8-mode layer against a float64 evaluation of its definition."""

import os

import numpy as np
import pytest

import moegen
from tests import np_ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "q8a_blocks.txt")


def golden_cases():
    cases, cur = [], None
    for ln in open(GOLDEN):
        ln = ln.strip()
        if not ln or ln.startswith("#"):
            continue
        key, _, rest = ln.partition(" ")
        if key == "case":
            cur = {"name": rest.split(":")[0]}
            cases.append(cur)
        elif key == "values":
            cur["values"] = np.array([float.fromhex(t) for t in rest.split()], np.float32)
        elif key == "scale":
            cur["scale"] = float.fromhex(rest)
        elif key == "codes":
            cur["codes"] = np.array([int(t) for t in rest.split()], np.int8)
    return cases


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c["name"])
def test_hand_computed_blocks(ref, case):
    codes, scales = ref.q8a_quantize(case["values"])
    assert scales.tolist() == [case["scale"]]
    assert codes.tolist() == case["codes"].tolist()


@pytest.mark.parametrize("dist", ["normal", "wide", "ties", "outlier"])
def test_quantiser_against_exact_search(ref, dist):
    """Every code is the nearest d q to v (exact comparison, halves away from
    zero), except where the exact quotient v / d lies within fp32 rounding of
    a half-integer: there the oracle's fp32 quotient decides, and the code may
    be the other neighbour."""
    rng = np.random.default_rng({"normal": 11, "wide": 12, "ties": 13, "outlier": 14}[dist])
    n = 32 * 128
    if dist == "normal":
        v = rng.standard_normal(n)
    elif dist == "wide":
        v = rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n // 32).repeat(32))
    elif dist == "ties":   # halves of a power-of-two scale: exact ties
        v = (rng.integers(-127, 127, n) + 0.5) / 8.0
        v[::32] = 127 / 8.0
    else:   # one large element per block: most codes small
        v = rng.standard_normal(n)
        v[::32] *= 1000.0
    v = v.astype(np.float32)
    codes, scales = ref.q8a_quantize(v)
    bc, bs = np_ref.q8a_brute(v)
    assert np.array_equal(scales, bs)
    diff = codes.astype(np.int64) != bc.astype(np.int64)
    if diff.any():
        d = np.repeat(scales.astype(np.float64), 32)[diff]
        t = v[diff].astype(np.float64) / d
        frac = np.abs(np.abs(t) - np.floor(np.abs(t)) - 0.5)
        assert np.all(frac <= 2.0 ** -22 * np.abs(t)), "a non-tie code differs"
        assert np.all(np.abs(codes[diff].astype(np.int64) - bc[diff]) == 1)
    assert diff.sum() <= n // 1000
    if dist == "ties":
        assert not diff.any()


def test_round_trip_bound_and_range(ref):
    """|v - d q| <= d / 2 (to fp32 rounding of the quotient); the block
    maximum takes code +-127; codes stay in -127..127."""
    rng = np.random.default_rng(15)
    v = (rng.standard_normal(32 * 256) * np.exp2(rng.integers(-20, 20, 256).repeat(32)))
    v = v.astype(np.float32)
    codes, scales = ref.q8a_quantize(v)
    d = np.repeat(scales.astype(np.float64), 32)
    back = codes.astype(np.float64) * d
    assert np.all(np.abs(back - v) <= d * (0.5 + 2.0 ** -20))
    assert codes.min() >= -127 and codes.max() <= 127
    blk = np.abs(v.reshape(-1, 32)).argmax(axis=1)
    assert np.all(np.abs(codes.reshape(-1, 32)[np.arange(256), blk]) == 127)


@pytest.mark.parametrize("qtype,shared", [("q8_0", 0), ("q4_0", 0), ("q4_0", 256)])
def test_q8a_layer_float64(ref, qtype, shared):
    """The int8-mode layer against numpy float64: x_q = d q per token and
    block; per pair a = silu(Wg x_q) * (Wu x_q), then the int8 round trip of
    fp32(a) into the down projection; slot-ordered combine plus the shared
    expert (Q8_0)."""
    q = {"q8_0": moegen.Q8_0, "q4_0": moegen.Q4_0}[qtype]
    cfg = moegen.TINY.with_(expert_q=q, hidden=256, ffn=256, n_experts=4, top_k=2,
                            shared_ffn=shared, shared_q=moegen.Q8_0)
    L = moegen.make_layer(cfg)
    T = 5
    x = moegen.as_numpy_bits(moegen.make_x(cfg, T))
    _, ids, w = ref.route(x, L.router.numpy(), None, k=cfg.top_k, act_dtype=cfg.act_dtype,
                          router_dtype=cfg.router_dtype, score="softmax")
    kw = dict(n_experts=cfg.n_experts, ffn=cfg.ffn, qtype=qtype, act_dtype=cfg.act_dtype)
    if shared:
        kw.update(s_gate=L.s_gate.numpy(), s_up=L.s_up.numpy(), s_down=L.s_down.numpy(),
                  shared_ffn=shared, shared_q="q8_0")
    out = ref.forward(x, L.w_gate.numpy(), L.w_up.numpy(), L.w_down.numpy(), ids, w,
                      act_quant="int8", **kw)
    H, F, E = cfg.hidden, cfg.ffn, cfg.n_experts
    dq = lambda buf, R, n, qt=qtype: np_ref.dequant_matrix(qt, buf, R, n)
    Wg = dq(L.w_gate.numpy(), E * F, H).reshape(E, F, H)
    Wu = dq(L.w_up.numpy(), E * F, H).reshape(E, F, H)
    Wd = dq(L.w_down.numpy(), E * H, F).reshape(E, H, F)
    X = np_ref.act(x)

    def ffn(wg, wu, wd, xq):
        a = (np_ref.silu(wg @ xq) * (wu @ xq)).astype(np.float32)
        return wd @ np_ref.q8a_round_trip(a)

    want = np.zeros((T, H))
    for t in range(T):
        xq = np_ref.q8a_round_trip(X[t].astype(np.float32))
        for j in range(cfg.top_k):
            want[t] += float(w[t, j]) * ffn(Wg[ids[t, j]], Wu[ids[t, j]], Wd[ids[t, j]], xq)
        if shared:
            Sg = dq(L.s_gate.numpy(), shared, H, "q8_0")
            Su = dq(L.s_up.numpy(), shared, H, "q8_0")
            Sd = dq(L.s_down.numpy(), H, shared, "q8_0")
            want[t] += ffn(Sg, Su, Sd, xq)
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-6 * np.abs(want).max())
    # the mode is not the identity, and it stays near the fp32-activation layer
    # (per element at most half a code step of x and of h, about 1 % of a block's
    # largest magnitude)
    plain = ref.forward(x, L.w_gate.numpy(), L.w_up.numpy(), L.w_down.numpy(), ids, w, **kw)
    dev = np.abs(plain - out).max() / np.abs(plain).max()
    assert 1e-5 < dev < 5e-2


def test_q8a_needs_q8_0_or_q4_0(ref):
    cfg = moegen.TINY.with_(expert_q=moegen.MXFP4)
    L = moegen.make_layer(cfg)
    x = moegen.as_numpy_bits(moegen.make_x(cfg, 2))
    ids = np.zeros((2, cfg.top_k), np.int32)
    ids[:, 1] = 1
    w = np.ones((2, cfg.top_k), np.float32)
    with pytest.raises(ValueError):
        ref.forward(x, L.w_gate.numpy(), L.w_up.numpy(), L.w_down.numpy(), ids, w,
                    n_experts=cfg.n_experts, ffn=cfg.ffn, qtype="mxfp4", act_dtype="f32",
                    act_quant="int8")
