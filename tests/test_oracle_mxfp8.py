"""Pins of the oracle's MXFP8 activation mode (MXFP4 experts on block-scaled
MFMA): the quantiser against hand-decoded blocks (golden/mxfp8_blocks.txt) and
against an exhaustive nearest-code search, the E4M3 decoder against its bit
fields, and the whole MXFP8-mode layer against a float64 evaluation built on
the exhaustive quantiser."""

import os

import numpy as np
import pytest

import moegen
from tests import np_ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "mxfp8_blocks.txt")


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
            cur["scale"] = int(rest)
        elif key == "codes":
            cur["codes"] = np.array([int(t, 16) for t in rest.split()], np.uint8)
    return cases


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c["name"])
def test_hand_decoded_blocks(ref, case):
    codes, scales = ref.mxfp8_quantize(case["values"])
    assert scales.tolist() == [case["scale"]]
    assert codes.tolist() == case["codes"].tolist()
    # the exhaustive search agrees with the hand decoding too
    bc, bs = np_ref.mxfp8_brute(case["values"])
    assert bs.tolist() == [case["scale"]] and bc.tolist() == case["codes"].tolist()


def test_e4m3_decoder_against_bit_fields(ref):
    tab = np_ref.e4m3_table()
    for c in range(256):
        v = ref.e4m3_value(c)
        if np.isnan(tab[c]):
            assert np.isnan(v)
        else:
            assert v == tab[c], hex(c)
    # a few values fixed by the format: 1, the largest finite, the smallest subnormal
    assert ref.e4m3_value(0x38) == 1.0 and ref.e4m3_value(0x7E) == 448.0
    assert ref.e4m3_value(0x01) == 2.0 ** -9 and ref.e4m3_value(0xB8) == -1.0


@pytest.mark.parametrize("dist", ["normal", "wide", "tiny", "ties"])
def test_quantiser_equals_exhaustive_search(ref, dist):
    rng = np.random.default_rng({"normal": 1, "wide": 2, "tiny": 3, "ties": 4}[dist])
    n = 32 * 64
    if dist == "normal":
        v = rng.standard_normal(n)
    elif dist == "wide":
        v = rng.standard_normal(n) * np.exp2(rng.integers(-40, 40, n))
    elif dist == "tiny":
        v = rng.standard_normal(n) * 2.0 ** -135
    else:   # every element on an E4M3 rounding tie of its block's scale
        v = (rng.integers(8, 16, n) + 0.5) * np.exp2(rng.integers(-5, 5, n)) * \
            np.where(rng.random(n) < 0.5, -1, 1)
    v = v.astype(np.float32)
    codes, scales = ref.mxfp8_quantize(v)
    bc, bs = np_ref.mxfp8_brute(v)
    assert np.array_equal(scales, bs)
    assert np.array_equal(codes, bc)


def test_round_trip_error_bound(ref):
    """An element at least 2^-6 of its block's scale times 2^8 (a normal
    E4M3 number after scaling) comes back within half a step: relative
    error at most 2^-4."""
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(32 * 256) * np.exp2(rng.integers(-10, 10, 32 * 256))).astype(np.float32)
    codes, scales = ref.mxfp8_quantize(v)
    tab = np_ref.e4m3_table()
    back = tab[codes] * np.repeat(np.exp2(scales.astype(np.float64) - 127), 32)
    X = np.repeat(np.exp2(scales.astype(np.float64) - 127), 32)
    normal = (np.abs(v) / X >= 2.0 ** -6) & (np.abs(v) / X < 448)
    rel = np.abs(back[normal] - v[normal]) / np.abs(v[normal])
    assert rel.max() <= 2.0 ** -4
    # the block maximum never saturates by more than one step (448 vs < 512)
    assert np.all(np.abs(back) <= 448 * X)


@pytest.mark.parametrize("shared", [0, 256])
def test_mx8_layer_float64(ref, shared):
    """The MXFP8-mode layer on MXFP4 experts against numpy float64 with the
    exhaustive quantiser: x_q = MXFP8(x) per token; per pair a = silu(Wg x_q)
    * (Wu x_q), then MXFP8(fp32(a)) into the down projection; slot-ordered
    combine plus the shared expert."""
    cfg = moegen.TINY.with_(expert_q=moegen.MXFP4, hidden=256, ffn=256, n_experts=4,
                            top_k=2, shared_ffn=shared, shared_q=moegen.MXFP4)
    L = moegen.make_layer(cfg)
    T = 5
    x = moegen.as_numpy_bits(moegen.make_x(cfg, T))
    _, ids, w = ref.route(x, L.router.numpy(), None, k=cfg.top_k, act_dtype=cfg.act_dtype,
                          router_dtype=cfg.router_dtype, score="softmax")
    kw = dict(n_experts=cfg.n_experts, ffn=cfg.ffn, qtype="mxfp4", act_dtype=cfg.act_dtype)
    if shared:
        kw.update(s_gate=L.s_gate.numpy(), s_up=L.s_up.numpy(), s_down=L.s_down.numpy(),
                  shared_ffn=shared, shared_q="mxfp4")
    out = ref.forward(x, L.w_gate.numpy(), L.w_up.numpy(), L.w_down.numpy(), ids, w,
                      act_quant="mxfp8", **kw)
    H, F, E = cfg.hidden, cfg.ffn, cfg.n_experts
    Wg = np_ref.mxfp4_matrix(L.w_gate.numpy(), E * F, H).reshape(E, F, H)
    Wu = np_ref.mxfp4_matrix(L.w_up.numpy(), E * F, H).reshape(E, F, H)
    Wd = np_ref.mxfp4_matrix(L.w_down.numpy(), E * H, F).reshape(E, H, F)
    X = np_ref.act(x)

    def ffn(wg, wu, wd, xq):
        a = (np_ref.silu(wg @ xq) * (wu @ xq)).astype(np.float32)
        return wd @ np_ref.mxfp8_round_trip(a)

    want = np.zeros((T, H))
    for t in range(T):
        xq = np_ref.mxfp8_round_trip(X[t].astype(np.float32))
        for j in range(cfg.top_k):
            want[t] += float(w[t, j]) * ffn(Wg[ids[t, j]], Wu[ids[t, j]], Wd[ids[t, j]], xq)
        if shared:
            Sg = np_ref.mxfp4_matrix(L.s_gate.numpy(), shared, H)
            Su = np_ref.mxfp4_matrix(L.s_up.numpy(), shared, H)
            Sd = np_ref.mxfp4_matrix(L.s_down.numpy(), H, shared)
            want[t] += ffn(Sg, Su, Sd, xq)
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-6 * np.abs(want).max())
    # and the mode is not the identity: MXFP8 activations move the output
    plain = ref.forward(x, L.w_gate.numpy(), L.w_up.numpy(), L.w_down.numpy(), ids, w, **kw)
    assert np.abs(plain - out).max() > 1e-3 * np.abs(plain).max()


def test_mx8_needs_mxfp4_experts(ref):
    cfg = moegen.TINY
    L = moegen.make_layer(cfg)
    x = moegen.as_numpy_bits(moegen.make_x(cfg, 2))
    ids = np.zeros((2, cfg.top_k), np.int32)
    ids[:, 1] = 1
    w = np.ones((2, cfg.top_k), np.float32)
    with pytest.raises(ValueError):
        ref.forward(x, L.w_gate.numpy(), L.w_up.numpy(), L.w_down.numpy(), ids, w,
                    n_experts=cfg.n_experts, ffn=cfg.ffn, qtype="q8_0", act_dtype="f32",
                    act_quant="mxfp8")
