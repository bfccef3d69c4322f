"""Pins of the oracle's block decoding: hand-decoded blocks, exact code
round trips, and the generator's quantizers."""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import moegen
from tests import np_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q_blocks.txt")


def golden_blocks():
    out = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        q, hx, d, vals = [s.strip() for s in line.split("|")]
        out.append((q, bytes.fromhex(hx), Fraction(d), [int(v) for v in vals.split()]))
    return out


@pytest.mark.parametrize("rec", golden_blocks(), ids=lambda r: f"{r[0]}-{r[1][:2].hex()}")
def test_hand_decoded_blocks(ref, rec):
    q, raw, d, mult = rec
    assert len(raw) == np_ref.BQ[q] and len(mult) == 32
    got = ref.dequant_row(q, np.frombuffer(raw, dtype=np.uint8), 32)
    want = np.array([float(d * m) for m in mult], dtype=np.float64)
    assert np.array_equal(got.astype(np.float64), want)
    # the independent numpy decoder used by the float64 cross-checks agrees too
    assert np.array_equal(np_ref.dequant(q, np.frombuffer(raw, dtype=np.uint8), 32), want)


def test_half_and_bf16_scalars(ref):
    assert ref.half_to_float(0x3C00) == 1.0
    assert ref.half_to_float(0xC000) == -2.0
    assert ref.half_to_float(0x0001) == 2.0 ** -24
    assert ref.half_to_float(0x03FF) == 1023 * 2.0 ** -24      # largest subnormal
    assert ref.half_to_float(0x0400) == 2.0 ** -14             # smallest normal
    assert ref.half_to_float(0x7BFF) == 65504.0
    assert np.isinf(ref.half_to_float(0x7C00))
    # every finite half agrees with numpy's binary16
    h = np.arange(0, 1 << 16, 97, dtype=np.uint16)
    fin = np.isfinite(h.view(np.float16))
    for v in h[fin][:700]:
        assert ref.half_to_float(int(v)) == float(np.uint16(v).view(np.float16))
    assert ref.bf16_to_float(0x3F80) == 1.0
    assert ref.bf16_to_float(0xC0A0) == -5.0
    assert ref.bf16_to_float(0x0001) == np.uint32(1 << 16).view(np.float32)


@pytest.mark.parametrize("qtype", ["q8_0", "q4_0"])
def test_code_round_trip_every_block(ref, qtype):
    """Dequantised values divided by fp32(d) give back exactly the stored codes,
    for every block of the tiny layer and of sample rows of the larger ones."""
    rows = []
    L = moegen.make_layer(moegen.TINY, qtype=qtype)
    rows += [(L.w_gate.reshape(-1, L.w_gate.shape[-1]).numpy(), 256),
             (L.w_down.reshape(-1, L.w_down.shape[-1]).numpy(), 512)]
    for cfg in (moegen.QWEN3_DECODE, moegen.DEEPSEEK, moegen.SWEEP_Q8):
        w = moegen.quantized_normal(4, cfg.hidden, cfg.w_std, qtype,
                                    moegen.seed_of(cfg.cid, moegen.T_GATE, 3), "cpu")
        rows.append((w.numpy(), cfg.hidden))
    bq = np_ref.BQ[qtype]
    for mat, n in rows:
        for r in mat:
            v = ref.dequant_row(qtype, r, n).reshape(-1, 32)
            blocks = r.reshape(-1, bq)
            d = blocks[:, 0:2].copy().view(np.float16)[:, 0].astype(np.float32)
            if qtype == "q8_0":
                codes = blocks[:, 2:].view(np.int8).astype(np.int32)
            else:
                b = blocks[:, 2:].astype(np.int32)
                codes = np.concatenate([b & 15, b >> 4], axis=1) - 8
            nz = d != 0
            assert np.array_equal(v[nz] / d[nz, None], codes[nz].astype(np.float32))
            assert not np.any(v[~nz])
            if qtype == "q4_0":
                assert codes.min() >= -8 and codes.max() <= 7


@pytest.mark.parametrize("qtype", ["q8_0", "q4_0"])
def test_quantizer_error_bound(ref, qtype):
    """The generator's quantizers reproduce their fp32 input to within one
    quantization step (half a step for Q8_0 plus the fp16 rounding of d)."""
    w = moegen.normal((64, 256), 0.02, 7)
    w[0, :32] = 0.0                        # an all-zero block
    w[1, 5] = w[1, :32].abs().max() * 3    # a single outlier
    raw = moegen.QUANTIZERS[qtype](w).numpy()
    x = w.numpy().astype(np.float64)
    for i in range(64):
        v = ref.dequant_row(qtype, raw[i], 256).astype(np.float64)
        d = np.abs(raw[i].reshape(-1, np_ref.BQ[qtype])[:, 0:2].copy()
                   .view(np.float16)[:, 0].astype(np.float64))
        err = np.abs(v - x[i]).reshape(-1, 32).max(axis=1)
        bound = (0.5 + 127 * 2.0 ** -11) * d if qtype == "q8_0" else (1.0 + 8 * 2.0 ** -11) * d
        assert np.all(err <= bound + 1e-12), (i, err, bound)
    assert not np.any(ref.dequant_row(qtype, raw[0], 256)[:32])


def test_q4_0_scale_sign_and_extreme():
    """Q4_0 maps the block's largest-magnitude element to code 0 with d = m/-8,
    so d < 0 whenever that element is positive."""
    w = torch.zeros(1, 32)
    w[0, 3] = 0.5
    w[0, 7] = -0.25
    raw = moegen.quantize_q4_0(w).numpy()[0]
    d = raw[0:2].copy().view(np.float16)[0]
    assert d == np.float16(-0.0625)
    assert raw[2 + 3] & 15 == 0                     # element 3 -> code 0 -> value 0.5
    assert raw[2 + 7] & 15 == 12                    # -0.25/-0.0625 + 8 = 12


# ---------------------------------------------------------------------------
# Q4_K (GGUF K-quant super-blocks).  The pages print no layout and no outside
# encoder is available here: the oracle's Q4_K decoding is pinned by a
# hand-packed super-block, by the case that reduces to Q4_0 (itself pinned by
# the hand-decoded fixture above), by brute force over every six-bit
# (scale, min) pair and every code position, and by the generator's error
# bound.

GOLDEN_K = os.path.join(os.path.dirname(__file__), "golden", "q4k_blocks.txt")


def golden_q4k():
    out = []
    for line in open(GOLDEN_K):
        if line.startswith("#") or not line.strip():
            continue
        name, d, dmin, sc, mn, rule, hx = [s.strip() for s in line.split("|")]
        out.append((name, Fraction(d), Fraction(dmin), [int(v) for v in sc.split()],
                    [int(v) for v in mn.split()], rule, bytes.fromhex(hx)))
    return out


@pytest.mark.parametrize("rec", golden_q4k(), ids=lambda r: r[0])
def test_q4k_hand_packed_block(ref, rec):
    name, d, dmin, sc, mn, rule, raw = rec
    assert len(raw) == 144 and rule == "updown"
    got = ref.dequant_row("q4_k", np.frombuffer(raw, dtype=np.uint8), 256)
    want = []
    for e in range(256):
        j = 2 * (e // 64) + (e % 64 >= 32)        # sub-block
        l = e % 32                                # byte within the group
        q = l % 16 if e % 64 < 32 else 15 - l % 16
        want.append(float(d * sc[j] * q - dmin * mn[j]))
    assert np.array_equal(got.astype(np.float64), np.array(want))
    assert np.array_equal(np_ref.dequant("q4_k", np.frombuffer(raw, dtype=np.uint8), 256),
                          np.array(want))


def _q4k_raw(d16, dmin16, scale_bytes, codes):
    """A super-block from its fields: codes [256] in element order."""
    codes = np.asarray(codes, dtype=np.uint8).reshape(4, 2, 32)
    qs = (codes[:, 0, :] | (codes[:, 1, :] << 4)).reshape(-1)
    hdr = np.array([d16, dmin16], dtype=np.float16).view(np.uint8)
    return np.concatenate([hdr, np.asarray(scale_bytes, dtype=np.uint8), qs])


def test_q4k_reduces_to_q4_0(ref):
    """scale = min = 1 in every sub-block and dmin = 8 d give d * (q - 8): the
    same values as eight Q4_0 blocks with scale d and the same codes."""
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, 256)
    d = np.float16(0.0234)
    ones = [1 | 0 << 6] * 4 + [1 | 0 << 6] * 4 + [1 | 1 << 4] * 4   # all scales, mins 1
    got = ref.dequant_row("q4_k", _q4k_raw(d, np.float16(8 * float(d)), ones, codes), 256)
    q40 = []
    for b in range(8):
        c = codes[32 * b:32 * b + 32]
        q40.append(np.concatenate([np.array([d], np.float16).view(np.uint8),
                                   (c[:16] | (c[16:] << 4)).astype(np.uint8)]))
    want = ref.dequant_row("q4_0", np.concatenate(q40), 256)
    assert np.array_equal(got, want)


def test_q4k_every_scale_and_min(ref):
    """Each sub-block j decodes every six-bit (scale, min) pair: with codes
    q = 0 and q = 1 the values are -min and scale - min (d = dmin = 1)."""
    for j in range(8):
        for s in range(64):
            m = (s * 37 + 11 * j) % 64
            sc = np.zeros(12, np.int64)
            if j < 4:
                sc[j] |= s
                sc[j + 4] |= m
            else:
                sc[j + 4] |= (s & 15) | (m & 15) << 4
                sc[j - 4] |= (s >> 4) << 6
                sc[j] |= (m >> 4) << 6
            codes = np.zeros(256, np.int64)
            e0 = 64 * (j // 2) + 32 * (j % 2)
            codes[e0 + 1] = 1
            v = ref.dequant_row("q4_k", _q4k_raw(1.0, 1.0, sc, codes), 256)
            assert v[e0] == -m and v[e0 + 1] == s - m, (j, s, m)
            others = np.delete(np.arange(256), np.arange(e0, e0 + 32))
            assert not np.any(v[others] > 0)


def test_q4k_every_code_position(ref):
    """A single non-zero code at position p changes exactly element p."""
    sc = [1] * 4 + [0] * 4 + [1] * 4          # scale 1, min 0 everywhere
    for p in range(256):
        codes = np.zeros(256, np.int64)
        codes[p] = 7
        v = ref.dequant_row("q4_k", _q4k_raw(1.0, 0.0, sc, codes), 256)
        assert v[p] == 7 and np.count_nonzero(v) == 1, p


def test_q4k_quantizer_error_bound(ref):
    """The generator's Q4_K quantizer reproduces its input to within one code
    step d * scale_j of each sub-block plus the six-bit rounding of the min;
    the numpy decoder agrees with the oracle exactly."""
    w = moegen.normal((16, 512), 0.02, 9)
    w[0, :256] = 0.0
    w[1, 40] = 0.3
    raw = moegen.quantize_q4_k(w).numpy()
    x = w.numpy().astype(np.float64)
    for i in range(16):
        v = ref.dequant_row("q4_k", raw[i], 512).astype(np.float64)
        assert np.array_equal(v, np_ref.dequant("q4_k", raw[i], 512).astype(np.float32))
        sb = raw[i].reshape(2, 144)
        d = sb[:, 0:2].copy().view(np.float16)[:, 0].astype(np.float64)
        dmin = sb[:, 2:4].copy().view(np.float16)[:, 0].astype(np.float64)
        s, m = np_ref._q4k_scales(sb[:, 4:16])
        err = np.abs(v - x[i]).reshape(2, 8, 32).max(axis=-1)
        bound = d[:, None] * np.maximum(s, 1) + dmin[:, None] * 0.5 + 1e-3 * 2.0 ** -7
        assert np.all(err <= bound), (i, err, bound)
    assert not np.any(ref.dequant_row("q4_k", raw[0], 512)[:256])


# Q6_K (GGUF K-quant super-blocks of 210 bytes).  As for Q4_K, no layout is
# printed and no outside encoder is available: the oracle's Q6_K decoding is
# pinned by hand-packed super-blocks, by the case that reduces to Q8_0 (pinned
# by the hand-decoded fixture above), by brute force over every code position,
# every code value and every int8 scale, and by the generator's error bound.

GOLDEN_6K = os.path.join(os.path.dirname(__file__), "golden", "q6k_blocks.txt")


def golden_q6k():
    out = []
    for line in open(GOLDEN_6K):
        if line.startswith("#") or not line.strip():
            continue
        name, d, sc, rule, hx = [s.strip() for s in line.split("|")]
        out.append((name, Fraction(d), [int(v) for v in sc.split()], rule, bytes.fromhex(hx)))
    return out


@pytest.mark.parametrize("rec", golden_q6k(), ids=lambda r: r[0])
def test_q6k_hand_packed_block(ref, rec):
    name, d, sc, rule, raw = rec
    assert len(raw) == 210 and rule == "kq" and len(sc) == 16
    want = []
    for e in range(256):
        k, l = (e % 128) // 32, e % 32
        q = 16 * k + (l % 16 if k < 2 else 15 - l % 16)
        want.append(float(d * sc[e // 16] * (q - 32)))
    want = np.array(want)
    got = ref.dequant_row("q6_k", np.frombuffer(raw, dtype=np.uint8), 256)
    assert np.array_equal(got.astype(np.float64), want)
    assert np.array_equal(np_ref.dequant("q6_k", np.frombuffer(raw, dtype=np.uint8), 256), want)


def _q6k_raw(d16, scales, codes):
    """A super-block from its fields, packed by the layout rule (codes [256]
    in element order, 0..63)."""
    q = np.asarray(codes, dtype=np.int64).reshape(2, 4, 32)      # [h][k][l]
    ql = np.stack([(q[:, 0] & 15) | ((q[:, 2] & 15) << 4),
                   (q[:, 1] & 15) | ((q[:, 3] & 15) << 4)], axis=1).reshape(-1)
    hi = q >> 4
    qh = (hi[:, 0] | hi[:, 1] << 2 | hi[:, 2] << 4 | hi[:, 3] << 6).reshape(-1)
    sc = np.asarray(scales, dtype=np.int64).astype(np.int8).view(np.uint8)
    dd = np.array([d16], dtype=np.float16).view(np.uint8)
    return np.concatenate([ql.astype(np.uint8), qh.astype(np.uint8), sc, dd])


def test_q6k_reduces_to_q8_0(ref):
    """Every scale 1: the values are d * (q - 32), the same as Q8_0 blocks with
    scale d and codes q - 32."""
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 64, 256)
    d = np.float16(0.0371)
    got = ref.dequant_row("q6_k", _q6k_raw(d, [1] * 16, codes), 256)
    q8 = []
    for b in range(8):
        c = (codes[32 * b:32 * b + 32] - 32).astype(np.int8)
        q8.append(np.concatenate([np.array([d], np.float16).view(np.uint8), c.view(np.uint8)]))
    assert np.array_equal(got, ref.dequant_row("q8_0", np.concatenate(q8), 256))


def test_q6k_every_code_position(ref):
    """A code of 33 (value d * scale) at position p and 32 (zero) elsewhere
    changes exactly element p."""
    for p in range(256):
        codes = np.full(256, 32)
        codes[p] = 33
        v = ref.dequant_row("q6_k", _q6k_raw(1.0, [3] * 16, codes), 256)
        assert v[p] == 3 and np.count_nonzero(v) == 1, p


def test_q6k_every_code_value_and_scale(ref):
    """Each of the 64 code values in every element slot of a 32-element run
    (covering both nibbles and all four top-bit pairs), and each of the 256
    int8 scales in every sub-block."""
    for q in range(64):
        codes = np.full(256, 32)
        e = np.arange(q % 4 * 32 + 128 * (q % 2), q % 4 * 32 + 128 * (q % 2) + 32)
        codes[e] = q
        v = ref.dequant_row("q6_k", _q6k_raw(0.5, [2] * 16, codes), 256)
        assert np.all(v[e] == q - 32) and np.count_nonzero(np.delete(v, e)) == 0, q
    for j in range(16):
        for s in range(-128, 128):
            sc = [0] * 16
            sc[j] = s
            codes = np.full(256, 63)
            v = ref.dequant_row("q6_k", _q6k_raw(0.25, sc, codes), 256)
            assert np.all(v[16 * j:16 * j + 16] == 0.25 * s * 31), (j, s)
            assert np.count_nonzero(np.delete(v, np.arange(16 * j, 16 * j + 16))) == 0


def test_q6k_quantizer_error_bound(ref):
    """The generator's Q6_K quantizer reproduces its input to within one code
    step d * |scale_j| of each 16-element sub-block; the numpy decoder agrees
    with the oracle exactly."""
    w = moegen.normal((16, 512), 0.02, 9)
    w[0, :256] = 0.0
    w[1, 40] = 0.3
    raw = moegen.quantize_q6_k(w).numpy()
    x = w.numpy().astype(np.float64)
    for i in range(16):
        v = ref.dequant_row("q6_k", raw[i], 512).astype(np.float64)
        assert np.array_equal(v, np_ref.dequant("q6_k", raw[i], 512).astype(np.float32))
        sb = raw[i].reshape(2, 210)
        d = sb[:, 208:210].copy().view(np.float16)[:, 0].astype(np.float64)
        sc = sb[:, 192:208].copy().view(np.int8).astype(np.float64)
        err = np.abs(v - x[i]).reshape(2, 16, 16).max(axis=-1)
        assert np.all(err <= d[:, None] * np.abs(sc) + 1e-12), (i, err)
    assert not np.any(ref.dequant_row("q6_k", raw[0], 512)[:256])


# MXFP4 (group 32, MLX packing).  No layout is printed and no outside encoder
# is available: the oracle's decoding is pinned by hand-packed rows, by the
# case that reduces to Q8_0, by every code at several scales, by the NaN
# scale, and by the generator's error bound.

GOLDEN_MX = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_blocks.txt")
E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def golden_mxfp4():
    out = []
    for line in open(GOLDEN_MX):
        if line.startswith("#") or not line.strip():
            continue
        name, sc, rule, hx = [s.strip() for s in line.split("|")]
        out.append((name, [int(v) for v in sc.split()], rule, bytes.fromhex(hx)))
    return out


def _e2m1(code):
    v = E2M1[code & 7]
    return -v if code & 8 else v


@pytest.mark.parametrize("rec", golden_mxfp4(), ids=lambda r: r[0])
def test_mxfp4_hand_packed_row(ref, rec):
    name, sc, rule, raw = rec
    assert len(raw) == 34 and len(sc) == 2 and rule in ("ramp", "rev")
    want = []
    for j in range(64):
        code = j % 16 if rule == "ramp" else 15 - j % 16
        want.append(float(_e2m1(code) * Fraction(2) ** (sc[j // 32] - 127)))
    got = ref.dequant_row("mxfp4", np.frombuffer(raw, dtype=np.uint8), 64)
    assert np.array_equal(got.astype(np.float64), np.array(want))
    assert np.array_equal(np_ref.dequant("mxfp4", np.frombuffer(raw, dtype=np.uint8), 64),
                          np.array(want))


def _mx_row(codes, scales):
    c = np.asarray(codes, dtype=np.uint8)
    return np.concatenate([(c[0::2] | (c[1::2] << 4)).astype(np.uint8),
                           np.asarray(scales, dtype=np.uint8)])


def _mx_want(code, s):
    """The exact value as fp32 would hold it: 2^128 and beyond are infinite."""
    v = _e2m1(code) * Fraction(2) ** (s - 127)
    if abs(v) >= 2 ** 128:
        return -np.inf if v < 0 else np.inf
    return float(v)


def test_mxfp4_every_code_and_scale(ref):
    """Each code in each element slot (both nibbles) at scales 1, 126, 127,
    128, 253 and 254 (where the larger values exceed fp32 and are infinite);
    scale 255 decodes to NaN."""
    for s in (1, 126, 127, 128, 253, 254):
        for code in range(16):
            for j0 in (0, 1, 30, 31):
                codes = np.zeros(32, np.int64)
                codes[j0] = code
                v = ref.dequant_row("mxfp4", _mx_row(codes, [s]), 32)
                assert v[j0] == _mx_want(code, s), (s, code, j0)
                assert np.count_nonzero(np.delete(v, j0)) == 0
    v = ref.dequant_row("mxfp4", _mx_row(np.full(32, 2), [255]), 32)
    assert np.all(np.isnan(v))


def test_mxfp4_reduces_to_q8_0(ref):
    """Scale 127: the values are the E2M1 values themselves, the same as a
    Q8_0 block with d = 1/2 and codes 2 * value."""
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 16, 32)
    got = ref.dequant_row("mxfp4", _mx_row(codes, [127]), 32)
    q8 = np.array([int(2 * _e2m1(c)) for c in codes], dtype=np.int8)
    blk = np.concatenate([np.array([0.5], np.float16).view(np.uint8), q8.view(np.uint8)])
    assert np.array_equal(got, ref.dequant_row("q8_0", blk, 32))


def test_mxfp4_quantizer_error_bound(ref):
    """The generator's MXFP4 quantizer reproduces its input within two E2M1
    steps of the group's scale (the largest spacing, 4 -> 6, halved, or the
    clip of values in (6, 8) x 2^e to 6); the matrix layout decodes row by row
    like single rows."""
    w = moegen.normal((16, 256), 0.02, 9)
    w[0, :32] = 0.0
    w[1, 40] = 0.3
    buf = moegen.quantize_mxfp4(w).numpy()
    m = np_ref.mxfp4_matrix(buf, 16, 256)
    x = w.numpy().astype(np.float64)
    sc = buf[16 * 128:].reshape(16, 8).astype(np.float64)
    for r in range(16):
        row = np.concatenate([buf[r * 128:(r + 1) * 128], buf[2048 + r * 8:2048 + (r + 1) * 8]])
        assert np.array_equal(ref.dequant_row("mxfp4", row, 256).astype(np.float64), m[r])
    err = np.abs(m - x).reshape(16, 8, 32).max(axis=-1)
    assert np.all(err <= 2.0 * np.exp2(sc - 127))
    assert not np.any(m[0, :32])
