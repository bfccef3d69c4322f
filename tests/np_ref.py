"""Independent numpy decoding of GGUF blocks, for float64 cross-checks of the
oracle.  Vectorised and written separately from the oracle's C loops; it is
itself pinned by the hand-decoded fixture in golden/q_blocks.txt."""

import numpy as np

BQ = {"q8_0": 34, "q4_0": 18, "q4_k": 18}   # bytes per 32 elements (Q4_K: 144 per 256)
SUPER = {"q4_k": 144, "q6_k": 210}           # bytes per 256-element super-block


def _q4k_scales(sc):
    """[..., 12] packed bytes -> (scale, min) [..., 8] as int64: sub-blocks
    0..3 in the low six bits of bytes 0..3 / 4..7; sub-blocks 4..7 combine the
    nibbles of bytes 8..11 with the top two bits of bytes 0..3 / 4..7."""
    sc = sc.astype(np.int64)
    s = np.concatenate([sc[..., 0:4] & 63, (sc[..., 8:12] & 15) | ((sc[..., 0:4] >> 6) << 4)], -1)
    m = np.concatenate([sc[..., 4:8] & 63, (sc[..., 8:12] >> 4) | ((sc[..., 4:8] >> 6) << 4)], -1)
    return s, m


E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def mxfp4_matrix(buf, R, n):
    """MLX MXFP4 matrix (R rows: R*n/2 code bytes, then R*n/32 E8M0 scales)
    -> float64 [R, n]."""
    buf = np.asarray(buf, dtype=np.uint8).reshape(-1)
    codes = buf[:R * n // 2].reshape(R, n // 2).astype(np.int64)
    sc = buf[R * n // 2:R * n // 2 + R * n // 32].reshape(R, n // 32).astype(np.float64)
    q = np.stack([codes & 15, codes >> 4], axis=-1).reshape(R, n)
    v = E2M1[q & 7] * np.where(q & 8, -1.0, 1.0)
    scale = np.where(sc == 255, np.nan, np.exp2(sc - 127.0))
    return v * np.repeat(scale, 32, axis=-1)


def dequant_matrix(qtype, buf, R, n):
    """A whole R x n matrix of any format -> float64 [R, n]."""
    if qtype == "mxfp4":
        return mxfp4_matrix(buf, R, n)
    return dequant(qtype, np.asarray(buf, dtype=np.uint8).reshape(R, -1), n)


def dequant(qtype, raw, n):
    """raw uint8 [..., n/32*Bq] -> float64 [..., n] (MXFP4: one row, its
    codes then its scales)."""
    raw = np.asarray(raw, dtype=np.uint8)
    lead = raw.shape[:-1]
    if qtype == "mxfp4":
        assert not lead
        return mxfp4_matrix(raw, 1, n)[0]
    if qtype == "q6_k":
        sb = raw.reshape(*lead, n // 256, 210)
        ql = sb[..., 0:128].astype(np.int64).reshape(*lead, n // 256, 2, 2, 32)   # [h][k%2][l]
        qh = sb[..., 128:192].astype(np.int64).reshape(*lead, n // 256, 2, 1, 32)  # [h][.][l]
        sc = sb[..., 192:208].copy().view(np.int8).astype(np.float64)           # [16]
        d = sb[..., 208:210].copy().view(np.float16)[..., 0].astype(np.float64)
        lo = np.concatenate([ql & 15, ql >> 4], axis=-2)                       # k = 0..3
        hi = np.concatenate([(qh >> (2 * k)) & 3 for k in range(4)], axis=-2)
        q = (lo | (hi << 4)).reshape(*lead, n // 256, 16, 16) - 32
        v = d[..., None, None] * sc[..., None] * q
        return v.reshape(*lead, n)
    if qtype == "q4_k":
        sb = raw.reshape(*lead, n // 256, 144)
        d = sb[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
        dmin = sb[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
        s, m = _q4k_scales(sb[..., 4:16])
        qs = sb[..., 16:].astype(np.int64).reshape(*lead, n // 256, 4, 32)
        codes = np.stack([qs & 15, qs >> 4], axis=-2).reshape(*lead, n // 256, 8, 32)
        v = (d[..., None, None] * s[..., None] * codes - dmin[..., None, None] * m[..., None])
        return v.reshape(*lead, n)
    blocks = raw.reshape(*lead, n // 32, BQ[qtype])
    d = blocks[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    if qtype == "q8_0":
        codes = blocks[..., 2:].view(np.int8).astype(np.float64)
    else:
        b = blocks[..., 2:].astype(np.int64)
        codes = np.concatenate([b & 15, b >> 4], axis=-1).astype(np.float64) - 8.0
    return (codes * d[..., None]).reshape(*lead, n)


def act(a):
    """Activations / router as float64 (uint16 arrays are bf16 bit patterns)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def silu(z):
    return z / (1.0 + np.exp(-z))


def e4m3_table():
    """Values of all 256 OCP E4M3FN codes (NaN for 0x7F / 0xFF), float64,
    decoded from the bit fields: sign 7, exponent 6..3 (bias 7), mantissa
    2..0; exponent 0 is subnormal."""
    c = np.arange(256)
    e, m = (c >> 3) & 15, c & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    v = np.where(c & 0x80, -v, v)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def mxfp8_brute(v):
    """MXFP8 quantisation by exhaustive search: per 32-element block the E8M0
    scale floor(log2 amax) - 8 (from frexp; clamped to -127..127; all-zero
    block: -127 and byte 0), then each element's code is the finite E4M3 value
    nearest to fp32(v) / 2^e (magnitudes above 448 clamped to 448), ties to
    the even code.  Returns (codes uint8 [n], scale bytes uint8 [n/32])."""
    v = np.asarray(v, dtype=np.float32).reshape(-1)
    tab = e4m3_table()
    finite = np.where(~np.isnan(tab))[0]
    codes = np.zeros(v.size, np.uint8)
    scales = np.zeros(v.size // 32, np.uint8)
    for b in range(v.size // 32):
        blk = v[32 * b:32 * b + 32]
        amax = float(np.max(np.abs(blk)))
        if amax == 0.0:
            codes[32 * b:32 * b + 32] = np.where(np.signbit(blk), 0x80, 0)
            continue
        e = int(np.frexp(amax)[1]) - 1 - 8
        e = min(max(e, -127), 127)
        scales[b] = e + 127
        for i, x in enumerate(blk):
            y = float(np.ldexp(np.float32(x), -e))
            y = min(max(y, -448.0), 448.0)
            d = np.abs(tab[finite] - y)
            best = finite[d == d.min()]
            if best.size > 1:   # a tie: the code with the even mantissa
                best = best[(best & 1) == 0]
            c = int(best[0])
            if y == 0.0 or (c & 0x7F) == 0:   # zero keeps the input's sign
                c = 0x80 if np.signbit(np.float32(x)) else 0
            codes[32 * b + i] = c
    return codes, scales


def mxfp8_round_trip(v):
    """fp32 values -> float64 values after an MXFP8 round trip (mxfp8_brute)."""
    c, s = mxfp8_brute(v)
    return e4m3_table()[c] * np.repeat(np.exp2(s.astype(np.float64) - 127.0), 32)


def q8a_brute(v):
    """int8 (Q8_1-style) quantisation by search: per 32-element block the fp32
    scale d = fp32(amax / 127); each element's code is the integer q in
    -127..127 whose d q is nearest to v, compared exactly (d q is exact in
    float64), ties to the larger magnitude; d = 0 gives codes 0.  The oracle
    divides in fp32 and rounds the quotient, so the two may differ by one
    where the exact quotient lies within fp32 rounding of a half-integer.
    Returns (codes int8 [n], scales float32 [n/32])."""
    v = np.asarray(v, dtype=np.float32).reshape(-1)
    codes = np.zeros(v.size, np.int8)
    scales = np.zeros(v.size // 32, np.float32)
    q = np.arange(-127, 128, dtype=np.float64)
    for b in range(v.size // 32):
        blk = v[32 * b:32 * b + 32].astype(np.float64)
        d = np.float32(np.max(np.abs(v[32 * b:32 * b + 32]))) / np.float32(127)
        scales[b] = d
        if d == 0:
            continue
        for i, x in enumerate(blk):
            err = np.abs(x - float(d) * q)
            best = q[err == err.min()]
            codes[32 * b + i] = int(best[np.argmax(np.abs(best))])
    return codes, scales


def q8a_quantize(v):
    """The int8 quantiser's definition in numpy: d = fp32(amax / 127), codes
    round(fp32(v / d)) with ties away from zero, clamped to -127..127."""
    v = np.asarray(v, dtype=np.float32).reshape(-1, 32)
    d = (np.max(np.abs(v), axis=1) / np.float32(127)).astype(np.float32)
    safe = np.where(d == 0, np.float32(1), d).astype(np.float32)
    t = (v / safe[:, None]).astype(np.float32).astype(np.float64)
    c = np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -127, 127)
    c = np.where(d[:, None] == 0, 0, c)
    return c.astype(np.int8).reshape(-1), d


def q8a_round_trip(v):
    """fp32 values -> float64 d * code after the int8 round trip."""
    c, d = q8a_quantize(v)
    return c.astype(np.float64) * np.repeat(d.astype(np.float64), 32)


def matrix_rows(qtype, buf, R, n, r0, r1):
    """Rows r0 .. r1 - 1 of an R x n matrix of any format -> float64 [r1 - r0, n]
    (decoding only those rows)."""
    buf = np.asarray(buf, dtype=np.uint8).reshape(-1)
    if qtype == "mxfp4":
        codes = buf[:R * n // 2].reshape(R, n // 2)[r0:r1]
        sc = buf[R * n // 2:R * n // 2 + R * n // 32].reshape(R, n // 32)[r0:r1]
        return mxfp4_matrix(np.concatenate([codes.reshape(-1), sc.reshape(-1)]), r1 - r0, n)
    rb = buf.size // R
    return dequant(qtype, buf.reshape(R, rb)[r0:r1], n)
