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
