"""Seeded synthetic inputs for the MoE layer: activations, router, bias and
GGUF-blocked expert weights.

Input generation only.  It contains none of the layer's arithmetic: no dequant,
no routing, no FFN.  The quantizers below *produce* Q8_0 / Q4_0 / Q4_K / Q6_K / MXFP4 weights from fp32
samples (the way a checkpoint converter would); the layer only ever *reads*
blocks.  Both the GPU path and the CPU oracle are fed from here.

Everything is plain torch so the same code runs on the CPU (small shapes) or on
the GPU (the multi-GB layers, where a CPU generator would take minutes).  A
(config, tensor, expert) triple names an independent torch generator, so each
tensor and each expert can be regenerated alone.  The CPU and GPU generators
draw different streams for the same seed: a test uses one device for one layer.

Block byte layout (GGUF, little-endian, no padding):
  Q8_0: [fp16 d][32 x int8 q]            34 bytes, value = d*q
  Q4_0: [fp16 d][16 bytes of nibbles]    18 bytes, value = d*(q-8);
        byte i holds element i in its low nibble and element i+16 in its high
        nibble.
  Q4_K: 256-element super-block, 144 bytes: [fp16 d][fp16 dmin][12 bytes of
        six-bit (scale, min) pairs for the eight 32-element sub-blocks]
        [128 bytes of nibbles: group c of 64 elements uses bytes 32c..32c+31,
        low nibbles first 32 elements, high nibbles the next 32];
        value = d*scale_j*q - dmin*min_j.
  Q6_K: 256-element super-block, 210 bytes: [128 bytes ql][64 bytes qh]
        [16 int8 scales][fp16 d]; half h (128 elements) uses ql bytes
        64h..64h+63 and qh bytes 32h..32h+31; its element 32k+l takes the
        low nibble (k < 2) or high nibble (k >= 2) of ql byte 64h+32(k%2)+l
        and bits 2k, 2k+1 of qh byte 32h+l: a six-bit code q; value =
        d*scale_j*(q-32), j the 16-element sub-block.
  MXFP4 (MLX packing, group 32): a matrix of R rows is R x K/2 bytes of E2M1
        codes (element j in nibble j%2 of byte j/2, low first) followed by
        R x K/32 E8M0 scale bytes; value = E2M1(code) * 2^(scale-127).
"""

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import BF16, F32, MXFP4, Q4_0, Q4_K, Q6_K, Q8_0, LayerConfig, row_bytes

BASE_SEED = 20261202

# tensor ids (part of every seed)
T_X, T_ROUTER, T_GATE, T_UP, T_DOWN, T_SGATE, T_SUP, T_SDOWN = range(8)


def seed_of(cid: int, tid: int, eid: int) -> int:
    """A 63-bit seed for tensor `tid`, expert (or batch) `eid` of workload `cid`."""
    h = BASE_SEED
    for v in (cid, tid, eid):
        h = (h * 6364136223846793005 + 1442695040888963407 + v) & ((1 << 64) - 1)
        h ^= h >> 29
    return h & ((1 << 63) - 1)


def normal(shape, std, seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def _round_half_away(v):
    return torch.sign(v) * torch.floor(torch.abs(v) + 0.5)


def quantize_q8_0(w: torch.Tensor) -> torch.Tensor:
    """fp32 [..., n] -> uint8 [..., n/32*34].  d = amax/127 (fp32), codes
    round-half-away(x/d) clamped to +-127, d stored as fp16 (round to nearest
    even).  An all-zero block gets d = 0 and zero codes."""
    *lead, n = w.shape
    assert n % 32 == 0
    b = w.reshape(*lead, n // 32, 32)
    amax = b.abs().amax(dim=-1, keepdim=True)
    d = amax / 127.0
    inv = torch.where(d > 0, 1.0 / torch.where(d > 0, d, torch.ones_like(d)),
                      torch.zeros_like(d))
    q = _round_half_away(b * inv).clamp(-127, 127).to(torch.int8)
    d16 = d.to(torch.float16).view(torch.int16).view(torch.uint8)  # [..., nb, 2]
    out = torch.cat([d16.reshape(*lead, n // 32, 2), q.view(torch.uint8)], dim=-1)
    return out.reshape(*lead, n // 32 * 34).contiguous()


def quantize_q4_0(w: torch.Tensor) -> torch.Tensor:
    """fp32 [..., n] -> uint8 [..., n/32*18].  m = the element of largest
    magnitude (first on ties, sign kept), d = m / -8, codes
    min(15, floor(x/d + 8.5)), d stored as fp16.  d is negative whenever m > 0.
    An all-zero block gets d = 0 and codes 8."""
    *lead, n = w.shape
    assert n % 32 == 0
    b = w.reshape(*lead, n // 32, 32)
    idx = b.abs().argmax(dim=-1, keepdim=True)
    m = torch.gather(b, -1, idx)
    d = m / -8.0
    nz = d != 0
    inv = torch.where(nz, 1.0 / torch.where(nz, d, torch.ones_like(d)),
                      torch.zeros_like(d))
    q = torch.floor(b * inv + 8.5).clamp(0, 15).to(torch.uint8)
    packed = q[..., :16] | (q[..., 16:] << 4)
    d16 = d.to(torch.float16).view(torch.int16).view(torch.uint8)
    out = torch.cat([d16.reshape(*lead, n // 32, 2), packed], dim=-1)
    return out.reshape(*lead, n // 32 * 18).contiguous()


def quantize_q4_k(w: torch.Tensor) -> torch.Tensor:
    """fp32 [..., n] -> uint8 [..., n/256*144] (GGUF Q4_K super-blocks).
    Per 32-element sub-block j: scale_j = (max - min(min, 0)) / 15 and
    min_j = -min(min, 0); per super-block d = max scale / 63 and dmin = max min
    / 63, both stored as fp16; 6-bit codes sc_j = round(scale_j / d),
    m_j = round(min_j / dmin); element codes round((x + dmin m_j) / (d sc_j))
    clamped to 0..15.  Zero scales give zero codes."""
    *lead, n = w.shape
    assert n % 256 == 0
    b = w.reshape(*lead, n // 256, 8, 32)
    lo = b.amin(dim=-1).clamp(max=0.0)
    hi = b.amax(dim=-1)
    scale = (hi - lo) / 15.0
    mn = -lo
    d16 = (scale.amax(dim=-1) / 63.0).to(torch.float16)
    dm16 = (mn.amax(dim=-1) / 63.0).to(torch.float16)
    d, dm = d16.float().unsqueeze(-1), dm16.float().unsqueeze(-1)
    safe = lambda v: torch.where(v > 0, v, torch.ones_like(v))
    sc = torch.where(d > 0, _round_half_away(scale / safe(d)), torch.zeros_like(scale))
    m = torch.where(dm > 0, _round_half_away(mn / safe(dm)), torch.zeros_like(mn))
    sc, m = sc.clamp(0, 63), m.clamp(0, 63)
    step = (d * sc).unsqueeze(-1)
    off = (dm * m).unsqueeze(-1)
    q = torch.where(step > 0, _round_half_away((b + off) / safe(step)), torch.zeros_like(b))
    q = q.clamp(0, 15).to(torch.uint8).reshape(*lead, n // 256, 4, 2, 32)
    qs = (q[..., 0, :] | (q[..., 1, :] << 4)).reshape(*lead, n // 256, 128)
    sc, m = sc.to(torch.uint8), m.to(torch.uint8)
    packed = torch.cat([sc[..., :4] | ((sc[..., 4:] >> 4) << 6),
                        m[..., :4] | ((m[..., 4:] >> 4) << 6),
                        (sc[..., 4:] & 15) | ((m[..., 4:] & 15) << 4)], dim=-1)
    hdr = torch.stack([d16, dm16], dim=-1).view(torch.int16).view(torch.uint8)
    out = torch.cat([hdr.reshape(*lead, n // 256, 4), packed, qs], dim=-1)
    return out.reshape(*lead, n // 256 * 144).contiguous()


def quantize_q6_k(w: torch.Tensor) -> torch.Tensor:
    """fp32 [..., n] -> uint8 [..., n/256*210] (GGUF Q6_K super-blocks).
    Per 16-element sub-block j: m_j = the element of largest magnitude (sign
    kept) and s_j = m_j / -32, so m_j is code 0; per super-block d = max |s_j|
    / 127 as fp16 and int8 scales sc_j = s_j / d rounded away from zero (so
    |d sc_j| >= |s_j| and every element is within 32 steps); element codes
    round(x / (d sc_j)) + 32 clamped to 0..63.  Zero scales give code 32."""
    *lead, n = w.shape
    assert n % 256 == 0
    b = w.reshape(*lead, n // 256, 16, 16)
    idx = b.abs().argmax(dim=-1, keepdim=True)
    m = torch.gather(b, -1, idx).squeeze(-1)
    s = m / -32.0
    d16 = (s.abs().amax(dim=-1) / 127.0).to(torch.float16)
    d = d16.float().unsqueeze(-1)
    safe = lambda v: torch.where(v != 0, v, torch.ones_like(v))
    r = s / safe(d)
    sc = torch.where(d > 0, torch.sign(r) * torch.ceil(r.abs()), torch.zeros_like(s)).clamp(-127, 127)
    step = (d * sc).unsqueeze(-1)
    q = torch.where(step != 0, _round_half_away(b / safe(step)), torch.zeros_like(b)) + 32
    q = q.clamp(0, 63).to(torch.int64).reshape(*lead, n // 256, 2, 4, 32)   # [h][k][l]
    lo, hi = q & 15, q >> 4
    ql = torch.stack([lo[..., 0, :] | (lo[..., 2, :] << 4),
                      lo[..., 1, :] | (lo[..., 3, :] << 4)], dim=-2)         # [h][k%2][l]
    qh = hi[..., 0, :] | (hi[..., 1, :] << 2) | (hi[..., 2, :] << 4) | (hi[..., 3, :] << 6)
    scb = sc.to(torch.int8).view(torch.uint8)
    d8 = d16.view(torch.int16).view(torch.uint8).reshape(*lead, n // 256, 2)
    out = torch.cat([ql.reshape(*lead, n // 256, 128).to(torch.uint8),
                     qh.reshape(*lead, n // 256, 64).to(torch.uint8), scb, d8], dim=-1)
    return out.reshape(*lead, n // 256 * 210).contiguous()


# E2M1 magnitudes by code (bits 2..0); bit 3 is the sign
E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def quantize_mxfp4(w: torch.Tensor) -> torch.Tensor:
    """fp32 [R, n] -> uint8 [R*n/2 + R*n/32]: the MLX MXFP4 codes of all rows,
    then their scales.  Per 32-element group (OCP MX): shared exponent
    e = floor(log2(amax)) - 2 (E2M1's largest exponent), scale byte e + 127
    clamped to 0..254; codes: the nearest E2M1 value to x / 2^e (ties to the
    smaller magnitude), saturating at 6.  All-zero groups: scale 0, codes 0."""
    R, n = w.shape
    assert n % 32 == 0
    b = w.reshape(R, n // 32, 32)
    amax = b.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax,
                                                                  torch.ones_like(amax)))) - 2,
                    torch.full_like(amax, -127.0)).clamp(-127, 127)
    y = b / torch.exp2(e).unsqueeze(-1)
    mag = torch.tensor(E2M1, dtype=torch.float32, device=w.device)
    dist = (y.abs().unsqueeze(-1) - mag).abs()            # [R, G, 32, 8]
    k = dist.argmin(dim=-1)                               # first (smaller) on ties
    code = (k | torch.where(y < 0, 8, 0)).to(torch.uint8).reshape(R, n)
    codes = (code[:, 0::2] | (code[:, 1::2] << 4)).reshape(-1)
    scales = (e + 127).to(torch.uint8).reshape(-1)
    return torch.cat([codes, scales]).contiguous()


QUANTIZERS = {Q8_0: quantize_q8_0, Q4_0: quantize_q4_0, Q4_K: quantize_q4_k,
              Q6_K: quantize_q6_k, MXFP4: quantize_mxfp4}


def quantized_normal(rows, cols, std, qtype, seed, device):
    return QUANTIZERS[qtype](normal((rows, cols), std, seed, device))


def to_act_dtype(t: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == F32:
        return t.contiguous()
    if dtype == BF16:
        return t.to(torch.bfloat16).contiguous()   # round to nearest even
    raise ValueError(dtype)


@dataclass
class Layer:
    cfg: LayerConfig
    router: torch.Tensor            # [E][H] f32|bf16
    bias: Optional[torch.Tensor]    # [E] f32 or None
    w_gate: torch.Tensor            # uint8 [E][F][H/32*Bq]
    w_up: torch.Tensor              # uint8 [E][F][H/32*Bq]
    w_down: torch.Tensor            # uint8 [E][H][F/32*Bq]
    s_gate: Optional[torch.Tensor] = None   # uint8 [Fs][H/32*Bs]
    s_up: Optional[torch.Tensor] = None
    s_down: Optional[torch.Tensor] = None   # uint8 [H][Fs/32*Bs]

    def to(self, device):
        f = lambda t: None if t is None else t.to(device)
        return Layer(self.cfg, f(self.router), f(self.bias), f(self.w_gate),
                     f(self.w_up), f(self.w_down), f(self.s_gate), f(self.s_up),
                     f(self.s_down))


def zipf_bias(n_experts: int, s: float) -> torch.Tensor:
    """b_e = -s*ln(e+1): expert 0 hottest."""
    return torch.tensor([-s * math.log(e + 1) for e in range(n_experts)],
                        dtype=torch.float32)


def make_layer(cfg: LayerConfig, device="cpu", qtype: Optional[str] = None) -> Layer:
    """All weights of one layer.  `qtype` overrides the routed-expert format
    (the sweep runs the same fp32 samples through both quantizers)."""
    H, E, F = cfg.hidden, cfg.n_experts, cfg.ffn
    q = qtype or cfg.expert_q
    c = cfg.cid
    router = to_act_dtype(normal((E, H), cfg.router_std, seed_of(c, T_ROUTER, 0), device),
                          cfg.router_dtype)
    bias = zipf_bias(E, cfg.zipf).to(device) if cfg.zipf else None
    if q == MXFP4:
        # one matrix per projection over all experts' rows: codes, then scales
        def stack(rows, cols, tid):
            m = torch.empty(E * rows * (cols // 2 + cols // 32), dtype=torch.uint8, device=device)
            cb, sb = rows * cols // 2, rows * cols // 32
            for e in range(E):
                one = quantized_normal(rows, cols, cfg.w_std, q, seed_of(c, tid, e), device)
                m[e * cb:(e + 1) * cb] = one[:cb]
                m[E * rows * cols // 2 + e * sb:E * rows * cols // 2 + (e + 1) * sb] = one[cb:]
            return m
        wg, wu, wd = stack(F, H, T_GATE), stack(F, H, T_UP), stack(H, F, T_DOWN)
    else:
        wg = torch.empty((E, F, row_bytes(q, H)), dtype=torch.uint8, device=device)
        wu = torch.empty_like(wg)
        wd = torch.empty((E, H, row_bytes(q, F)), dtype=torch.uint8, device=device)
        for e in range(E):
            wg[e] = quantized_normal(F, H, cfg.w_std, q, seed_of(c, T_GATE, e), device)
            wu[e] = quantized_normal(F, H, cfg.w_std, q, seed_of(c, T_UP, e), device)
            wd[e] = quantized_normal(H, F, cfg.w_std, q, seed_of(c, T_DOWN, e), device)
    layer = Layer(cfg, router, bias, wg, wu, wd)
    if cfg.shared_ffn:
        Fs, qs = cfg.shared_ffn, cfg.shared_q
        layer.s_gate = quantized_normal(Fs, H, cfg.w_std, qs, seed_of(c, T_SGATE, 0), device)
        layer.s_up = quantized_normal(Fs, H, cfg.w_std, qs, seed_of(c, T_SUP, 0), device)
        layer.s_down = quantized_normal(H, Fs, cfg.w_std, qs, seed_of(c, T_SDOWN, 0), device)
    return layer


def make_x(cfg: LayerConfig, T: int, device="cpu", variant: int = 0) -> torch.Tensor:
    """[T][H] activations, N(0,1) rounded to the activation dtype."""
    return to_act_dtype(normal((T, cfg.hidden), 1.0,
                               seed_of(cfg.cid, T_X, T + 100003 * variant), device),
                        cfg.act_dtype)


def as_numpy_bits(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Host copy with bf16 exposed as its uint16 bit pattern (numpy has no bf16)."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
