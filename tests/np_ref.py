"""Independent numpy decoding of GGUF blocks, for float64 cross-checks of the
oracle.  Vectorised and written separately from the oracle's C loops; it is
itself pinned by the hand-decoded fixture in golden/q_blocks.txt."""

import numpy as np

BQ = {"q8_0": 34, "q4_0": 18}


def dequant(qtype, raw, n):
    """raw uint8 [..., n/32*Bq] -> float64 [..., n]."""
    raw = np.asarray(raw, dtype=np.uint8)
    lead = raw.shape[:-1]
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
