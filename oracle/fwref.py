"""ctypes wrapper of the CPU oracle library (liboracle.so, built from fwref.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU path.  Arguments are numpy
arrays in host memory; bf16 tensors travel as their uint16 bit patterns.
"""

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FWREF_LIB") or os.path.join(HERE, "liboracle.so")
SRC_PATH = os.path.join(HERE, "fwref.c")

REF_F32, REF_BF16 = 0, 1
REF_Q8_0, REF_Q4_0, REF_Q4_K, REF_Q6_K, REF_MXFP4 = 0, 1, 2, 3, 4
REF_SOFTMAX, REF_SIGMOID = 0, 1
DTYPE = {"f32": REF_F32, "bf16": REF_BF16}
QTYPE = {"q8_0": REF_Q8_0, "q4_0": REF_Q4_0, "q4_k": REF_Q4_K, "q6_k": REF_Q6_K,
         "mxfp4": REF_MXFP4}
SCORE = {"softmax": REF_SOFTMAX, "sigmoid": REF_SIGMOID}

GCC_CMD = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", SRC_PATH, "-o", LIB_PATH, "-lm"]

_lib = None


def build():
    subprocess.check_call(GCC_CMD)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P, I = ctypes.c_void_p, ctypes.c_int
        L.fwref_half_to_float.argtypes = [ctypes.c_uint16]
        L.fwref_half_to_float.restype = ctypes.c_float
        L.fwref_bf16_to_float.argtypes = [ctypes.c_uint16]
        L.fwref_bf16_to_float.restype = ctypes.c_float
        L.fwref_dequant_row.argtypes = [I, P, I, P]
        L.fwref_dequant_row.restype = None
        L.fwref_route.argtypes = [I] * 7 + [P] * 7
        L.fwref_route.restype = I
        L.fwref_permute.argtypes = [I, I, I, P, P, P, P]
        L.fwref_permute.restype = I
        L.fwref_forward.argtypes = [I] * 9 + [P] * 10 + [I]
        L.fwref_forward.restype = I
        L.fwref_forward_mx8.argtypes = [I] * 9 + [P] * 10 + [I]
        L.fwref_forward_mx8.restype = I
        L.fwref_forward_q8a.argtypes = [I] * 9 + [P] * 10 + [I]
        L.fwref_forward_q8a.restype = I
        L.fwref_q8a_quantize.argtypes = [P, I, P, P]
        L.fwref_q8a_quantize.restype = None
        L.fwref_mxfp8_quantize.argtypes = [P, I, P, P]
        L.fwref_mxfp8_quantize.restype = None
        L.fwref_e4m3_value.argtypes = [I]
        L.fwref_e4m3_value.restype = ctypes.c_double
        L.fwref_threads.argtypes = [I]
        L.fwref_threads.restype = I
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arguments must be C-contiguous"
    return a.ctypes.data


def half_to_float(h: int) -> float:
    return lib().fwref_half_to_float(h)


def bf16_to_float(b: int) -> float:
    return lib().fwref_bf16_to_float(b)


def dequant_row(qtype: str, row: np.ndarray, n: int) -> np.ndarray:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    out = np.empty(n, dtype=np.float32)
    lib().fwref_dequant_row(QTYPE[qtype], _p(row), n, _p(out))
    return out


def route(x, router_w, bias, *, k, act_dtype, router_dtype, score, logits_in=None):
    """x [T][H], router_w [E][H] (float32 or uint16 bf16 bits), bias [E] or None.
    Returns (logits [T][E] f32, ids [T][k] i32, w [T][k] f32)."""
    T, H = x.shape
    E = router_w.shape[0]
    logits = np.empty((T, E), dtype=np.float32)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
    if logits_in is not None:
        logits_in = np.ascontiguousarray(logits_in, dtype=np.float32)
    rc = lib().fwref_route(T, H, E, k, DTYPE[act_dtype], DTYPE[router_dtype], SCORE[score],
                           _p(np.ascontiguousarray(x)), _p(np.ascontiguousarray(router_w)),
                           _p(bias), _p(logits_in), _p(logits), _p(ids), _p(w))
    if rc != 0:
        raise ValueError("fwref_route rejected its arguments")
    return logits, ids, w


def permute(ids, n_experts):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    offsets = np.empty(n_experts + 1, dtype=np.int32)
    sorted_pairs = np.empty(T * k, dtype=np.int32)
    inv_pos = np.empty(T * k, dtype=np.int32)
    rc = lib().fwref_permute(T, n_experts, k, _p(ids), _p(offsets), _p(sorted_pairs),
                             _p(inv_pos))
    if rc != 0:
        raise ValueError("fwref_permute: expert id out of range")
    return offsets, sorted_pairs, inv_pos


def e4m3_value(code: int) -> float:
    return lib().fwref_e4m3_value(code)


def mxfp8_quantize(v: np.ndarray):
    """fp32 [n] (n a multiple of 32) -> (E4M3 codes uint8 [n], E8M0 scales uint8 [n/32])."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    assert v.ndim == 1 and v.size % 32 == 0
    codes = np.empty(v.size, dtype=np.uint8)
    scales = np.empty(v.size // 32, dtype=np.uint8)
    lib().fwref_mxfp8_quantize(_p(v), v.size, _p(codes), _p(scales))
    return codes, scales


def q8a_quantize(v: np.ndarray):
    """fp32 [n] (n a multiple of 32) -> (int8 codes [n], fp32 scales [n/32])."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    assert v.ndim == 1 and v.size % 32 == 0
    codes = np.empty(v.size, dtype=np.int8)
    scales = np.empty(v.size // 32, dtype=np.float32)
    lib().fwref_q8a_quantize(_p(v), v.size, _p(codes), _p(scales))
    return codes, scales


def forward(x, w_gate, w_up, w_down, ids, w, *, n_experts, ffn, qtype, act_dtype,
            s_gate=None, s_up=None, s_down=None, shared_ffn=0, shared_q="q8_0",
            n_threads=0, act_quant="none"):
    """Layer output [T][H] f32 for tokens x with routing (ids, w).  act_quant
    "mxfp8": the experts' inputs (x, and the SwiGLU output before the down
    projection) are MXFP8 round trips (MXFP4 experts only); "int8": they are
    int8 round trips, d = amax / 127 per 32 (Q8_0 / Q4_0 experts only)."""
    T, H = x.shape
    k = ids.shape[1]
    out = np.empty((T, H), dtype=np.float32)
    c = np.ascontiguousarray
    fn = {"none": lib().fwref_forward, "mxfp8": lib().fwref_forward_mx8,
          "int8": lib().fwref_forward_q8a}[act_quant]
    rc = fn(
        T, H, n_experts, k, ffn, QTYPE[qtype], shared_ffn, QTYPE[shared_q],
        DTYPE[act_dtype], _p(c(x)), _p(c(w_gate)), _p(c(w_up)), _p(c(w_down)),
        _p(None if s_gate is None else c(s_gate)), _p(None if s_up is None else c(s_up)),
        _p(None if s_down is None else c(s_down)), _p(c(ids, dtype=np.int32)),
        _p(c(w, dtype=np.float32)), _p(out), n_threads)
    if rc != 0:
        raise ValueError("fwref_forward rejected its arguments")
    return out


def threads(n_threads=0):
    return lib().fwref_threads(n_threads)
