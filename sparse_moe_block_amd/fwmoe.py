"""Python binding of libfwmoe.so: the C ABI of include/fwmoe.h, one function per
entry point with the same name.  Argument marshalling only -- torch tensors (or
None) become device pointers, the stream defaults to torch's current stream --
and a non-zero return code raises FwMoeError.  Every step of the layer runs in
the HIP kernels of the library; there is no other implementation behind these
calls, and a missing library is an error."""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfwmoe.so")

FW_OK, FW_EINVAL, FW_EUNSUPPORTED, FW_EWORKSPACE, FW_EALIGN, FW_EHIP = 0, -1, -2, -3, -4, -5
FW_STATUS_BAD_EXPERT_ID, FW_STATUS_BAD_OFFSETS, FW_STATUS_BAD_PAIR, FW_STATUS_RANGE = 1, 2, 4, 8
FW_F32, FW_BF16 = 0, 1
FW_Q8_0, FW_Q4_0, FW_Q4_K, FW_Q6_K, FW_MXFP4 = 0, 1, 2, 3, 4
FW_SOFTMAX_RENORM, FW_SIGMOID_RENORM = 0, 1
FW_PATH_AUTO, FW_PATH_GEMV, FW_PATH_GEMM = 0, 1, 2
FW_N_STAGE_EVENTS = 6
FW_NOALLOC_SCRATCH_BYTES = 64 << 20

DTYPES = {"f32": FW_F32, "bf16": FW_BF16}
QTYPES = {"q8_0": FW_Q8_0, "q4_0": FW_Q4_0, "q4_k": FW_Q4_K, "q6_k": FW_Q6_K,
          "mxfp4": FW_MXFP4}
SCORES = {"softmax": FW_SOFTMAX_RENORM, "sigmoid": FW_SIGMOID_RENORM}
PATHS = {"auto": FW_PATH_AUTO, "gemv": FW_PATH_GEMV, "gemm": FW_PATH_GEMM}
FW_ACT_NONE, FW_ACT_MXFP8, FW_ACT_INT8 = 0, 1, 2
ACT_QUANTS = {"none": FW_ACT_NONE, "mxfp8": FW_ACT_MXFP8, "int8": FW_ACT_INT8}


class FwMoeError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} returned {code} ({status_string(code)})")
        self.code = code


class fw_moe_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "n_experts", "top_k", "ffn", "shared_ffn", "act_dtype", "router_dtype",
        "expert_q", "shared_q", "score", "path", "act_quant")]


def make_desc(hidden, n_experts, top_k, ffn, shared_ffn=0, act_dtype="bf16",
              router_dtype=None, expert_q="q4_0", shared_q="q8_0", score="softmax",
              path="auto", act_quant="none"):
    """A descriptor from readable names (dtype / format / score / path strings
    or the FW_* integers)."""
    enum = lambda table, v: table[v] if isinstance(v, str) else int(v)
    return fw_moe_desc(hidden, n_experts, top_k, ffn, shared_ffn,
                       enum(DTYPES, act_dtype), enum(DTYPES, router_dtype or act_dtype),
                       enum(QTYPES, expert_q), enum(QTYPES, shared_q),
                       enum(SCORES, score), enum(PATHS, path), enum(ACT_QUANTS, act_quant))


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, I, D = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(fw_moe_desc)
        sig = {
            "fw_moe_version": ([], ctypes.c_char_p),
            "fw_moe_validate": ([D], ctypes.c_int),
            "fw_moe_workspace_size": ([D, I], ctypes.c_size_t),
            "fw_moe_forward_path": ([D, I], ctypes.c_int),
            "fw_moe_workspace_offsets": ([D, I, ctypes.POINTER(ctypes.c_size_t),
                                          ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
            "fw_moe_route": ([D, I] + [P] * 8, ctypes.c_int),
            "fw_moe_permute": ([D, I, P, P, P, P, P, ctypes.c_size_t, P], ctypes.c_int),
            "fw_moe_forward": ([D, I] + [P] * 13 + [ctypes.c_size_t, P], ctypes.c_int),
            "fw_moe_layer": ([D, I] + [P] * 17 + [ctypes.c_size_t, P], ctypes.c_int),
            "fw_moe_clear_status": ([P, P], ctypes.c_int),
            "fw_moe_read_status": ([P, ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
            "fw_moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "fw_moe_layer_timed": ([D, I] + [P] * 17 + [ctypes.c_size_t, P, P], ctypes.c_int),
            "fw_moe_layer_noalloc": ([D, I] + [P] * 17 + [P], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, code):
    if code != FW_OK:
        raise FwMoeError(fn, code)
    return code


def fw_moe_version():
    return lib().fw_moe_version().decode()


def fw_moe_validate(desc):
    return lib().fw_moe_validate(ctypes.byref(desc))


def fw_moe_workspace_size(desc, max_T):
    return lib().fw_moe_workspace_size(ctypes.byref(desc), max_T)


def fw_moe_forward_path(desc, T):
    return lib().fw_moe_forward_path(ctypes.byref(desc), T)


def fw_moe_workspace_offsets(desc, T):
    """(x staging, h staging) byte offsets inside a workspace for T tokens."""
    xo, ho = ctypes.c_size_t(), ctypes.c_size_t()
    _check("fw_moe_workspace_offsets", lib().fw_moe_workspace_offsets(
        ctypes.byref(desc), T, ctypes.byref(xo), ctypes.byref(ho)))
    return xo.value, ho.value


def fw_moe_route(desc, T, x, router_w, logit_bias, logits_in, logits, topk_ids, topk_w,
                 stream=None):
    return _check("fw_moe_route", lib().fw_moe_route(
        ctypes.byref(desc), T, _ptr(x), _ptr(router_w), _ptr(logit_bias), _ptr(logits_in),
        _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _stream(stream)))


def fw_moe_permute(desc, T, topk_ids, expert_offsets, sorted_pairs, inv_pos, workspace,
                   ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    return _check("fw_moe_permute", lib().fw_moe_permute(
        ctypes.byref(desc), T, _ptr(topk_ids), _ptr(expert_offsets), _ptr(sorted_pairs),
        _ptr(inv_pos), _ptr(workspace), ws_bytes, _stream(stream)))


def fw_moe_forward(desc, T, x, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, topk_w,
                   expert_offsets, sorted_pairs, inv_pos, out, workspace, ws_bytes=None,
                   stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    return _check("fw_moe_forward", lib().fw_moe_forward(
        ctypes.byref(desc), T, _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(ws_gate),
        _ptr(ws_up), _ptr(ws_down), _ptr(topk_w), _ptr(expert_offsets), _ptr(sorted_pairs),
        _ptr(inv_pos), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))


def fw_moe_layer(desc, T, x, router_w, logit_bias, w_gate, w_up, w_down, ws_gate, ws_up,
                 ws_down, logits, topk_ids, topk_w, expert_offsets, sorted_pairs, inv_pos, out,
                 workspace, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    return _check("fw_moe_layer", lib().fw_moe_layer(
        ctypes.byref(desc), T, _ptr(x), _ptr(router_w), _ptr(logit_bias), _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), _ptr(logits),
        _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(inv_pos),
        _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))


def fw_moe_clear_status(workspace, stream=None):
    return _check("fw_moe_clear_status",
                  lib().fw_moe_clear_status(_ptr(workspace), _stream(stream)))


def fw_moe_read_status(workspace):
    v = ctypes.c_int32(0)
    _check("fw_moe_read_status", lib().fw_moe_read_status(_ptr(workspace), ctypes.byref(v)))
    return v.value


def fw_moe_status_string(code):
    return lib().fw_moe_status_string(code).decode()


status_string = fw_moe_status_string


def fw_moe_layer_timed(desc, T, x, router_w, logit_bias, w_gate, w_up, w_down, ws_gate,
                       ws_up, ws_down, logits, topk_ids, topk_w, expert_offsets, sorted_pairs,
                       inv_pos, out, workspace, stage_events, ws_bytes=None, stream=None):
    """stage_events: FW_N_STAGE_EVENTS torch.cuda.Event objects (enable_timing=True)."""
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    assert len(stage_events) == FW_N_STAGE_EVENTS
    for e in stage_events:
        if e.cuda_event == 0:      # torch creates the HIP event lazily
            e.record()
    arr = (ctypes.c_void_p * FW_N_STAGE_EVENTS)(*[e.cuda_event for e in stage_events])
    return _check("fw_moe_layer_timed", lib().fw_moe_layer_timed(
        ctypes.byref(desc), T, _ptr(x), _ptr(router_w), _ptr(logit_bias), _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), _ptr(logits),
        _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(inv_pos),
        _ptr(out), _ptr(workspace), ws_bytes, arr, _stream(stream)))


def fw_moe_layer_noalloc(desc, T, x, router_w, logit_bias, w_gate, w_up, w_down, ws_gate,
                         ws_up, ws_down, logits, topk_ids, topk_w, expert_offsets,
                         sorted_pairs, inv_pos, out, status=None, stream=None):
    """status: an int32 device tensor of one element, or None."""
    return _check("fw_moe_layer_noalloc", lib().fw_moe_layer_noalloc(
        ctypes.byref(desc), T, _ptr(x), _ptr(router_w), _ptr(logit_bias), _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), _ptr(logits),
        _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(inv_pos),
        _ptr(out), _ptr(status), _stream(stream)))
