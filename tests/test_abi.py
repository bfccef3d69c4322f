"""The C ABI without a GPU: the library loads, exports every function that
include/fwmoe.h declares, and refuses bad arguments synchronously (these calls
return before touching the HIP runtime)."""

import ctypes
import os
import re

import pytest

from sparse_moe_block_amd import fwmoe as fw

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "fwmoe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fw_moe_\w+)\s*\(", src)))


def test_header_functions_are_exported():
    names = declared_functions()
    assert "fw_moe_route" in names and "fw_moe_permute" in names and "fw_moe_forward" in names
    lib = ctypes.CDLL(fw.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in fwmoe.h but not exported"


def good_desc(**kw):
    d = dict(hidden=2048, n_experts=128, top_k=8, ffn=768, act_dtype="bf16",
             expert_q="q4_0", score="softmax")
    d.update(kw)
    return fw.make_desc(**d)


@pytest.mark.parametrize("field,value", [
    ("hidden", 300), ("hidden", 0), ("hidden", 16640), ("n_experts", 0), ("n_experts", 513),
    ("top_k", 0), ("top_k", 17), ("ffn", 100), ("ffn", 0), ("act_dtype", 7), ("expert_q", 5),
    ("expert_q", 99), ("expert_q", -1), ("shared_q", 5), ("score", 3)])
def test_invalid_descriptors(field, value):
    d = good_desc()
    setattr(d, field, value)
    assert fw.fw_moe_validate(d) == fw.FW_EINVAL
    assert fw.fw_moe_workspace_size(d, 16) == 0


def test_top_k_above_experts_and_mixed_dtypes():
    assert fw.fw_moe_validate(good_desc(n_experts=4, top_k=5)) == fw.FW_EINVAL
    assert fw.fw_moe_validate(good_desc(act_dtype="f32", router_dtype="bf16")) == \
        fw.FW_EUNSUPPORTED
    assert fw.fw_moe_validate(good_desc()) == fw.FW_OK
    assert fw.fw_moe_validate(good_desc(shared_ffn=2048, shared_q="q8_0")) == fw.FW_OK
    assert fw.fw_moe_validate(good_desc(expert_q="q4_k")) == fw.FW_OK
    assert fw.fw_moe_validate(good_desc(expert_q="q4_k", shared_ffn=2048,
                                        shared_q="q4_k")) == fw.FW_OK
    assert fw.fw_moe_validate(good_desc(expert_q="q6_k", shared_ffn=2048,
                                        shared_q="q6_k")) == fw.FW_OK
    assert fw.fw_moe_validate(good_desc(expert_q="mxfp4", shared_ffn=2048,
                                        shared_q="mxfp4")) == fw.FW_OK
    assert fw.fw_moe_validate(good_desc(expert_q=5)) == fw.FW_EINVAL


def test_workspace_size_grows_with_T():
    d = good_desc()
    sizes = [fw.fw_moe_workspace_size(d, T) for T in (0, 1, 16, 2048)]
    assert sizes[0] > 0 and sizes == sorted(sizes) and sizes[3] > sizes[2]
    assert fw.fw_moe_workspace_size(d, -1) == 0


def test_path_choice():
    d = good_desc()
    assert fw.fw_moe_forward_path(d, 1) == fw.FW_PATH_GEMV
    assert fw.fw_moe_forward_path(d, 4096) == fw.FW_PATH_GEMM
    # the measured decode-to-prefill crossover of the sweep layer lies between 32 and 48
    assert fw.fw_moe_forward_path(d, 32) == fw.FW_PATH_GEMV
    assert fw.fw_moe_forward_path(d, 33) == fw.FW_PATH_GEMM
    # the rule follows routed rows per expert (T * k <= 2 E), not T
    ds = good_desc(hidden=7168, n_experts=256, top_k=8, ffn=2048)
    assert fw.fw_moe_forward_path(ds, 64) == fw.FW_PATH_GEMV
    assert fw.fw_moe_forward_path(ds, 65) == fw.FW_PATH_GEMM
    dt = good_desc(hidden=256, n_experts=8, top_k=2, ffn=512)
    assert fw.fw_moe_forward_path(dt, 8) == fw.FW_PATH_GEMV
    assert fw.fw_moe_forward_path(dt, 9) == fw.FW_PATH_GEMM
    assert fw.fw_moe_forward_path(good_desc(path="gemv"), 4096) == fw.FW_PATH_GEMV
    assert fw.fw_moe_forward_path(good_desc(path="gemm"), 1) == fw.FW_PATH_GEMM


def _route(d, T, x=16, w=16, logits=16, ids=16, tw=16):
    return fw.lib().fw_moe_route(ctypes.byref(d), T, x, w, None, None, logits, ids, tw, None)


def test_route_validation():
    d = good_desc()
    assert _route(d, 0) == fw.FW_OK                    # nothing to do
    assert _route(d, -1) == fw.FW_EINVAL
    assert _route(d, 4, x=None) == fw.FW_EINVAL
    assert _route(d, 4, logits=None) == fw.FW_EINVAL   # logits required without logits_in
    assert _route(d, 4, ids=None) == fw.FW_EINVAL
    assert _route(d, 4, x=24) == fw.FW_EALIGN
    bad = good_desc(hidden=100)
    assert _route(bad, 4) == fw.FW_EINVAL


def _forward(d, T, ws_bytes, ws=256, out=16, shared=(None, None, None), x=16):
    P = ctypes.c_void_p
    return fw.lib().fw_moe_forward(ctypes.byref(d), T, x, 16, 16, 16, *shared, 16, 16, 16,
                                   16, out, ws, ws_bytes, None)


def test_forward_validation():
    d = good_desc()
    need = fw.fw_moe_workspace_size(d, 8)
    assert _forward(d, 0, 0) == fw.FW_OK
    assert _forward(d, 8, need, x=None) == fw.FW_EINVAL
    assert _forward(d, 8, need, out=None) == fw.FW_EINVAL
    assert _forward(d, 8, need, out=20) == fw.FW_EALIGN
    assert _forward(d, 8, need, ws=128) == fw.FW_EALIGN
    assert _forward(d, 8, need - 1) == fw.FW_EWORKSPACE
    ds = good_desc(shared_ffn=768)
    assert _forward(ds, 8, fw.fw_moe_workspace_size(ds, 8)) == fw.FW_EINVAL   # no shared weights


def _layer(d, T, ws_bytes, ws=256, x=16, router=16, logits=16, ids=16, out=16,
           shared=(None, None, None)):
    return fw.lib().fw_moe_layer(ctypes.byref(d), T, x, router, None, 16, 16, 16, *shared,
                                 logits, ids, 16, 16, 16, 16, out, ws, ws_bytes, None)


def test_layer_validation():
    """Every refusal of fw_moe_layer happens before its first launch."""
    d = good_desc()
    need = fw.fw_moe_workspace_size(d, 8)
    assert _layer(d, 0, 0) == fw.FW_OK                       # nothing to do
    assert _layer(d, -1, need) == fw.FW_EINVAL
    assert _layer(good_desc(hidden=100), 8, need) == fw.FW_EINVAL
    assert _layer(d, 8, need, router=None) == fw.FW_EINVAL
    assert _layer(d, 8, need, logits=None) == fw.FW_EINVAL   # logits are always written
    assert _layer(d, 8, need, x=None) == fw.FW_EINVAL
    assert _layer(d, 8, need, out=None) == fw.FW_EINVAL
    assert _layer(d, 8, need, ids=24) == fw.FW_EALIGN
    assert _layer(d, 8, need, router=40) == fw.FW_EALIGN
    assert _layer(d, 8, need, ws=128) == fw.FW_EALIGN
    assert _layer(d, 8, need - 1) == fw.FW_EWORKSPACE
    ds = good_desc(shared_ffn=768)
    assert _layer(ds, 8, fw.fw_moe_workspace_size(ds, 8)) == fw.FW_EINVAL   # no shared weights


def test_forward_batch_limit():
    """T * k * max(H, F, Fs) must stay below 2^31 (32-bit row offsets)."""
    d = good_desc(hidden=7168, n_experts=256, top_k=8, ffn=2048)
    t_max = ((1 << 31) - 1) // (8 * 7168)
    assert t_max == 37449
    assert fw.fw_moe_forward_path(d, t_max) == fw.FW_PATH_GEMM
    assert fw.fw_moe_forward_path(d, t_max + 1) == fw.FW_EINVAL
    big = t_max + 1
    need = fw.fw_moe_workspace_size(d, big)
    assert need > 0      # route / permute are not limited by it
    assert _forward(d, big, need) == fw.FW_EINVAL
    assert _layer(d, big, need) == fw.FW_EINVAL
    # a wide shared expert sets the bound too
    ds = good_desc(hidden=256, n_experts=8, top_k=1, ffn=256, shared_ffn=16384)
    assert fw.fw_moe_forward_path(ds, (1 << 31) // 16384) == fw.FW_EINVAL
    assert fw.fw_moe_forward_path(ds, (1 << 31) // 16384 - 1) in (fw.FW_PATH_GEMV,
                                                                  fw.FW_PATH_GEMM)


def test_permute_validation():
    d = good_desc()
    lib = fw.lib()
    assert lib.fw_moe_permute(ctypes.byref(d), 4, 16, 16, 16, 16, 256, 255, None) == \
        fw.FW_EWORKSPACE
    assert lib.fw_moe_permute(ctypes.byref(d), 4, 16, None, 16, 16, 256, 256, None) == \
        fw.FW_EINVAL
    assert lib.fw_moe_permute(ctypes.byref(d), 4, 16, 16, 16, 16, 64, 256, None) == \
        fw.FW_EALIGN
    # above 2048 pairs the sort needs the full workspace (checked before launching)
    T = 4096 // d.top_k
    assert lib.fw_moe_permute(ctypes.byref(d), T, 16, 16, 16, 16, 256, 256, None) == \
        fw.FW_EWORKSPACE


def test_status_strings_and_version():
    for code in (fw.FW_OK, fw.FW_EINVAL, fw.FW_EUNSUPPORTED, fw.FW_EWORKSPACE, fw.FW_EALIGN,
                 fw.FW_EHIP):
        assert fw.fw_moe_status_string(code) != "unknown status"
    assert fw.fw_moe_status_string(99) == "unknown status"
    assert "gfx950" in fw.fw_moe_version()


def test_layer_timed_validation():
    """fw_moe_layer_timed takes its events per call: missing events are
    refused before anything is enqueued, and so is everything fw_moe_layer
    refuses."""
    d = good_desc()
    need = fw.fw_moe_workspace_size(d, 8)
    lib = fw.lib()
    ev = (ctypes.c_void_p * fw.FW_N_STAGE_EVENTS)(*([16] * fw.FW_N_STAGE_EVENTS))
    ev_missing = (ctypes.c_void_p * fw.FW_N_STAGE_EVENTS)(*([16] * 4 + [None]))

    def call(events, T=8, router=16, ws=256):
        return lib.fw_moe_layer_timed(ctypes.byref(d), T, 16, router, None, 16, 16, 16, None,
                                      None, None, 16, 16, 16, 16, 16, 16, 16, ws, need, events,
                                      None)
    assert call(None) == fw.FW_EINVAL
    assert call(ev_missing) == fw.FW_EINVAL
    assert call(ev, router=None) == fw.FW_EINVAL
    assert call(ev, ws=128) == fw.FW_EALIGN
    assert call(ev, T=-1) == fw.FW_EINVAL


def test_mx8_mode_refusals():
    """MXFP8 activations need MXFP4 experts (and an MXFP4 shared expert) and
    the grouped-GEMM family; AUTO takes the GEMM at every T."""
    def d(**kw):
        base = dict(hidden=2048, n_experts=128, top_k=8, ffn=768, expert_q="mxfp4",
                    act_quant="mxfp8")
        base.update(kw)
        return fw.make_desc(**base)
    assert fw.fw_moe_validate(d()) == fw.FW_OK
    assert fw.fw_moe_validate(d(expert_q="q4_0")) == fw.FW_EUNSUPPORTED
    assert fw.fw_moe_validate(d(shared_ffn=256, shared_q="q8_0")) == fw.FW_EUNSUPPORTED
    assert fw.fw_moe_validate(d(shared_ffn=256, shared_q="mxfp4")) == fw.FW_OK
    assert fw.fw_moe_validate(d(path="gemv")) == fw.FW_EUNSUPPORTED
    assert fw.fw_moe_validate(d(act_quant=3)) == fw.FW_EINVAL
    assert fw.fw_moe_validate(d(act_quant=-1)) == fw.FW_EINVAL
    assert fw.fw_moe_forward_path(d(), 1) == fw.FW_PATH_GEMM
    assert fw.fw_moe_forward_path(d(), 4096) == fw.FW_PATH_GEMM


def test_int8_mode_refusals():
    """int8 activations need Q8_0 or Q4_0 experts (and shared expert) and the
    grouped-GEMM family; AUTO takes the GEMM at every T."""
    def d(**kw):
        base = dict(hidden=2048, n_experts=128, top_k=8, ffn=768, expert_q="q4_0",
                    act_quant="int8")
        base.update(kw)
        return fw.make_desc(**base)
    assert fw.fw_moe_validate(d()) == fw.FW_OK
    assert fw.fw_moe_validate(d(expert_q="q8_0")) == fw.FW_OK
    for q in ("q4_k", "q6_k", "mxfp4"):
        assert fw.fw_moe_validate(d(expert_q=q)) == fw.FW_EUNSUPPORTED
        assert fw.fw_moe_validate(d(shared_ffn=256, shared_q=q)) == fw.FW_EUNSUPPORTED
    assert fw.fw_moe_validate(d(shared_ffn=256, shared_q="q8_0")) == fw.FW_OK
    assert fw.fw_moe_validate(d(path="gemv")) == fw.FW_EUNSUPPORTED
    assert fw.fw_moe_validate(d(path="gemm")) == fw.FW_OK
    assert fw.fw_moe_forward_path(d(), 1) == fw.FW_PATH_GEMM
    assert fw.fw_moe_forward_path(d(), 4096) == fw.FW_PATH_GEMM
