"""Descriptor extremes the C ABI accepts, through every path, against the CPU
oracle: the smallest hidden and ffn sizes with the most experts and the
largest top-k; the largest hidden size with top-1 sigmoid routing; unit counts
that split unevenly (3 and 5 units per row), k = E and a Q4_0 shared expert;
a single expert with fp32 activations and router (a dense SwiGLU FFN)."""

import numpy as np
import pytest
import torch

import moegen
from moegen.configs import LayerConfig
from sparse_moe_block_amd import fwmoe as fw
from tests import gpu_util as G
from tests.test_gpu_fused_layer import _one_call, _three_calls

pytestmark = pytest.mark.gpu

C = moegen
EDGE_MIN = LayerConfig(5, "edge: H=256 F=256 E=512 k=16", 256, 512, 16, 256, C.Q8_0, C.BF16,
                       C.BF16, C.SOFTMAX, 0.02)
EDGE_WIDE = LayerConfig(6, "edge: H=16384 E=4 k=1 sigmoid", 16384, 4, 1, 256, C.Q4_0, C.BF16,
                        C.BF16, C.SIGMOID, 0.01)
EDGE_RAGGED = LayerConfig(7, "edge: H=768 F=1280 E=k=3 shared q4_0", 768, 3, 3, 1280, C.Q4_0,
                          C.BF16, C.BF16, C.SOFTMAX, 0.02, shared_ffn=512, shared_q=C.Q4_0)
EDGE_ONE = LayerConfig(8, "edge: E=1 k=1 f32", 512, 1, 1, 512, C.Q8_0, C.F32, C.F32, C.SOFTMAX,
                       0.02)
CASES = [(c, T) for c, Ts in [(EDGE_MIN, (1, 7, 33)), (EDGE_WIDE, (1, 5, 40)),
                              (EDGE_RAGGED, (1, 9, 70)), (EDGE_ONE, (3, 100))] for T in Ts]
IDS = [f"c{c.cid}-T{T}" for c, T in CASES]


@pytest.mark.parametrize("path", ["auto", "gemv", "gemm"])
@pytest.mark.parametrize("cfg,T", CASES, ids=IDS)
def test_edge_shape(ref, cfg, T, path):
    print(f"edge {cfg.name} T={T} path={path}", flush=True)
    dl = G.layer(cfg)
    desc = G.desc_of(cfg, path=path)
    x = moegen.make_x(cfg, T, device=G.DEV)
    xh = moegen.as_numpy_bits(x)
    one = _one_call(desc, cfg, dl, x)
    sep = _three_calls(desc, cfg, dl, x)
    for name, a, b in zip(["logits", "ids", "w", "offsets", "sorted", "inv", "out"], sep, one):
        assert torch.equal(a, b), f"{name}: fw_moe_layer differs from the three calls"
    logits, ids, w, off, _, _, out = (t.cpu().numpy() for t in one[:7])
    rl, rids, rw = G.oracle_route(ref, cfg, dl, xh)
    assert np.abs(logits - rl).max() <= G.LOGIT_MAX_ABS
    assert np.abs(w.astype(np.float64).sum(axis=1) - 1).max() <= 1e-5
    # tokens without a near tie: the oracle's selection and weights exactly
    ok = ~G.small_gaps(rl, cfg.top_k)
    if ok.any():
        assert np.array_equal(ids[ok], rids[ok])
        assert np.abs(w[ok] - rw[ok]).max() <= G.W_MAX_ABS
    # near ties (512 experts make them common): the selection is still a top-k
    # of the oracle's logits up to the gap, without repeats
    for t in np.nonzero(~ok)[0]:
        sel = ids[t]
        assert len(set(sel.tolist())) == cfg.top_k and sel.min() >= 0
        rest = np.setdiff1d(np.arange(cfg.n_experts), sel)
        if rest.size:
            assert rl[t, sel].min() >= rl[t, rest].max() - G.GAP
    roff, _, _ = ref.permute(ids, cfg.n_experts)     # the GPU's own ids
    assert np.array_equal(off, roff)
    # every token's output against the oracle's forward on the same routing
    want = G.oracle_forward(ref, cfg, dl, xh, ids, w)
    G.check_out(out, want)
