"""Pins of the oracle's expert FFN and combine: designed inputs with closed-form
outputs, reduction to a dense SwiGLU FFN checked by a float64 library product,
and exact invariants (zero / doubled scales, token permutation, linearity in
the gate weights, the shared expert's additivity)."""

import math

import numpy as np
import pytest

import moegen
from tests import np_ref

HALF = {0.25: 0x3400, 0.5: 0x3800, 1.0: 0x3C00, 2.0: 0x4000}


def q8_block(d, codes):
    b = np.zeros(34, np.uint8)
    b[0:2] = np.array([HALF[d]], np.uint16).view(np.uint8)
    b[2:] = np.array(codes, np.int8).view(np.uint8)
    return b


def q8_row(d, codes):
    """One Q8_0 row; len(codes) is a multiple of 32."""
    return np.concatenate([q8_block(d, codes[i:i + 32]) for i in range(0, len(codes), 32)])


def silu(z):
    return z / (1.0 + math.exp(-z))


def test_designed_one_hot_expert(ref):
    """H = F = 32, one expert, x = 2*e_h0.  Then g_f = d_g*cg[f]*2, u_f =
    d_u*cu[f]*2 and y_o = d_d * sum_f cd[o][f] * silu(g_f) * u_f.  Gate and up
    use different codes and scales, so swapping them, transposing a matrix or
    reading the wrong column changes the result."""
    H = F = 32
    h0 = 5
    rng = np.random.default_rng(0)
    cg = rng.integers(-6, 7, F)
    cu = rng.integers(-6, 7, F)
    cd = rng.integers(-5, 6, (H, F))
    wg = np.zeros((1, F, 34), np.uint8)
    wu = np.zeros((1, F, 34), np.uint8)
    for f in range(F):
        row_g = np.zeros(32, np.int64)
        row_g[h0] = cg[f]
        row_g[(h0 + 7) % 32] = 100          # a weight that x never touches
        row_u = np.zeros(32, np.int64)
        row_u[h0] = cu[f]
        wg[0, f] = q8_block(0.5, row_g)
        wu[0, f] = q8_block(1.0, row_u)
    wd = np.stack([q8_block(0.25, cd[o]) for o in range(H)])[None]
    x = np.zeros((1, H), np.float32)
    x[0, h0] = 2.0
    out = ref.forward(x, wg, wu, wd, np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32),
                      n_experts=1, ffn=F, qtype="q8_0", act_dtype="f32")
    a = [silu(0.5 * cg[f] * 2.0) * (1.0 * cu[f] * 2.0) for f in range(F)]
    want = [0.25 * sum(cd[o][f] * a[f] for f in range(F)) for o in range(H)]
    np.testing.assert_allclose(out[0], want, rtol=1e-6, atol=1e-6)


def test_designed_combine_and_shared(ref):
    """Two experts whose outputs are constant vectors c0, c1 (one-hot x, one
    active hidden unit) and a shared expert with output c2: out = w0*c0 +
    w1*c1 + c2, with the slot weights applied to the right experts."""
    H = F = 32

    def const_expert(gcode, ucode, dcode):
        # g_0 = 1*gcode*1, u_0 = 1*ucode*1; only hidden unit 0 is non-zero;
        # down: every output row reads unit 0 with code dcode -> y_o = dcode*a_0
        g = np.zeros((F, 34), np.uint8)
        u = np.zeros((F, 34), np.uint8)
        for f in range(F):
            g[f] = q8_block(1.0, [gcode if (f == 0 and i == 0) else 0 for i in range(32)])
            u[f] = q8_block(1.0, [ucode if (f == 0 and i == 0) else 0 for i in range(32)])
        d = np.stack([q8_block(1.0, [dcode] + [0] * 31) for _ in range(H)])
        return g, u, d, dcode * silu(gcode) * ucode

    e0 = const_expert(2, 3, 1)
    e1 = const_expert(-1, 5, 2)
    es = const_expert(1, 1, 4)
    wg = np.stack([e0[0], e1[0]])
    wu = np.stack([e0[1], e1[1]])
    wd = np.stack([e0[2], e1[2]])
    x = np.zeros((2, H), np.float32)
    x[:, 0] = 1.0
    ids = np.array([[1, 0], [0, 1]], np.int32)
    w = np.array([[0.75, 0.25], [0.5, 0.5]], np.float32)
    out = ref.forward(x, wg, wu, wd, ids, w, n_experts=2, ffn=F, qtype="q8_0",
                      act_dtype="f32", s_gate=es[0], s_up=es[1], s_down=es[2],
                      shared_ffn=F, shared_q="q8_0")
    np.testing.assert_allclose(out[0], 0.75 * e1[3] + 0.25 * e0[3] + es[3], rtol=1e-6)
    np.testing.assert_allclose(out[1], 0.5 * e0[3] + 0.5 * e1[3] + es[3], rtol=1e-6)


def _layer(qtype="q4_0", H=512, F=256, E=4, shared=0, std=0.05):
    cfg = moegen.QWEN3_DECODE.with_(hidden=H, ffn=F, n_experts=E, top_k=2, w_std=std,
                                    shared_ffn=shared)
    L = moegen.make_layer(cfg, qtype=qtype)
    return cfg, L


@pytest.mark.parametrize("H,F", [(512, 256), (256, 768)])
@pytest.mark.parametrize("qtype", ["q8_0", "q4_0", "q4_k", "q6_k", "mxfp4"])
def test_single_expert_is_dense_swiglu_float64(ref, qtype, H, F):
    """E = 1, k = 1: the layer is the textbook dense FFN
    W_d (silu(W_g x) * (W_u x)); checked with numpy float64 matrix products on
    independently decoded matrices."""
    cfg, L = _layer(qtype, H=H, F=F, E=1)
    x = moegen.as_numpy_bits(moegen.make_x(cfg, 6))
    out = ref.forward(x, L.w_gate.numpy(), L.w_up.numpy(), L.w_down.numpy(),
                      np.zeros((6, 1), np.int32), np.ones((6, 1), np.float32),
                      n_experts=1, ffn=cfg.ffn, qtype=qtype, act_dtype="bf16")
    Wg = np_ref.dequant_matrix(qtype, L.w_gate.numpy(), cfg.ffn, cfg.hidden)
    Wu = np_ref.dequant_matrix(qtype, L.w_up.numpy(), cfg.ffn, cfg.hidden)
    Wd = np_ref.dequant_matrix(qtype, L.w_down.numpy(), cfg.hidden, cfg.ffn)
    X = np_ref.act(x)
    want = (np_ref.silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-6 * np.abs(want).max())


def test_routed_layer_float64(ref):
    """The tiny workload in full against a float64 evaluation (per-pair
    library matrix products, slot-ordered combine)."""
    cfg = moegen.TINY
    L = moegen.make_layer(cfg)
    x = moegen.as_numpy_bits(moegen.make_x(cfg, 4))
    _, ids, w = ref.route(x, L.router.numpy(), None, k=cfg.top_k, act_dtype="f32",
                          router_dtype="f32", score="softmax")
    out = ref.forward(x, L.w_gate.numpy(), L.w_up.numpy(), L.w_down.numpy(), ids, w,
                      n_experts=cfg.n_experts, ffn=cfg.ffn, qtype="q8_0", act_dtype="f32")
    X = np_ref.act(x)
    want = np.zeros_like(X)
    for t in range(4):
        for j in range(cfg.top_k):
            e = ids[t, j]
            Wg = np_ref.dequant("q8_0", L.w_gate.numpy()[e], cfg.hidden)
            Wu = np_ref.dequant("q8_0", L.w_up.numpy()[e], cfg.hidden)
            Wd = np_ref.dequant("q8_0", L.w_down.numpy()[e], cfg.ffn)
            y = Wd @ (np_ref.silu(Wg @ X[t]) * (Wu @ X[t]))
            want[t] += float(w[t, j]) * y
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-6 * np.abs(want).max())


def _fwd(ref, cfg, L, x, ids, w, wd=None, **kw):
    return ref.forward(x, L.w_gate.numpy(), L.w_up.numpy(),
                       L.w_down.numpy() if wd is None else wd, ids, w,
                       n_experts=cfg.n_experts, ffn=cfg.ffn, qtype=kw.get("qtype", "q4_0"),
                       act_dtype="bf16")


def _routing(T, E, k, seed=0):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    return ids, w


def test_zero_and_doubled_down_scales(ref):
    cfg, L = _layer()
    x = moegen.as_numpy_bits(moegen.make_x(cfg, 5))
    ids, w = _routing(5, cfg.n_experts, 2)
    base = _fwd(ref, cfg, L, x, ids, w)
    wd = L.w_down.numpy().copy()
    blk = wd.reshape(-1, 18)
    d = blk[:, 0:2].copy().view(np.uint16)[:, 0]
    zero = blk.copy()
    zero[:, 0:2] = 0
    assert not np.any(_fwd(ref, cfg, L, x, ids, w, wd=zero.reshape(wd.shape)))
    # doubling an fp16 scale = adding one to its exponent (all scales here are normal)
    ex = (d >> 10) & 31
    assert np.all((ex > 0) & (ex < 30))
    dbl = blk.copy()
    dbl[:, 0:2] = (d + (1 << 10)).astype(np.uint16).view(np.uint8).reshape(-1, 2)
    assert np.array_equal(_fwd(ref, cfg, L, x, ids, w, wd=dbl.reshape(wd.shape)), 2 * base)


def test_token_permutation_and_duplication(ref):
    cfg, L = _layer()
    x = moegen.as_numpy_bits(moegen.make_x(cfg, 6))
    ids, w = _routing(6, cfg.n_experts, 2, seed=1)
    base = _fwd(ref, cfg, L, x, ids, w)
    perm = np.array([3, 3, 0, 5, 1, 2, 4, 0])
    got = _fwd(ref, cfg, L, x[perm], ids[perm], w[perm])
    assert np.array_equal(got, base[perm])


def test_linear_in_gate_weights(ref):
    cfg, L = _layer()
    x = moegen.as_numpy_bits(moegen.make_x(cfg, 4))
    ids, w = _routing(4, cfg.n_experts, 2, seed=2)
    base = _fwd(ref, cfg, L, x, ids, w)
    assert np.array_equal(_fwd(ref, cfg, L, x, ids, 2 * w), 2 * base)
    # one slot's weight zero: the output is that of the other slot alone
    w1 = w.copy()
    w1[:, 1] = 0
    alone = _fwd(ref, cfg, L, x, ids[:, :1].copy(), w[:, :1].copy())
    np.testing.assert_allclose(_fwd(ref, cfg, L, x, ids, w1), alone, rtol=1e-6, atol=1e-7)


def test_shared_expert_is_additive(ref):
    cfg, L = _layer(shared=768)
    x = moegen.as_numpy_bits(moegen.make_x(cfg, 3))
    ids, w = _routing(3, cfg.n_experts, 2, seed=3)
    routed = _fwd(ref, cfg, L, x, ids, w)
    both = ref.forward(x, L.w_gate.numpy(), L.w_up.numpy(), L.w_down.numpy(), ids, w,
                       n_experts=cfg.n_experts, ffn=cfg.ffn, qtype="q4_0", act_dtype="bf16",
                       s_gate=L.s_gate.numpy(), s_up=L.s_up.numpy(), s_down=L.s_down.numpy(),
                       shared_ffn=768, shared_q="q8_0")
    shared_alone = ref.forward(x, L.s_gate.numpy()[None], L.s_up.numpy()[None],
                               L.s_down.numpy()[None], np.zeros((3, 1), np.int32),
                               np.ones((3, 1), np.float32), n_experts=1, ffn=768,
                               qtype="q8_0", act_dtype="bf16")
    np.testing.assert_allclose(both, routed + shared_alone, rtol=0,
                               atol=2e-6 * np.abs(both).max())


def test_forward_rejects_bad_ids(ref):
    cfg, L = _layer()
    x = moegen.as_numpy_bits(moegen.make_x(cfg, 1))
    with pytest.raises(ValueError):
        _fwd(ref, cfg, L, x, np.array([[0, 4]], np.int32), np.ones((1, 2), np.float32))
