"""Pins of the oracle's router: logits against exact integer products and a
float64 library product, top-k against brute force, gate weights against closed
forms and invariants."""

import itertools
import math

import numpy as np
import pytest

import moegen
from tests import np_ref


def brute_topk(l, k):
    """The unique k-subset S such that every member beats every non-member
    (greater logit, or equal logit and lower index), listed in descending
    logit order with ties to the lower index."""
    E = len(l)
    found = []
    for S in itertools.combinations(range(E), k):
        rest = [u for u in range(E) if u not in S]
        if all(l[s] > l[u] or (l[s] == l[u] and s < u) for s in S for u in rest):
            found.append(S)
    assert len(found) == 1
    return sorted(found[0], key=lambda e: (-l[e], e))


@pytest.mark.parametrize("seed", range(40))
def test_topk_brute_force_with_ties(ref, seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 11))
    k = int(rng.integers(1, min(E, 3) + 1))
    T = 6
    logits = rng.integers(-3, 4, size=(T, E)).astype(np.float32)   # many exact ties
    logits[0] = 1.0                                                 # a fully tied row
    x = np.zeros((T, 32), np.float32)
    wr = np.zeros((E, 32), np.float32)
    got_l, ids, w = ref.route(x, wr, None, k=k, act_dtype="f32", router_dtype="f32",
                              score="softmax", logits_in=logits)
    assert np.array_equal(got_l, logits)
    for t in range(T):
        assert list(ids[t]) == brute_topk(list(logits[t]), k)


def test_logits_exact_integer_products(ref):
    """Small integers: every product and partial sum is exact, so the logits
    equal the integer matrix product plus the bias exactly."""
    rng = np.random.default_rng(1)
    T, H, E = 5, 64, 7
    x = rng.integers(-4, 5, (T, H)).astype(np.float32)
    wr = rng.integers(-4, 5, (E, H)).astype(np.float32)
    bias = np.array([0.5 * e - 1 for e in range(E)], np.float32)
    l, _, _ = ref.route(x, wr, bias, k=2, act_dtype="f32", router_dtype="f32",
                        score="softmax")
    want = x.astype(np.int64) @ wr.astype(np.int64).T + bias[None, :]
    assert np.array_equal(l, want.astype(np.float32))


def test_logits_one_hot_picks_router_column(ref):
    """x = 3*e_h: logit e is 3*W_r[e][h] (bf16 activations and router)."""
    cfg = moegen.QWEN3_DECODE
    L = moegen.make_layer(cfg.with_(n_experts=16, ffn=256, hidden=256))
    wr = moegen.as_numpy_bits(L.router)
    x = np.zeros((1, 256), np.uint16)
    x[0, 77] = 0x4040                                 # bf16 3.0
    l, _, _ = ref.route(x, wr, None, k=4, act_dtype="bf16", router_dtype="bf16",
                        score="softmax")
    assert np.array_equal(l[0].astype(np.float64), 3.0 * np_ref.act(wr)[:, 77])


@pytest.mark.parametrize("cfg", [moegen.TINY, moegen.QWEN3_PREFILL], ids=lambda c: c.name)
def test_logits_match_float64_product(ref, cfg):
    small = cfg.with_(hidden=min(cfg.hidden, 1024))
    L = moegen.make_layer(small.with_(ffn=256, n_experts=min(cfg.n_experts, 32)))
    x = moegen.as_numpy_bits(moegen.make_x(small, 9))
    wr = moegen.as_numpy_bits(L.router)
    bias = None if L.bias is None else L.bias.numpy()
    l, _, _ = ref.route(x, wr, bias, k=2, act_dtype=small.act_dtype,
                        router_dtype=small.router_dtype, score="softmax")
    want = np_ref.act(x) @ np_ref.act(wr).T
    if bias is not None:
        want += bias[None, :]
    np.testing.assert_allclose(l, want, rtol=0, atol=2e-6 * np.abs(want).max())


def _routed(ref, logits, k, score):
    T, E = logits.shape
    x = np.zeros((T, 32), np.float32)
    wr = np.zeros((E, 32), np.float32)
    return ref.route(x, wr, None, k=k, act_dtype="f32", router_dtype="f32", score=score,
                     logits_in=logits)


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_softmax_renorm_is_softmax_over_selected(ref, k):
    """Renormalising a softmax over all experts to the selected ones equals a
    softmax over the selected logits alone; the weights sum to one."""
    rng = np.random.default_rng(k)
    logits = (rng.standard_normal((50, 16)) * 3).astype(np.float32)
    _, ids, w = _routed(ref, logits, k, "softmax")
    for t in range(50):
        sel = [float(logits[t, e]) for e in ids[t]]
        m = max(sel)
        z = sum(math.exp(v - m) for v in sel)
        want = [math.exp(v - m) / z for v in sel]
        np.testing.assert_allclose(w[t], want, rtol=2e-7, atol=0)
        assert abs(float(np.sum(w[t].astype(np.float64))) - 1.0) <= 1e-6
        assert np.all(np.diff(w[t]) <= 0)      # slot order = descending score


def test_softmax_k_equals_E_is_full_softmax(ref):
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((8, 10)).astype(np.float32)
    _, ids, w = _routed(ref, logits, 10, "softmax")
    for t in range(8):
        p = np.exp(logits[t].astype(np.float64) - logits[t].max())
        p /= p.sum()
        np.testing.assert_allclose(w[t], p[ids[t]], rtol=2e-7)
        assert sorted(ids[t]) == list(range(10))


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_k1_weight_is_one(ref, score):
    logits = np.random.default_rng(4).standard_normal((20, 12)).astype(np.float32)
    _, ids, w = _routed(ref, logits, 1, score)
    assert np.all(w == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(logits, axis=1))


def test_sigmoid_special_values(ref):
    # all logits 0: sigma = 1/2 everywhere, ties -> experts 0..k-1, w = 1/k
    _, ids, w = _routed(ref, np.zeros((1, 9), np.float32), 4, "sigmoid")
    assert list(ids[0]) == [0, 1, 2, 3]
    assert np.all(w == np.float32(0.25))
    # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4: weights 3/4 and 1/4
    l = np.array([[-50.0, math.log(3), -math.log(3), -60.0]], np.float32)
    _, ids, w = _routed(ref, l, 2, "sigmoid")
    assert list(ids[0]) == [1, 2]
    np.testing.assert_allclose(w[0], [0.75, 0.25], rtol=1e-6)


def test_sigmoid_weight_ratio(ref):
    """Sigmoid weights are proportional to sigma(l); unlike softmax, their ratio
    is not exp of the logit difference."""
    rng = np.random.default_rng(5)
    logits = (rng.standard_normal((30, 32)) * 4).astype(np.float32)
    _, ids, w = _routed(ref, logits, 8, "sigmoid")
    for t in range(30):
        l0, l1 = float(logits[t, ids[t, 0]]), float(logits[t, ids[t, 1]])
        ratio = (1 + math.exp(-l1)) / (1 + math.exp(-l0))
        assert abs(w[t, 0] / w[t, 1] - ratio) <= 1e-6 * ratio
        assert abs(float(np.sum(w[t].astype(np.float64))) - 1.0) <= 1e-6


def test_bias_shifts_selection(ref):
    """A per-expert bias is added before selection (and before scoring)."""
    x = np.zeros((1, 32), np.float32)
    wr = np.zeros((4, 32), np.float32)
    bias = np.array([0.0, 2.0, -1.0, 1.0], np.float32)
    l, ids, w = ref.route(x, wr, bias, k=2, act_dtype="f32", router_dtype="f32",
                          score="softmax")
    assert np.array_equal(l[0], bias)
    assert list(ids[0]) == [1, 3]
    np.testing.assert_allclose(w[0], [math.e / (math.e + 1), 1 / (math.e + 1)], rtol=1e-6)
