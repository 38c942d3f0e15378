"""Pins for the oracle's GEMV, router and MoE composition.

Checks against brute force over subsets, library routines (scipy's softmax and
expit), the equivalence stated by the lynn-engine tutorials index (note 06: softmax
over all experts -> top-k -> renormalise equals softmax over the top-k logits),
special cases with closed forms, and reductions of the layer to a dense SwiGLU.
"""

import itertools

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
from oracle import formats as F
from oracle import ops
from bit_block_scaled_router_amd import synth


def _quant(fmt, w):
    return oracle.quantize(fmt, w)


# ---------------------------------------------------------------- GEMV


@pytest.mark.parametrize("fmt", [F.FMT_E2M1, F.FMT_INT4])
def test_gemv_one_hot_picks_dequantised_column(fmt):
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((24, 256)) * 0.02).astype(np.float32)
    codes, scales = _quant(fmt, w)
    deq = oracle.dequant(fmt, codes, scales)
    for j in (0, 17, 255):
        x = np.zeros(256, dtype=np.uint16)
        x[j] = 0x3F80  # 1.0
        assert np.array_equal(oracle.gemv(fmt, codes, scales, x), deq[:, j].astype(np.float64))


def test_gemv_equals_explicit_loop_on_tiny_input():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((5, 32)) * 0.3).astype(np.float32)
    codes, scales = _quant(F.FMT_E2M1, w)
    x = synth.f32_to_bf16_bits(rng.standard_normal(32).astype(np.float32))
    xv = oracle.bf16_bits_to_f64(x)
    nib = oracle.unpack_nibbles(codes)
    s = scales.view(np.float16).astype(np.float64)
    want = []
    for n in range(5):
        acc = 0.0
        for k in range(32):
            acc += float(oracle.e2m1_value(nib[n, k])) * s[n, k // 16] * xv[k]
        want.append(acc)
    np.testing.assert_allclose(oracle.gemv(F.FMT_E2M1, codes, scales, x), want, rtol=1e-14, atol=1e-16)


# ---------------------------------------------------------------- router


def test_router_softmax_matches_scipy():
    z = np.random.default_rng(3).standard_normal(256)
    np.testing.assert_allclose(ops.router_probs(z), softmax(z), rtol=1e-14)


@pytest.mark.parametrize("e,k", [(4, 1), (6, 2), (8, 2), (10, 3), (12, 4), (12, 12)])
def test_topk_is_best_subset_brute_force(e, k):
    rng = np.random.default_rng(100 + e * 13 + k)
    for _ in range(20):
        z = rng.standard_normal(e)
        ids, w = ops.route(z, k)
        p = softmax(z)
        best = max(itertools.combinations(range(e), k), key=lambda c: sum(p[list(c)]))
        assert sorted(ids.tolist()) == sorted(best)
        assert np.all(np.diff(p[ids]) <= 0)  # sorted by descending probability
        np.testing.assert_allclose(w, p[ids] / p[ids].sum(), rtol=1e-15)
        np.testing.assert_allclose(w.sum(), 1.0, rtol=1e-15)


def test_softmax_all_then_topk_equals_topk_then_softmax():
    rng = np.random.default_rng(4)
    for _ in range(200):
        e = int(rng.integers(2, 300))
        k = int(rng.integers(1, min(e, 16) + 1))
        z = rng.standard_normal(e) * rng.uniform(0.1, 5)
        ids_a, w_a = ops.route(z, k)
        ids_b, w_b = ops.route_topk_softmax(z, k)
        assert np.array_equal(ids_a, ids_b)
        np.testing.assert_allclose(w_a, w_b, rtol=1e-13, atol=0)


def test_router_special_cases():
    z = np.array([0.3, -1.0, 2.5, 2.5, 0.0, 1.0])
    ids, w = ops.route(z, 1)
    assert ids.tolist() == [2] and w.tolist() == [1.0]  # tie -> lower index, weight exactly 1
    ids, w = ops.route(z, 2)
    assert ids.tolist() == [2, 3] and w.tolist() == [0.5, 0.5]
    ids, w = ops.route(z, 6)  # k = E: the full softmax, in descending order
    np.testing.assert_allclose(w, softmax(z)[ids], rtol=1e-15)
    assert ids.tolist() == [2, 3, 5, 0, 4, 1]


def test_router_bias_is_added_before_softmax():
    rng = np.random.default_rng(8)
    wr = synth.f32_to_bf16_bits((rng.standard_normal((16, 64)) * 0.02).astype(np.float32))
    x = synth.f32_to_bf16_bits(rng.standard_normal(64).astype(np.float32))
    bias = np.zeros(16, dtype=np.float32)
    bias[9] = 50.0  # forces expert 9 first
    logits = ops.router_logits(wr, x, bias)
    ids, w = ops.route(logits, 3)
    assert ids[0] == 9 and w[0] > 0.999


def test_shared_gate_special_case_and_expit():
    x = synth.f32_to_bf16_bits(np.random.default_rng(9).standard_normal(128).astype(np.float32))
    assert ops.shared_gate(np.zeros(128, dtype=np.uint16), x) == 0.5
    wsg = synth.f32_to_bf16_bits((np.random.default_rng(10).standard_normal(128) * 0.02).astype(np.float32))
    t = oracle.bf16_bits_to_f64(wsg) @ oracle.bf16_bits_to_f64(x)
    np.testing.assert_allclose(ops.shared_gate(wsg, x), expit(t), rtol=1e-15)


def test_silu_matches_expit():
    g = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(ops.silu(g), g * expit(g), rtol=1e-14, atol=1e-300)


# ---------------------------------------------------------------- layer composition


def _small_layer(fmt, hidden, inter, e, k, shared, seed, bias=None):
    shape = synth.MoEShape("t", hidden, inter, e, k, inter if shared else 0, 1, 0.0, seed)
    c13, s13, c2, s2 = [], [], [], []
    for i in range(e):
        a, b = _quant(fmt, synth.expert_w13(shape, i))
        c13.append(a), s13.append(b)
        a, b = _quant(fmt, synth.expert_w2(shape, i))
        c2.append(a), s2.append(b)
    kw = {}
    if shared:
        kw = dict(shared_w13=_quant(fmt, synth.shared_w13(shape)),
                  shared_w2=_quant(fmt, synth.shared_w2(shape)),
                  shared_gate_w=synth.shared_gate_weight(shape))
    layer = ops.MoELayer(fmt, hidden, inter, e, k, synth.router_weight(shape),
                         (np.array(c13), np.array(s13)), (np.array(c2), np.array(s2)),
                         router_bias=bias, **kw)
    return shape, layer


def _dense_swiglu_via_gemv(fmt, w13, w2, x_bits, inter):
    """SwiGLU built from oracle.gemv calls on the two quantised matrices."""
    (c13, s13), (c2, s2) = w13, w2
    g = oracle.gemv(fmt, c13[:inter], s13[:inter], x_bits)
    u = oracle.gemv(fmt, c13[inter:], s13[inter:], x_bits)
    h = g * expit(g) * u
    w2d = oracle.dequant(fmt, c2, s2).astype(np.float64)
    return w2d @ h


@pytest.mark.parametrize("fmt", [F.FMT_E2M1, F.FMT_INT4])
def test_single_expert_layer_is_dense_swiglu(fmt):
    hidden, inter = 128, 128
    shape, layer = _small_layer(fmt, hidden, inter, 1, 1, False, 3)
    x = synth.x_row(0, hidden, 0)
    out, ids, w = ops.moe_forward(layer, x)
    assert ids.tolist() == [[0]] and w.tolist() == [[1.0]]
    c13, s13 = layer._w13
    c2, s2 = layer._w2
    want = _dense_swiglu_via_gemv(fmt, (c13[0], s13[0]), (c2[0], s2[0]), x, inter)
    np.testing.assert_allclose(out[0], want, rtol=1e-12, atol=1e-15)


def test_shared_expert_adds_sigmoid_gated_dense_swiglu():
    hidden, inter = 128, 128
    shape, layer = _small_layer(F.FMT_E2M1, hidden, inter, 1, 1, True, 4)
    x = synth.x_row(0, hidden, 1)
    out, _, _ = ops.moe_forward(layer, x)
    c13, s13 = layer._w13
    c2, s2 = layer._w2
    routed = _dense_swiglu_via_gemv(F.FMT_E2M1, (c13[0], s13[0]), (c2[0], s2[0]), x, inter)
    shared = _dense_swiglu_via_gemv(F.FMT_E2M1, layer.shared_w13, layer.shared_w2, x, inter)
    sig = expit(oracle.bf16_bits_to_f64(layer.shared_gate_w) @ oracle.bf16_bits_to_f64(x))
    np.testing.assert_allclose(out[0], routed + sig * shared, rtol=1e-12, atol=1e-15)


def test_bf16_shared_expert_is_exact_bf16_swiglu():
    """A bf16 shared expert (the pages' production format for it, lynn-engine README
    P15/P37) adds sigma times the dense SwiGLU on the bf16-rounded weights."""
    hidden, inter = 128, 128
    shape, layer4 = _small_layer(F.FMT_E2M1, hidden, inter, 1, 1, True, 6)
    sw13, sw2 = synth.shared_w13(shape), synth.shared_w2(shape)
    layer = ops.MoELayer(F.FMT_E2M1, hidden, inter, 1, 1, layer4.router_w, layer4._w13, layer4._w2,
                         shared_w13=oracle.quantize(F.FMT_BF16, sw13), shared_w2=oracle.quantize(F.FMT_BF16, sw2),
                         shared_gate_w=layer4.shared_gate_w, shared_fmt=F.FMT_BF16)
    x = synth.x_row(0, hidden, 2)
    out, _, _ = ops.moe_forward(layer, x)
    c13, s13 = layer._w13
    c2, s2 = layer._w2
    routed = _dense_swiglu_via_gemv(F.FMT_E2M1, (c13[0], s13[0]), (c2[0], s2[0]), x, inter)
    # bf16 weights: fp32 -> bf16 round to nearest even, written out bit by bit
    def rne(a):
        u = a.astype(np.float32).view(np.uint32).astype(np.uint64)
        return (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    xf = oracle.bf16_bits_to_f64(x)
    gu = rne(sw13) @ xf
    h = gu[:inter] * expit(gu[:inter]) * gu[inter:]
    shared = rne(sw2) @ h
    sig = expit(oracle.bf16_bits_to_f64(layer.shared_gate_w) @ xf)
    np.testing.assert_allclose(out[0], routed + sig * shared, rtol=1e-12, atol=1e-15)
    # and it differs from the 4-bit shared expert by the quantisation error only
    out4, _, _ = ops.moe_forward(layer4, x)
    assert not np.allclose(out4, out, rtol=1e-6) and np.allclose(out4, out, rtol=0.2, atol=0.05)


def test_zero_input_gives_zero_output():
    _, layer = _small_layer(F.FMT_E2M1, 256, 128, 8, 2, True, 5)
    out, _, _ = ops.moe_forward(layer, np.zeros(256, dtype=np.uint16))
    assert np.all(out == 0)


def test_combine_is_order_free_and_linear_in_weights():
    _, layer = _small_layer(F.FMT_E2M1, 256, 128, 8, 3, False, 6)
    x = synth.x_row(0, 256, 2)
    ids = np.array([[5, 1, 6]])
    w = np.array([[0.5, 0.3, 0.2]])
    a = ops.moe_experts(layer, x, ids, w)
    b = ops.moe_experts(layer, x, ids[:, ::-1], w[:, ::-1])
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-16)
    parts = [ops.moe_experts(layer, x, ids[:, j:j + 1], np.ones((1, 1))) for j in range(3)]
    np.testing.assert_allclose(a, sum(w[0, j] * parts[j] for j in range(3)), rtol=1e-12, atol=1e-16)


def test_batch_is_a_loop_over_tokens():
    _, layer = _small_layer(F.FMT_E2M1, 256, 128, 8, 2, True, 7)
    xs = np.stack([synth.x_row(0, 256, t) for t in range(3)])
    out, ids, w = ops.moe_forward(layer, xs)
    for t in range(3):
        o1, i1, w1 = ops.moe_forward(layer, xs[t])
        assert np.array_equal(out[t], o1[0]) and np.array_equal(ids[t], i1[0])


def test_error_metrics_on_known_vectors():
    r = oracle.error_report([1.0, 2.0, -2.0], [1.0, 2.0, -1.0])
    assert r["max_abs"] == 1.0 and r["max_ref"] == 2.0
    assert r["rel_l1"] == pytest.approx(1.0 / 4.0)
    assert r["rel_l2"] == pytest.approx(1.0 / 6 ** 0.5)
