"""GPU parity of the decode kernels (down projections stored K-tiled,
W4_LAYOUT_GFX950_KT16): one launch computes, per (token, slot, 16 intermediate
values), the gate/up rows, SiLU * up and that K tile's contribution to every
output row; a second adds the contributions in a fixed order.

Against the oracle: bit-exact top-k ids, routing weights within 2e-6, bf16
outputs within the parity bar, on the tiny and 35B-A3B shapes, E2M1 and NVFP4,
single tokens and batches, caller routing (an invalid id poisons its token
only), the router's extremes (k = 1, k = E), hidden sizes off the 2048 grid
(fewer lanes per row, two K steps), W13 in either row layout; repeated calls
are bitwise equal."""

import numpy as np
import pytest
import torch

import oracle
from oracle import ops
import bit_block_scaled_router_amd as w4
from bit_block_scaled_router_amd import synth, workloads as wl
from moe_cases import assert_bf16_close, oracle_layer, tie_free_tokens

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"
V1 = w4.W4_LAYOUT_GFX950_V1
KT = w4.W4_LAYOUT_GFX950_KT16


def _layer(shape, w13_layout=V1):
    return wl.build_moe_layer(shape, device=DEV, layout=w13_layout, w2_layout=KT)


def _run(layer, xb, K):
    T = xb.shape[0]
    ids = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    wts = torch.zeros((T, K), dtype=torch.float32, device=DEV)
    y = w4.moe_w4a16_forward(layer, wl.bf16_tensor(xb, DEV), topk_ids=ids, topk_w=wts)
    torch.cuda.synchronize()
    return wl.bf16_bits(y), ids.cpu().numpy(), wts.cpu().numpy()


def _check(shape, layer, or_layer, T, first, what, rows=None):
    xb = tie_free_tokens(shape, or_layer, T, first=first)
    assert w4.moe_w4a16_stage_count(layer, T) == 3
    got, ids, wts = _run(layer, xb, shape.top_k)
    rows = np.arange(T) if rows is None else rows
    ref, rids, rw = ops.moe_forward(or_layer, xb, tokens=list(rows))
    assert np.array_equal(ids[rows], rids), what
    np.testing.assert_allclose(wts[rows], rw, rtol=2e-6, atol=1e-7)
    assert_bf16_close(got[rows], ref, what)
    return xb, got


CASES = [
    (synth.TINY_MOE, V1, (1, 3, 6)),
    (synth.MoEShape("dec-tiny-shared", 256, 128, 8, 2, 128, 1, 0.0, 41), V1, (1, 2, 40)),
    (synth.MoEShape("dec-tiny-shared-nvfp4", 256, 128, 8, 2, 128, 1, 0.0, 42, "nvfp4"), V1, (1, 5)),
    (synth.MoEShape("dec-tiny-canon-w13", 256, 128, 8, 2, 128, 1, 0.0, 43), w4.W4_LAYOUT_CANONICAL, (1, 3)),
    (synth.MoEShape("dec-h320-i96", 320, 96, 16, 4, 96, 1, 0.0, 44), V1, (1, 4)),     # 16 lanes per row
    (synth.MoEShape("dec-h4096", 4096, 128, 8, 2, 128, 1, 0.0, 45), V1, (1, 2)),      # two K steps
    (synth.MoEShape("dec-k1", 256, 128, 8, 1, 128, 1, 0.0, 46), V1, (1, 5)),
    (synth.MoEShape("dec-kE", 256, 128, 8, 8, 128, 1, 0.0, 47), V1, (1, 5)),
    (synth.MoEShape("dec-e1024-k16", 256, 128, 1024, 16, 128, 1, 0.0, 48), V1, (1, 3)),
]


@pytest.mark.parametrize("shape,w13_layout,Ts", CASES, ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_decode_kernels_small_shapes(shape, w13_layout, Ts):
    layer = _layer(shape, w13_layout)
    or_layer = oracle_layer(shape)
    for T in Ts:
        print(f"decode {shape.name} T={T}", flush=True)
        _check(shape, layer, or_layer, T, 17 * T, f"{shape.name} T={T}")


@pytest.fixture(scope="module")
def qwen_dec():
    shape = synth.QWEN_MOE_T1
    print("building the 35B-A3B-shaped layer with K-tiled down projections", flush=True)
    return shape, _layer(shape), oracle_layer(shape)


def test_decode_qwen_single_tokens(qwen_dec):
    shape, layer, or_layer = qwen_dec
    for t in range(3):
        print(f"decode qwen token {t}", flush=True)
        xb, got = _check(shape, layer, or_layer, 1, t, f"qwen t={t}")
        got2, _, _ = _run(layer, xb, shape.top_k)
        assert np.array_equal(got, got2)  # deterministic


def test_decode_qwen_batch(qwen_dec):
    shape, layer, or_layer = qwen_dec
    print("decode qwen T=8", flush=True)
    _check(shape, layer, or_layer, 8, 100, "qwen T=8", rows=np.array([0, 3, 7]))


def test_decode_qwen_nvfp4():
    shape = synth.QWEN_MOE_T1_NVFP4
    layer, or_layer = _layer(shape), oracle_layer(shape)
    print("decode qwen nvfp4", flush=True)
    _check(shape, layer, or_layer, 2, 5, "qwen nvfp4 T=2")


def test_decode_caller_routing_and_invalid_id():
    shape = synth.MoEShape("dec-experts", 256, 128, 8, 2, 128, 1, 0.0, 49)
    layer, or_layer = _layer(shape), oracle_layer(shape)
    xb = tie_free_tokens(shape, or_layer, 3, first=7)
    ids = np.array([[1, 6], [3, 3], [0, 7]], dtype=np.int32)
    w = np.array([[0.7, 0.3], [1.0, 0.25], [0.125, -0.5]], dtype=np.float32)
    y = w4.moe_w4a16_experts(layer, wl.bf16_tensor(xb, DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV))
    ref = ops.moe_experts(or_layer, xb, ids, w)
    assert_bf16_close(wl.bf16_bits(y), ref, "decode experts")
    bad = ids.copy()
    bad[1, 0] = 8
    y = w4.moe_w4a16_experts(layer, wl.bf16_tensor(xb, DEV), torch.from_numpy(bad).to(DEV), torch.from_numpy(w).to(DEV))
    yb = oracle.bf16_bits_to_f64(wl.bf16_bits(y))
    assert np.all(np.isnan(yb[1])) and np.all(np.isfinite(yb[[0, 2]]))


def test_k_tiled_matrices_only_serve_the_down_projection():
    shape = synth.TINY_MOE
    layer = _layer(shape)
    with pytest.raises(w4.W4Error) as e:
        w4.w4_dequant_device(layer.w2)
    assert e.value.status == w4.W4_ERR_UNSUPPORTED
    x = torch.zeros(shape.inter, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(w4.W4Error):
        w4.w4a16_gemv(w4.QMatrix(layer.w2.fmt, 1, shape.hidden, shape.inter, layer.w2.codes, None, layout=KT), x)
