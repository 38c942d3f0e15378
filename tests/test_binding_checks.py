"""The Python binding rejects tensors whose dtype, shape, contiguity or device do
not match what the C ABI assumes, before anything reaches the library (the C
functions take raw pointers and cannot see buffer sizes).  Host only: every
call below raises ValueError before the library is loaded or called."""

import numpy as np
import pytest
import torch

import bit_block_scaled_router_amd as w4

H, I, E, K, T = 256, 128, 8, 2, 3


def _layer():
    def q(groups, n, k):
        return w4.QMatrix(w4.W4_FMT_E2M1_F16S16, groups, n, k, torch.zeros((groups, n, k // 2), dtype=torch.uint8),
                          torch.zeros((groups, n, k // 16), dtype=torch.int16))
    return w4.MoELayer(H, I, E, K, torch.zeros((E, H), dtype=torch.int16), q(E, 2 * I, H), q(E, H, I))


def _bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


@pytest.mark.parametrize("case", [
    "x_1d", "x_dtype", "x_width", "x_noncontig", "x_host", "y_small", "y_dtype", "ids_dtype", "ids_shape",
    "w_dtype", "w_shape", "ws_dtype",
])
def test_forward_rejects(case):
    layer = _layer()
    x, y = _bf16(T, H), _bf16(T, H)
    kw = {}
    if case == "x_1d":
        x = _bf16(H)
    elif case == "x_dtype":
        x = torch.zeros((T, H), dtype=torch.float16)
    elif case == "x_width":
        x = _bf16(T, H + 64)
    elif case == "x_noncontig":
        x = _bf16(H, T).t()
    elif case == "y_small":
        y = _bf16(T - 1, H)
    elif case == "y_dtype":
        y = torch.zeros((T, H), dtype=torch.float32)
    elif case == "ids_dtype":
        kw["topk_ids"] = torch.zeros((T, K), dtype=torch.int64)
    elif case == "ids_shape":
        kw["topk_ids"] = torch.zeros((T, K + 1), dtype=torch.int32)
    elif case == "w_dtype":
        kw["topk_w"] = torch.zeros((T, K), dtype=torch.float64)
    elif case == "w_shape":
        kw["topk_w"] = torch.zeros((T + 1, K), dtype=torch.float32)
    elif case == "ws_dtype":
        kw["ws"] = torch.zeros(1024, dtype=torch.float32)
    # every case: host tensors or a wrong dtype/shape, so the binding must refuse
    with pytest.raises(ValueError):
        w4.moe_w4a16_forward(layer, x, y=y, **kw)


@pytest.mark.parametrize("case", ["ids_dtype", "ids_shape", "w_shape", "host"])
def test_experts_rejects(case):
    layer = _layer()
    x, y = _bf16(T, H), _bf16(T, H)
    ids, wts = torch.zeros((T, K), dtype=torch.int32), torch.zeros((T, K), dtype=torch.float32)
    if case == "ids_dtype":
        ids = ids.to(torch.int16)
    elif case == "ids_shape":
        ids = torch.zeros((T, K - 1), dtype=torch.int32)
    elif case == "w_shape":
        wts = torch.zeros((T * K,), dtype=torch.float32)
    with pytest.raises(ValueError):
        w4.moe_w4a16_experts(layer, x, ids, wts, y=y)


def test_shape_checks_come_before_the_device_check():
    layer = _layer()
    with pytest.raises(ValueError, match="shape"):
        w4.moe_w4a16_forward(layer, _bf16(T, H), y=_bf16(T, H - 64))
    with pytest.raises(ValueError, match="device"):
        w4.moe_w4a16_forward(layer, _bf16(T, H), y=_bf16(T, H))


@pytest.mark.parametrize("case", ["x_len", "x_dtype", "y_shape", "y_rank", "host"])
def test_gemv_rejects(case):
    n, k = 64, 256
    W = w4.QMatrix(w4.W4_FMT_E2M1_F16S16, 1, n, k, torch.zeros((1, n, k // 2), dtype=torch.uint8),
                   torch.zeros((1, n, k // 16), dtype=torch.int16))
    x, y = _bf16(k), _bf16(n)
    if case == "x_len":
        x = _bf16(k - 32)
    elif case == "x_dtype":
        x = torch.zeros(k, dtype=torch.float32)
    elif case == "y_shape":
        y = _bf16(n - 1)
    elif case == "y_rank":
        y = _bf16(1, n)
    with pytest.raises(ValueError):
        w4.w4a16_gemv(W, x, y=y)


def test_dequant_rejects_small_output():
    W = w4.QMatrix(w4.W4_FMT_E2M1_F16S16, 2, 8, 64, torch.zeros((2, 8, 32), dtype=torch.uint8),
                   torch.zeros((2, 8, 4), dtype=torch.int16))
    with pytest.raises(ValueError):
        w4.w4_dequant_device(W, out=torch.zeros((1, 8, 64), dtype=torch.float32))
    assert np.all(W.codes.numpy() == 0)
