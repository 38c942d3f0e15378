"""GPU parity of the device weight layout (W4_LAYOUT_GFX950_V1: per row, the
codes then the block scales in one 16-byte-aligned record).

Dequantisation of every format from that layout is bit-exact against the
oracle (which reads the canonical arrays the records were packed from); the
dense GEMV and the MoE layer on every path (single-token, batched, large-batch,
MX) match the oracle within the parity bar, and give bit for bit the output of
the same weights in the canonical layout (the kernels do the same arithmetic,
only the addresses differ)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from oracle import ops
import bit_block_scaled_router_amd as w4
from bit_block_scaled_router_amd import synth, workloads as wl
from moe_cases import assert_bf16_close, oracle_layer, tie_free_tokens

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"
V1 = w4.W4_LAYOUT_GFX950_V1
CANON = w4.W4_LAYOUT_CANONICAL

FMTS = [
    (w4.W4_FMT_E2M1_F16S16, F.FMT_E2M1, np.uint16, 0x7800),
    (w4.W4_FMT_INT4_F16S128, F.FMT_INT4, np.uint16, 0x7800),
    (w4.W4_FMT_NVFP4_E4M3S16, F.FMT_NVFP4, np.uint8, 0x7F),
    (w4.W4_FMT_MXFP4_E8M0S32, F.FMT_MXFP4, np.uint8, 251),
]


@pytest.mark.parametrize("fmt,ofmt,sdt,smax", FMTS, ids=["e2m1", "int4", "nvfp4", "mxfp4"])
@pytest.mark.parametrize("n,k", [(8, 256), (37, 384), (5, 2176)])
def test_dequant_from_device_layout_bit_exact(fmt, ofmt, sdt, smax, n, k):
    if k % F.group_size(ofmt):
        pytest.skip("k not a multiple of the format's group")
    print(f"layout dequant fmt={fmt} n={n} k={k}", flush=True)
    rng = np.random.default_rng(n * 131 + k + fmt)
    codes = rng.integers(0, 256, size=(2, n, k // 2), dtype=np.uint8)
    codes[0].reshape(-1)[:256] = np.arange(256, dtype=np.uint8)
    scales = rng.integers(0, smax, size=(2, n, k // F.group_size(ofmt)), dtype=np.int64).astype(sdt)
    g = np.array([0.75, 3.0], dtype=np.float32) if fmt == w4.W4_FMT_NVFP4_E4M3S16 else None
    W = w4.QMatrix.upload(fmt, codes, scales, DEV, global_np=g, layout=V1)
    assert W.scales is None and W.codes.numel() == w4.w4_codes_bytes(fmt, 2, n, k, V1)
    got = w4.w4_dequant_device(W).cpu().numpy()
    want = np.stack([oracle.dequant(ofmt, codes[i], scales[i], *((g[i],) if g is not None else ()))
                     for i in range(2)])
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("shape", [synth.GEMV_E2M1, synth.GEMV_INT4, synth.GEMV_NVFP4], ids=lambda s: s.name)
def test_gemv_device_layout(shape):
    print(f"layout gemv {shape.name}", flush=True)
    a = wl.build_dense(shape, DEV)
    b = wl.build_dense(shape, DEV, layout=V1)
    x = wl.bf16_tensor(synth.dense_x(shape), DEV)
    ya, yb = wl.bf16_bits(w4.w4a16_gemv(a, x)), wl.bf16_bits(w4.w4a16_gemv(b, x))
    assert np.array_equal(ya, yb)
    ofmt = {"e2m1": F.FMT_E2M1, "int4": F.FMT_INT4, "nvfp4": F.FMT_NVFP4}[shape.fmt]
    q = oracle.quantize(ofmt, synth.dense_weight(shape))
    ref = oracle.gemv(ofmt, q[0], q[1], synth.dense_x(shape), *q[2:])
    assert_bf16_close(yb, ref, shape.name)
    # one-hot columns: the dequantised column, rounded once, bit for bit
    for j in (0, 777, shape.k - 1):
        e = np.zeros(shape.k, dtype=np.uint16)
        e[j] = 0x3F80
        col = wl.bf16_bits(w4.w4a16_gemv(b, wl.bf16_tensor(e, DEV)))
        want = oracle.f64_to_bf16_bits(oracle.dequant(ofmt, *q)[:, j])
        assert np.array_equal(col, want), j


def _run(layer, xb, T, K):
    ids = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    wts = torch.zeros((T, K), dtype=torch.float32, device=DEV)
    y = w4.moe_w4a16_forward(layer, wl.bf16_tensor(xb, DEV), topk_ids=ids, topk_w=wts)
    torch.cuda.synchronize()
    return wl.bf16_bits(y), ids.cpu().numpy(), wts.cpu().numpy()


MOE = [
    (synth.TINY_MOE, (1, 3, 40)),                 # single-token and batched paths
    (synth.TINY_MOE_BF16SH, (2, 300)),            # bf16 shared expert (both layouts coincide for it)
    (synth.QWEN_MOE_T1, (1,)),                    # the decode layer
    (synth.QWEN_MOE_T32, (32,)),                  # batched, Zipf-biased routing
    (synth.QWEN_MOE_T32_INT4, (32,)),
    (synth.QWEN_MOE_T32_NVFP4, (32,)),
    (synth.QWEN_MOE_T32_MX, (3, 32)),
    (synth.MoEShape("layout-prefill", 256, 128, 16, 4, 128, 1, 0.0, 31), (1200,)),  # large-batch kernels
]


@pytest.mark.parametrize("shape,Ts", MOE, ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_moe_device_layout(shape, Ts):
    a = wl.build_moe_layer(shape, device=DEV)
    b = wl.build_moe_layer(shape, device=DEV, layout=V1)
    or_layer = oracle_layer(shape)
    for T in Ts:
        print(f"layout moe {shape.name} T={T} stages={w4.moe_w4a16_stage_count(b, T)}", flush=True)
        xb = tie_free_tokens(shape, or_layer, T, first=13 * T)
        ya, ia, wa = _run(a, xb, T, shape.top_k)
        yb, ib, wb = _run(b, xb, T, shape.top_k)
        assert np.array_equal(ia, ib) and np.array_equal(wa.view(np.uint32), wb.view(np.uint32))
        assert np.array_equal(ya, yb), f"{shape.name} T={T}: layouts differ"
        if shape.fmt == "mxfp4":
            continue  # the MX path's own bounds are checked in test_gpu_mx on the canonical layout
        rows = np.arange(T) if T <= 40 else np.unique(np.linspace(0, T - 1, 12).astype(int))
        ref, rids, rw = ops.moe_forward(or_layer, xb, tokens=list(rows))
        assert np.array_equal(ib[rows], rids)
        np.testing.assert_allclose(wb[rows], rw, rtol=2e-6, atol=1e-7)
        assert_bf16_close(yb[rows], ref, f"{shape.name} T={T}")
