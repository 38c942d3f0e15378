"""GPU parity of the NVFP4 variant (E2M1 codes, UE4M3 per-16 scales, fp32 global
scale per matrix) through the C ABI against the CPU oracle: bit-exact dequant
(every UE4M3 scale byte), bit-exact one-hot GEMV, GEMVs and MoE layers within the
parity tolerance."""

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from oracle import ops
import bit_block_scaled_router_amd as w4
from bit_block_scaled_router_amd import synth, workloads as wl
from moe_cases import assert_bf16_close, oracle_layer, tie_free_tokens

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"
NV = w4.W4_FMT_NVFP4_E4M3S16


def _upload(codes, scales, gsc):
    return w4.QMatrix.upload(NV, codes, scales, DEV, global_np=gsc)


@pytest.mark.parametrize("n,k", [(8, 256), (37, 384), (5, 2176), (3, 4096)])
def test_nvfp4_dequant_bit_exact(n, k):
    print(f"nvfp4 dequant n={n} k={k}", flush=True)
    rng = np.random.default_rng(n * 31 + k)
    codes = rng.integers(0, 256, size=(3, n, k // 2), dtype=np.uint8)
    codes[0].reshape(-1)[:256] = np.arange(256, dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(3, n, k // 16), dtype=np.uint8)  # finite UE4M3 bytes
    m = min(scales[0].size, 0x7F)
    scales[0].reshape(-1)[:m] = np.arange(m, dtype=np.uint8)  # every scale byte
    gsc = np.array([1.0, 3.0517578e-05, 7.123456], dtype=np.float32)
    got = w4.w4_dequant_device(_upload(codes, scales, gsc)).cpu().numpy()
    want = np.stack([oracle.dequant(F.FMT_NVFP4, codes[g], scales[g], gsc[g]) for g in range(3)])
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_ue4m3_all_bytes_hardware_witness():
    """Every finite UE4M3 byte through the device decode (code 1.0, global 1.0)
    equals the typed OCP E4M3 values."""
    scales = np.arange(0x80, dtype=np.uint8).reshape(1, 1, 128)
    scales[0, 0, 0x7F] = 0  # NaN byte left out
    codes = np.full((1, 1, 1024), 0x22, dtype=np.uint8)  # both nibbles code 2 = 1.0
    got = w4.w4_dequant_device(_upload(codes, scales, np.ones(1, np.float32))).cpu().numpy().reshape(128, 16)
    want = F.e4m3_value(scales[0, 0]).astype(np.float32)
    assert np.array_equal(got[:, 0], want) and np.all(got == got[:, :1])


def test_nvfp4_gemv_one_hot_bit_exact():
    w = (np.random.default_rng(4).standard_normal((300, 2048)) * 0.02).astype(np.float32)
    codes, scales, g = oracle.quantize(F.FMT_NVFP4, w)
    W = _upload(codes, scales, np.array([g], np.float32))
    deq = oracle.dequant(F.FMT_NVFP4, codes, scales, g)
    for j in (0, 31, 32, 1000, 2047):
        x = np.zeros(2048, dtype=np.uint16)
        x[j] = 0x3F80
        got = wl.bf16_bits(w4.w4a16_gemv(W, wl.bf16_tensor(x)))
        assert np.array_equal(got, oracle.f64_to_bf16_bits(deq[:, j].astype(np.float64))), j


@pytest.mark.parametrize("n,k,m", [(1, 128, 1), (37, 384, 1), (130, 2048, 1), (129, 4096, 1), (33, 1024, 3),
                                   (17, 256, 64)])
def test_nvfp4_gemv_random(n, k, m):
    print(f"nvfp4 gemv n={n} k={k} m={m}", flush=True)
    rng = np.random.default_rng(n + 17 * k + m)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    codes, scales, g = w4.w4_quantize(NV, w)
    x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    y = w4.w4a16_gemv(_upload(codes, scales, np.array([g], np.float32)), wl.bf16_tensor(x))
    packed, sb, go = oracle.quantize(F.FMT_NVFP4, w)
    assert_bf16_close(wl.bf16_bits(y), oracle.gemv(F.FMT_NVFP4, packed, sb, x, go), f"nvfp4 gemv {n}x{k} m={m}")


def test_nvfp4_gemv_full_size():
    shape = synth.GEMV_NVFP4
    print(f"gemv full {shape.name}", flush=True)
    W = wl.build_dense(shape, DEV)
    x = synth.dense_x(shape)
    y = w4.w4a16_gemv(W, wl.bf16_tensor(x))
    packed, sb, g = oracle.quantize(F.FMT_NVFP4, synth.dense_weight(shape))
    assert_bf16_close(wl.bf16_bits(y), oracle.gemv(F.FMT_NVFP4, packed, sb, x, g), shape.name)


def _check_moe(shape, dev_layer, or_layer, x_bits, what):
    T = x_bits.shape[0]
    ids = torch.full((T, shape.top_k), -7, dtype=torch.int32, device=DEV)
    wts = torch.zeros((T, shape.top_k), dtype=torch.float32, device=DEV)
    y = w4.moe_w4a16_forward(dev_layer, wl.bf16_tensor(x_bits), topk_ids=ids, topk_w=wts)
    ref, rids, rw = ops.moe_forward(or_layer, x_bits)
    assert np.array_equal(ids.cpu().numpy(), rids), what
    np.testing.assert_allclose(wts.cpu().numpy(), rw, rtol=2e-6, atol=1e-7)
    return assert_bf16_close(wl.bf16_bits(y), ref, what)


@pytest.fixture(scope="module")
def tiny_nv():
    shape = synth.TINY_MOE
    return shape, wl.build_moe_layer(shape, fmt=NV, device=DEV), oracle_layer(shape, F.FMT_NVFP4)


def test_nvfp4_moe_tiny(tiny_nv):
    shape, dev_layer, or_layer = tiny_nv
    for t in range(3):
        print(f"nvfp4 moe tiny token {t}", flush=True)
        _check_moe(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, 1, first=t), f"nvfp4 tiny t={t}")
    # batches of 4 or more take the grouped path (MFMA for groups of >= 2 rows)
    assert w4.moe_w4a16_stage_count(dev_layer, 3) == 3
    assert w4.moe_w4a16_stage_count(dev_layer, 7) == 5
    _check_moe(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, 3, first=30), "nvfp4 tiny T=3")
    for T in (7, 40, 300):
        print(f"nvfp4 moe tiny T={T}", flush=True)
        _check_moe(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, T, first=10), f"nvfp4 tiny T={T}")


def test_nvfp4_moe_tiny_batched_experts_entry(tiny_nv):
    """Caller routing on the grouped path: one group of >= 16 rows (MFMA), small
    groups (VALU), an invalid id that turns its token into NaN."""
    shape, dev_layer, or_layer = tiny_nv
    T = 24
    xb = tie_free_tokens(shape, or_layer, T, first=300)
    rng = np.random.default_rng(6)
    ids = np.stack([rng.choice(shape.num_experts, shape.top_k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[:20, 0] = 3
    ids[:20, 1] = np.where(ids[:20, 1] == 3, 4, ids[:20, 1])
    w = rng.uniform(0.1, 1.0, size=(T, shape.top_k)).astype(np.float32)
    y = w4.moe_w4a16_experts(dev_layer, wl.bf16_tensor(xb), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV))
    assert_bf16_close(wl.bf16_bits(y), ops.moe_experts(or_layer, xb, ids, w.astype(np.float64)), "nvfp4 batched entry")
    bad = ids.copy()
    bad[7, 1] = -1
    y2 = w4.moe_w4a16_experts(dev_layer, wl.bf16_tensor(xb), torch.from_numpy(bad).to(DEV),
                              torch.from_numpy(w).to(DEV))
    g = oracle.bf16_bits_to_f64(wl.bf16_bits(y2))
    assert np.all(np.isnan(g[7])) and np.all(np.isfinite(np.delete(g, 7, axis=0)))


def test_nvfp4_moe_batch32_zipf():
    """The 35B-A3B-shaped NVFP4 layer, 32 tokens with the Zipf(1.1) routing bias:
    the grouped path, every token checked."""
    shape = synth.QWEN_MOE_T32_NVFP4
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    assert w4.moe_w4a16_stage_count(dev_layer, 32) == 5
    or_layer = oracle_layer(shape)
    print("nvfp4 batch 32", flush=True)
    print(_check_moe(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, 32, first=50), shape.name), flush=True)


def test_nvfp4_moe_tiny_experts_entry(tiny_nv):
    shape, dev_layer, or_layer = tiny_nv
    xb = tie_free_tokens(shape, or_layer, 3, first=20)
    ids = np.array([[1, 6], [6, 1], [3, 3]], dtype=np.int32)
    w = np.array([[0.7, 0.3], [0.5, 0.5], [1.0, 0.25]], dtype=np.float32)
    y = w4.moe_w4a16_experts(dev_layer, wl.bf16_tensor(xb), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV))
    assert_bf16_close(wl.bf16_bits(y), ops.moe_experts(or_layer, xb, ids, w.astype(np.float64)), "nvfp4 experts")


def test_nvfp4_moe_full_t1():
    shape = synth.QWEN_MOE_T1
    print("building the 35B-A3B-shaped NVFP4 layer", flush=True)
    dev_layer = wl.build_moe_layer(shape, fmt=NV, device=DEV)
    or_layer = oracle_layer(shape, F.FMT_NVFP4)
    for t in range(2):
        print(f"nvfp4 moe full token {t}", flush=True)
        print(_check_moe(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, 1, first=t), f"nvfp4 full t={t}"),
              flush=True)
