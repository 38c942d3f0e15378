"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bit-exact: dequantised weights, GEMV with one-hot activations, top-k expert ids.
Within tolerance (tests/moe_cases.py): every bf16 output.  Shapes span several
tiles and ragged tails, the full workload sizes and the degenerate cases.
"""

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
FMTS = [(w4.W4_FMT_E2M1_F16S16, F.FMT_E2M1), (w4.W4_FMT_INT4_F16S128, F.FMT_INT4)]


def _sync():
    torch.cuda.synchronize()


def _upload(fmt, codes, scales):
    return w4.QMatrix.upload(fmt, codes, scales, DEV)


# ---------------------------------------------------------------- decode tables on the device


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("n,k", [(8, 256), (37, 384), (5, 2176), (3, 4096)])
def test_dequant_bit_exact(fmt, ofmt, n, k):
    if k % F.group_size(ofmt):
        pytest.skip("k not a multiple of the int4 group")
    print(f"dequant fmt={fmt} n={n} k={k}", flush=True)
    rng = np.random.default_rng(n * 7919 + k)
    codes = rng.integers(0, 256, size=(2, n, k // 2), dtype=np.uint8)
    codes[0].reshape(-1)[:256] = np.arange(256, dtype=np.uint8)  # every byte value
    scales = rng.integers(0, 0x7800, size=(2, n, k // F.group_size(ofmt)), dtype=np.uint16)
    special = [0x7BFF, 0x0400, 0x0001]  # fp16 max, smallest normal, smallest subnormal
    scales[0].reshape(-1)[:3] = special
    W = _upload(fmt, codes, scales)
    got = w4.w4_dequant_device(W).cpu().numpy()
    _sync()
    want = np.stack([oracle.dequant(ofmt, codes[g], scales[g]) for g in range(2)])
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_e2m1_all_bytes_hardware_witness():
    """All 256 code bytes through the device decode equal the typed E2M1 table."""
    codes = np.arange(256, dtype=np.uint8).reshape(1, 8, 32)
    scales = np.full((1, 8, 4), 0x3C00, dtype=np.uint16)  # scale 1.0
    got = w4.w4_dequant_device(_upload(w4.W4_FMT_E2M1_F16S16, codes, scales)).cpu().numpy().ravel()
    table = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6], dtype=np.float32)
    b = np.arange(256)
    want = np.stack([table[b & 15], table[b >> 4]], axis=1).ravel()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------- dense GEMV


@pytest.mark.parametrize("fmt,ofmt", FMTS)
def test_gemv_one_hot_bit_exact(fmt, ofmt):
    w = (np.random.default_rng(3).standard_normal((300, 2048)) * 0.02).astype(np.float32)
    codes, scales = oracle.quantize(ofmt, w)
    W = _upload(fmt, codes, scales)
    deq = oracle.dequant(ofmt, codes, scales)
    for j in (0, 31, 32, 1000, 2047):
        x = np.zeros(2048, dtype=np.uint16)
        x[j] = 0x3F80
        y = w4.w4a16_gemv(W, wl.bf16_tensor(x))
        got = wl.bf16_bits(y)
        want = oracle.f64_to_bf16_bits(deq[:, j].astype(np.float64))
        assert np.array_equal(got, want), j


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("n,k,m", [(1, 128, 1), (37, 384, 1), (130, 2048, 1), (129, 4096, 1),
                                   (64, 2048 + 128, 1), (33, 1024, 3), (17, 256, 64)])
def test_gemv_random_within_tolerance(fmt, ofmt, n, k, m):
    if k % F.group_size(ofmt):
        pytest.skip("k not a multiple of the int4 group")
    print(f"gemv fmt={fmt} n={n} k={k} m={m}", flush=True)
    rng = np.random.default_rng(n + 13 * k + m)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    codes, scales = w4.w4_quantize(fmt, w)
    x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    y = w4.w4a16_gemv(_upload(fmt, codes, scales), wl.bf16_tensor(x))
    ref = oracle.gemv(ofmt, *oracle.quantize(ofmt, w), x)
    assert_bf16_close(wl.bf16_bits(y), ref, f"gemv {n}x{k} m={m}")


@pytest.mark.parametrize("shape", [synth.GEMV_E2M1, synth.GEMV_INT4], ids=lambda s: s.name)
def test_gemv_full_size(shape):
    print(f"gemv full {shape.name}", flush=True)
    W = wl.build_dense(shape, DEV)
    x = synth.dense_x(shape)
    y = w4.w4a16_gemv(W, wl.bf16_tensor(x))
    ofmt = F.FMT_E2M1 if shape.fmt == "e2m1" else F.FMT_INT4
    ref = oracle.gemv(ofmt, *oracle.quantize(ofmt, synth.dense_weight(shape)), x)
    assert_bf16_close(wl.bf16_bits(y), ref, shape.name)


def test_gemv_canary_and_determinism():
    shape = synth.GEMV_E2M1
    W = wl.build_dense(shape, DEV)
    x = wl.bf16_tensor(synth.dense_x(shape))
    guard = 4096
    buf = torch.full((shape.n + 2 * guard,), 12345, dtype=torch.int16, device=DEV)
    y = buf[guard:guard + shape.n].view(torch.bfloat16)
    w4.w4a16_gemv(W, x, y=y)
    first = y.clone()
    for _ in range(3):
        w4.w4a16_gemv(W, x, y=y)
        assert torch.equal(y.view(torch.int16), first.view(torch.int16))
    assert torch.all(buf[:guard] == 12345) and torch.all(buf[guard + shape.n:] == 12345)


# ---------------------------------------------------------------- MoE layer


@pytest.fixture(scope="module")
def tiny():
    shape = synth.TINY_MOE
    return shape, wl.build_moe_layer(shape, device=DEV), oracle_layer(shape)


def _check_moe(shape, dev_layer, or_layer, x_bits, what):
    T = x_bits.shape[0]
    x = wl.bf16_tensor(x_bits)
    ids = torch.full((T, shape.top_k), -7, dtype=torch.int32, device=DEV)
    wts = torch.zeros((T, shape.top_k), dtype=torch.float32, device=DEV)
    y = w4.moe_w4a16_forward(dev_layer, x, topk_ids=ids, topk_w=wts)
    ref, rids, rw = ops.moe_forward(or_layer, x_bits)
    assert np.array_equal(ids.cpu().numpy(), rids), what
    np.testing.assert_allclose(wts.cpu().numpy(), rw, rtol=2e-6, atol=1e-7)
    return assert_bf16_close(wl.bf16_bits(y), ref, what)


def test_moe_tiny_t1(tiny):
    shape, dev_layer, or_layer = tiny
    for t in range(4):
        print(f"moe tiny token {t}", flush=True)
        _check_moe(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, 1, first=t), f"tiny t={t}")


def test_moe_tiny_batch(tiny):
    shape, dev_layer, or_layer = tiny
    _check_moe(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, 7, first=10), "tiny T=7")


def test_moe_tiny_experts_entry_and_bad_ids(tiny):
    shape, dev_layer, or_layer = tiny
    xb = tie_free_tokens(shape, or_layer, 3, first=20)
    ids = np.array([[1, 6], [6, 1], [3, 3]], dtype=np.int32)
    w = np.array([[0.7, 0.3], [0.5, 0.5], [1.0, 0.25]], dtype=np.float32)
    y = w4.moe_w4a16_experts(dev_layer, wl.bf16_tensor(xb), torch.from_numpy(ids).to(DEV),
                             torch.from_numpy(w).to(DEV))
    ref = ops.moe_experts(or_layer, xb, ids, w.astype(np.float64))
    assert_bf16_close(wl.bf16_bits(y), ref, "experts entry")
    # an id outside [0, E) reads nothing and turns that token's output into NaN
    bad = ids.copy()
    bad[1, 0] = shape.num_experts + 5
    y2 = w4.moe_w4a16_experts(dev_layer, wl.bf16_tensor(xb), torch.from_numpy(bad).to(DEV),
                              torch.from_numpy(w).to(DEV))
    g = oracle.bf16_bits_to_f64(wl.bf16_bits(y2))
    assert np.all(np.isnan(g[1])) and np.all(np.isfinite(g[0])) and np.all(np.isfinite(g[2]))


@pytest.mark.parametrize("T", [4, 40, 64])
def test_moe_tiny_batched_groups(tiny, T):
    """Batched path: small and MFMA-sized (>= 16 token) expert groups, ragged tiles."""
    shape, dev_layer, or_layer = tiny
    assert w4.moe_w4a16_stage_count(dev_layer, T) == 5
    print(f"moe tiny batched T={T}", flush=True)
    _check_moe(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, T, first=100 + T), f"tiny T={T}")


def test_moe_tiny_batched_experts_entry(tiny):
    shape, dev_layer, or_layer = tiny
    T = 24
    xb = tie_free_tokens(shape, or_layer, T, first=300)
    rng = np.random.default_rng(5)
    ids = np.stack([rng.choice(shape.num_experts, shape.top_k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[:20, 0] = 3  # one expert with a group of >= 16 rows (MFMA)
    ids[:20, 1] = np.where(ids[:20, 1] == 3, 4, ids[:20, 1])
    w = rng.uniform(0.1, 1.0, size=(T, shape.top_k)).astype(np.float32)
    y = w4.moe_w4a16_experts(dev_layer, wl.bf16_tensor(xb), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV))
    ref = ops.moe_experts(or_layer, xb, ids, w.astype(np.float64))
    assert_bf16_close(wl.bf16_bits(y), ref, "batched experts entry")
    bad = ids.copy()
    bad[7, 1] = -1
    y2 = w4.moe_w4a16_experts(dev_layer, wl.bf16_tensor(xb), torch.from_numpy(bad).to(DEV),
                              torch.from_numpy(w).to(DEV))
    g = oracle.bf16_bits_to_f64(wl.bf16_bits(y2))
    assert np.all(np.isnan(g[7])) and np.all(np.isfinite(np.delete(g, 7, axis=0)))


def test_moe_tiny_zero_input(tiny):
    shape, dev_layer, _ = tiny
    y = w4.moe_w4a16_forward(dev_layer, torch.zeros((2, shape.hidden), dtype=torch.bfloat16, device=DEV))
    assert torch.all(y.float() == 0)


@pytest.fixture(scope="module")
def qwen():
    shape = synth.QWEN_MOE_T1
    print("building the 35B-A3B-shaped layer", flush=True)
    return shape, wl.build_moe_layer(shape, device=DEV), oracle_layer(shape)


def test_moe_full_t1(qwen):
    shape, dev_layer, or_layer = qwen
    for t in range(3):
        print(f"moe full token {t}", flush=True)
        rep = _check_moe(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, 1, first=t), f"full t={t}")
        print(rep, flush=True)


def test_moe_full_determinism_and_canary(qwen):
    shape, dev_layer, or_layer = qwen
    x = wl.bf16_tensor(tie_free_tokens(shape, or_layer, 1, first=5))
    guard = 2048
    buf = torch.full((shape.hidden + 2 * guard,), 777, dtype=torch.int16, device=DEV)
    y = buf[guard:guard + shape.hidden].view(torch.bfloat16).view(1, -1)
    ws = w4.alloc_workspace(dev_layer, 1)
    w4.moe_w4a16_forward(dev_layer, x, y=y, ws=ws)
    first = y.clone()
    for _ in range(3):
        w4.moe_w4a16_forward(dev_layer, x, y=y, ws=ws)
        assert torch.equal(y.view(torch.int16), first.view(torch.int16))
    assert torch.all(buf[:guard] == 777) and torch.all(buf[guard + shape.hidden:] == 777)


def test_moe_full_batch32_zipf():
    shape = synth.QWEN_MOE_T32
    print("building the batch-32 Zipf layer", flush=True)
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    assert w4.moe_w4a16_stage_count(dev_layer, shape.tokens) == 5
    or_layer = oracle_layer(shape)
    xb = tie_free_tokens(shape, or_layer, shape.tokens)
    # the group sizes this batch produces (the oracle's routing): some use MFMA
    _, rids, _ = ops.moe_forward(or_layer, xb)
    sizes = np.bincount(rids.ravel(), minlength=shape.num_experts)
    print("groups", int((sizes > 0).sum()), "of >= 16 rows:", int((sizes >= 16).sum()), "largest", int(sizes.max()),
          flush=True)
    assert (sizes >= 16).any()
    rep = _check_moe(shape, dev_layer, or_layer, xb, "batch32")
    print(rep, flush=True)
    # determinism across runs
    x = wl.bf16_tensor(xb)
    y1 = w4.moe_w4a16_forward(dev_layer, x)
    y2 = w4.moe_w4a16_forward(dev_layer, x)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_gemv_lmhead_sampled_rows():
    """The lm_head-sized projection (248,320 x 2048, 318 MB packed) in the launch
    configuration bench.py times, checked on sampled rows (the oracle computes rows
    independently: the first and last 256 and 2,048 random ones)."""
    shape = synth.GEMV_LMHEAD
    print(f"gemv {shape.name}", flush=True)
    w = synth.dense_weight(shape)
    codes, scales = w4.w4_quantize(w4.W4_FMT_E2M1_F16S16, w)
    W = _upload(w4.W4_FMT_E2M1_F16S16, codes, scales)
    del codes, scales
    x = synth.dense_x(shape)
    got = wl.bf16_bits(w4.w4a16_gemv(W, wl.bf16_tensor(x)))
    rng = np.random.default_rng(17)
    rows = np.unique(np.concatenate([np.arange(256), np.arange(shape.n - 256, shape.n),
                                     rng.choice(shape.n, 2048, replace=False)]))
    ref = oracle.gemv(F.FMT_E2M1, *oracle.quantize(F.FMT_E2M1, w[rows]), x)
    assert_bf16_close(got[rows], ref, shape.name)


# ---------------------------------------------------------------- bf16 shared expert


@pytest.mark.parametrize("shape", [synth.TINY_MOE_BF16SH, synth.QWEN_MOE_T1_BF16SH], ids=lambda s: s.name)
def test_moe_bf16_shared_expert(shape):
    """Routed E2M1 experts with an unquantised bf16 shared expert."""
    print(f"building {shape.name}", flush=True)
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    assert dev_layer.shared_w13.fmt == w4.W4_FMT_BF16
    or_layer = oracle_layer(shape)
    for t in range(2):
        print(f"bf16 shared token {t}", flush=True)
        print(_check_moe(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, 1, first=t), f"{shape.name} t={t}"),
              flush=True)
    # batches run grouped, the shared expert's bf16 rows as MFMA operands
    assert w4.moe_w4a16_stage_count(dev_layer, 6) == 5
    _check_moe(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, 6, first=40), f"{shape.name} T=6")


def test_moe_bf16_shared_expert_batches():
    """Tiny layer: grouped batches (the shared expert a bf16 MFMA group of T
    rows), past 1024 pairs with the three-launch grouping."""
    shape = synth.TINY_MOE_BF16SH
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    or_layer = oracle_layer(shape)
    for T, stages in ((300, 5), (512, 5), (513, 7), (2049, 7)):  # top-2: 1024 pairs at T = 512
        print(f"bf16 shared tiny T={T}", flush=True)
        assert w4.moe_w4a16_stage_count(dev_layer, T) == stages, T
        _check_moe(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, T, first=500), f"bf16 shared T={T}")


def test_moe_bf16_shared_expert_t32_zipf_sampled():
    """35B-A3B shape, T = 32 with the Zipf router bias: the whole batch on the
    device, every fourth token against the oracle."""
    shape = synth.QWEN_MOE_T32_BF16SH
    print(f"building {shape.name}", flush=True)
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    or_layer = oracle_layer(shape)
    xb = tie_free_tokens(shape, or_layer, shape.tokens, first=60)
    assert w4.moe_w4a16_stage_count(dev_layer, shape.tokens) == 5
    ids = torch.full((shape.tokens, shape.top_k), -7, dtype=torch.int32, device=DEV)
    y = wl.bf16_bits(w4.moe_w4a16_forward(dev_layer, wl.bf16_tensor(xb), topk_ids=ids))
    rows = list(range(0, shape.tokens, 4))
    ref, rids, _ = ops.moe_forward(or_layer, xb[rows])
    assert np.array_equal(ids.cpu().numpy()[rows], rids)
    print(assert_bf16_close(y[rows], ref, "bf16 shared T=32"), flush=True)


# ---------------------------------------------------------------- int4 batches


def test_moe_int4_batches_tiny():
    """int4 experts (FP16 scale per 128) on the grouped path: tiny layer, groups
    from 1 row (VALU) to ~75 rows (MFMA; the scale applied per 128-wide chunk),
    caller routing with a repeated expert; past 4096 pairs the single-token path."""
    shape = synth.MoEShape("tiny-int4", 256, 128, 8, 2, 128, 1, 0.0, 5, "int4")
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    or_layer = oracle_layer(shape)
    for T, stages in ((5, 5), (40, 5), (300, 5), (2049, 3)):
        print(f"int4 tiny T={T}", flush=True)
        assert w4.moe_w4a16_stage_count(dev_layer, T) == stages, T
        _check_moe(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, T, first=900), f"int4 T={T}")
    xb = tie_free_tokens(shape, or_layer, 6, first=30)
    ids = np.array([[1, 6], [6, 1], [3, 3], [0, 7], [2, 5], [4, 4]], dtype=np.int32)
    w = np.array([[0.7, 0.3], [0.5, 0.5], [1.0, 0.25], [0.125, -0.5], [0.9, 0.1], [0.3, 0.3]], dtype=np.float32)
    y = w4.moe_w4a16_experts(dev_layer, wl.bf16_tensor(xb), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV))
    ref = ops.moe_experts(or_layer, xb, ids, w.astype(np.float64))
    print(assert_bf16_close(wl.bf16_bits(y), ref, "int4 experts entry"), flush=True)


def test_moe_int4_t32_zipf_sampled():
    """35B-A3B shape with int4 experts at T = 32 with the Zipf bias: every
    fourth token against the oracle."""
    shape = synth.QWEN_MOE_T32_INT4
    print(f"building {shape.name}", flush=True)
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    or_layer = oracle_layer(shape)
    xb = tie_free_tokens(shape, or_layer, shape.tokens, first=80)
    assert w4.moe_w4a16_stage_count(dev_layer, shape.tokens) == 5
    ids = torch.full((shape.tokens, shape.top_k), -7, dtype=torch.int32, device=DEV)
    y = wl.bf16_bits(w4.moe_w4a16_forward(dev_layer, wl.bf16_tensor(xb), topk_ids=ids))
    rows = list(range(0, shape.tokens, 4))
    ref, rids, _ = ops.moe_forward(or_layer, xb[rows])
    assert np.array_equal(ids.cpu().numpy()[rows], rids)
    print(assert_bf16_close(y[rows], ref, "int4 T=32"), flush=True)


def test_moe_nvfp4_with_bf16_shared_expert():
    shape = synth.MoEShape("tiny-nvfp4-bf16shared", 256, 128, 8, 2, 128, 1, 0.0, 0, "nvfp4", "bf16")
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    or_layer = oracle_layer(shape)
    _check_moe(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, 3, first=7), "nvfp4 + bf16 shared")
    assert w4.moe_w4a16_stage_count(dev_layer, 40) == 5
    _check_moe(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, 40, first=70), "nvfp4 + bf16 shared T=40")
