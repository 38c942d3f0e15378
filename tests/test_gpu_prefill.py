"""GPU parity of prefill-sized batches (more than 1024 (token, slot) pairs): the
router as an MFMA GEMM, the grouping over three launches (per-block top-k and
expert histograms, one scan, a scatter), and the grouped expert kernels with
groups of hundreds of rows.  Routing ids are compared for every token; outputs
for every token of the tiny layer and for sampled tokens of the 35B-A3B-shaped
layer (E2M1, NVFP4, a bf16 shared expert, and MX)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import ops
import bit_block_scaled_router_amd as w4
from bit_block_scaled_router_amd import synth, workloads as wl
from moe_cases import assert_bf16_close, oracle_layer, tie_free_tokens

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


def _run(dev_layer, xb, K):
    T = xb.shape[0]
    ids = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    wts = torch.zeros((T, K), dtype=torch.float32, device=DEV)
    y = w4.moe_w4a16_forward(dev_layer, wl.bf16_tensor(xb), topk_ids=ids, topk_w=wts)
    torch.cuda.synchronize()
    return wl.bf16_bits(y), ids.cpu().numpy(), wts.cpu().numpy()


def _check_routing(or_layer, xb, ids, wts, K):
    for t in range(xb.shape[0]):
        rids, rw = ops.route(ops.router_logits(or_layer.router_w, xb[t], or_layer.router_bias), K)
        assert np.array_equal(ids[t], rids), t
        np.testing.assert_allclose(wts[t], rw, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("fmt,shared_fmt", [("e2m1", None), ("nvfp4", None), ("e2m1", "bf16"), ("nvfp4", "bf16")])
def test_prefill_tiny_every_token(fmt, shared_fmt):
    """Tiny layer (8 experts, top-2), T = 3000: 6000 pairs, groups of ~750 rows;
    E2M1 or NVFP4 routed experts, the shared expert in their format or bf16."""
    shape = synth.MoEShape("tiny-prefill-3000", 256, 128, 8, 2, 128, 3000, 0.0, 11, fmt, shared_fmt)
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    assert w4.moe_w4a16_stage_count(dev_layer, 3000) == 7
    or_layer = oracle_layer(shape)
    xb = tie_free_tokens(shape, or_layer, 3000)
    what = f"tiny prefill T=3000 {fmt} shared {shared_fmt or fmt}"
    print(what, flush=True)
    y, ids, wts = _run(dev_layer, xb, shape.top_k)
    _check_routing(or_layer, xb, ids, wts, shape.top_k)
    ref, _, _ = ops.moe_forward(or_layer, xb)
    print(assert_bf16_close(y, ref, what), flush=True)


def test_prefill_tiny_experts_entry_with_invalid_ids():
    """Caller routing at T = 2500 (5000 pairs) with skewed and invalid ids: the
    invalid slots join no group and their tokens come out NaN."""
    shape = synth.MoEShape("tiny-prefill-2500", 256, 128, 8, 2, 128, 2500, 0.0, 12)
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    or_layer = oracle_layer(shape)
    T = 2500
    xb = np.stack([synth.x_row(shape.seed, shape.hidden, t) for t in range(T)])
    rng = np.random.default_rng(13)
    ids = np.stack([rng.choice(8, 2, replace=False) for _ in range(T)]).astype(np.int32)
    ids[:1500, 0] = 5  # one group of > 1500 rows
    ids[:1500, 1] = np.where(ids[:1500, 1] == 5, 2, ids[:1500, 1])
    w = rng.uniform(0.1, 1.0, size=(T, 2)).astype(np.float32)
    bad = ids.copy()
    bad[[7, 1200, 2499], [1, 0, 1]] = [-1, 8, 99]
    print("tiny prefill experts entry", flush=True)
    y = w4.moe_w4a16_experts(dev_layer, wl.bf16_tensor(xb), torch.from_numpy(bad).to(DEV),
                             torch.from_numpy(w).to(DEV))
    g = oracle.bf16_bits_to_f64(wl.bf16_bits(y))
    nan_rows = [7, 1200, 2499]
    assert all(np.all(np.isnan(g[r])) for r in nan_rows)
    keep = np.setdiff1d(np.arange(T), nan_rows)
    sample = keep[::50]
    ref = ops.moe_experts(or_layer, xb[sample], bad[sample], w[sample].astype(np.float64))
    assert np.all(np.isfinite(g[keep]))
    print(assert_bf16_close(wl.bf16_bits(y)[sample], ref, "tiny prefill experts entry"), flush=True)


@pytest.mark.parametrize("shape", [synth.QWEN_MOE_PREFILL, synth.QWEN_MOE_PREFILL_NVFP4, synth.QWEN_MOE_PREFILL_BF16SH],
                         ids=lambda s: s.name)
def test_prefill_full_sampled(shape):
    """35B-A3B shape, T = 2048 (16,384 pairs): ids for every token, outputs for 8."""
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    T = shape.tokens
    assert w4.moe_w4a16_stage_count(dev_layer, T) == 7
    or_layer = oracle_layer(shape)
    xb = tie_free_tokens(shape, or_layer, T)
    print(f"{shape.name}", flush=True)
    y, ids, wts = _run(dev_layer, xb, shape.top_k)
    _check_routing(or_layer, xb, ids, wts, shape.top_k)
    rows = [0, 1, 511, 1024, 1500, 2000, 2046, 2047]
    ref, _, _ = ops.moe_forward(or_layer, xb, tokens=rows)
    print(assert_bf16_close(y[rows], ref, shape.name), flush=True)


def _sampled_check(shape, T, rows, what):
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    or_layer = oracle_layer(shape)
    xb = np.stack([synth.x_row(shape.seed, shape.hidden, t) for t in range(T)])
    y, ids, wts = _run(dev_layer, xb, shape.top_k)
    import moe_cases
    keep = [r for r in rows if moe_cases.min_gap(or_layer, xb[r]) >= moe_cases.GAP]
    print(f"{what}: {len(keep)} tie-free sampled tokens", flush=True)
    _check_routing(or_layer, xb[keep], ids[keep], wts[keep], shape.top_k)
    ref, _, _ = ops.moe_forward(or_layer, xb, tokens=keep)
    print(assert_bf16_close(y[keep], ref, what), flush=True)


def test_prefill_largest_pair_count():
    """65,536 (token, slot) pairs, the largest grouped call: T = 8192 on the
    35B-A3B shape (~256 pairs per expert, four column tiles per group)."""
    shape = synth.MoEShape("qwen-prefill-8192", 2048, 512, 256, 8, 512, 8192, 0.0, 21)
    rng = np.random.default_rng(31)
    rows = np.unique(np.concatenate([[0, 8191], rng.choice(8192, 10, replace=False)]))
    _sampled_check(shape, 8192, rows, "T=8192 (65536 pairs)")


def test_prefill_largest_token_count():
    """T = 16384 tokens (the entry points' limit) on the tiny layer, top-2:
    32,768 pairs, groups of ~4000 rows."""
    shape = synth.MoEShape("tiny-prefill-16384", 256, 128, 8, 2, 128, 16384, 0.0, 22)
    rng = np.random.default_rng(32)
    rows = np.unique(np.concatenate([[0, 16383], rng.choice(16384, 30, replace=False)]))
    _sampled_check(shape, 16384, rows, "T=16384 tiny")
