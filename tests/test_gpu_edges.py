"""GPU parity at the edges of the supported ranges: the largest expert count and
top-k, hidden sizes off the 128 grid (single-token path), int4 experts, the
largest batches of the two grouping paths (T k = 1024 and 4096 pairs) and the
largest token count."""

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import ops
import bit_block_scaled_router_amd as w4
from bit_block_scaled_router_amd import synth, workloads as wl
from moe_cases import assert_bf16_close, oracle_layer, tie_free_tokens

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


def _run(shape, dev_layer, x_bits):
    T = x_bits.shape[0]
    ids = torch.full((T, shape.top_k), -7, dtype=torch.int32, device=DEV)
    wts = torch.zeros((T, shape.top_k), dtype=torch.float32, device=DEV)
    y = w4.moe_w4a16_forward(dev_layer, wl.bf16_tensor(x_bits), topk_ids=ids, topk_w=wts)
    return wl.bf16_bits(y), ids.cpu().numpy(), wts.cpu().numpy()


def _check(shape, dev_layer, or_layer, x_bits, what, rows=None):
    got, ids, wts = _run(shape, dev_layer, x_bits)
    rows = np.arange(x_bits.shape[0]) if rows is None else rows
    ref, rids, rw = ops.moe_forward(or_layer, x_bits, tokens=list(rows))
    assert np.array_equal(ids[rows], rids), what
    np.testing.assert_allclose(wts[rows], rw, rtol=2e-6, atol=1e-7)
    return assert_bf16_close(got[rows], ref, what)


EDGE_SHAPES = [
    # largest expert count and top-k (64 lanes x 16 logits ranked per wave); T = 5 is grouped
    (synth.MoEShape("edge-e1024-k16", 256, 128, 1024, 16, 0, 1, 0.0, 3), (1, 5)),
    # hidden off the 128 grid, ragged intermediate: the single-token path for every T
    (synth.MoEShape("edge-h320-i96", 320, 96, 16, 4, 96, 1, 0.0, 4), (1, 6)),
    # int4 experts (FP16 scale per 128) with an int4 shared expert
    (synth.MoEShape("edge-int4", 256, 128, 8, 2, 128, 1, 0.0, 5, "int4"), (1, 6)),
]


@pytest.mark.parametrize("shape,Ts", EDGE_SHAPES, ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_edge_layers(shape, Ts):
    print(f"edge {shape.name}", flush=True)
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    or_layer = oracle_layer(shape)
    for T in Ts:
        print(f"  T={T} stages={w4.moe_w4a16_stage_count(dev_layer, T)}", flush=True)
        _check(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, T, first=11 * T), f"{shape.name} T={T}")


@pytest.mark.parametrize("T,stages", [(128, 5), (512, 7)])
def test_largest_grouped_batches(T, stages):
    """T k = 1024 (token, slot) pairs, the largest batch of the one-launch
    grouping and the per-group MFMA kernels, and T k = 4096 on the three-launch
    grouping and the large-batch kernels (groups of ~64 rows)."""
    shape = synth.MoEShape("edge-pairs", 256, 128, 64, 8, 128, T, 0.0, 6)
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    assert w4.moe_w4a16_stage_count(dev_layer, T) == stages
    or_layer = oracle_layer(shape)
    print(f"pairs {8 * T}", flush=True)
    _check(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, T), f"T={T} k=8")


def test_largest_token_count_sampled():
    """T = 4096 on the single-token path (int4 experts), checked on 48 sampled tokens."""
    shape = synth.MoEShape("edge-t4096-int4", 256, 128, 8, 2, 128, 4096, 0.0, 7, "int4")
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    assert w4.moe_w4a16_stage_count(dev_layer, 4096) == 3
    or_layer = oracle_layer(shape)
    x = np.stack([synth.x_row(shape.seed, shape.hidden, t) for t in range(4096)])
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 4095], rng.choice(4096, 46, replace=False)]))
    # sampled tokens must be tie-free for the id comparison
    keep = [r for r in rows if __import__("moe_cases").min_gap(or_layer, x[r]) >= 1e-3]
    print(f"T=4096 sampled {len(keep)}", flush=True)
    _check(shape, dev_layer, or_layer, x, "T=4096", rows=np.array(keep))


# The router's special cases: k = 1 (the single selected expert's renormalised
# weight is exactly 1) and k = E (every expert selected; the weights are the full
# softmax, ids in descending order).  Both on the single-token path (T < 4) and
# the grouped path (T >= 4), with and without a shared expert.
ROUTER_EDGE = [
    synth.MoEShape("edge-k1", 256, 128, 8, 1, 0, 1, 0.0, 21),
    synth.MoEShape("edge-k1-shared", 256, 128, 8, 1, 128, 1, 0.0, 22),
    synth.MoEShape("edge-kE", 256, 128, 8, 8, 0, 1, 0.0, 23),
    synth.MoEShape("edge-kE-shared", 256, 128, 8, 8, 128, 1, 0.0, 24),
]


@pytest.mark.parametrize("shape", ROUTER_EDGE, ids=lambda s: s.name)
@pytest.mark.parametrize("T", [1, 3, 6, 40])
def test_router_extremes(shape, T):
    print(f"router edge {shape.name} T={T}", flush=True)
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    or_layer = oracle_layer(shape)
    x = tie_free_tokens(shape, or_layer, T, first=7 * T)
    got, ids, wts = _run(shape, dev_layer, x)
    ref, rids, rw = ops.moe_forward(or_layer, x)
    assert np.array_equal(ids, rids), (ids, rids)
    if shape.top_k == 1:
        assert np.all(wts == 1.0), wts  # w / sum(w) over one expert: exactly 1
    else:
        assert np.array_equal(np.sort(ids, axis=1), np.tile(np.arange(shape.num_experts), (T, 1)))
        np.testing.assert_allclose(wts.sum(axis=1), 1.0, rtol=1e-6)
    np.testing.assert_allclose(wts, rw, rtol=2e-6, atol=1e-7)
    assert_bf16_close(got, ref, f"{shape.name} T={T}")


def test_ranking_blocks_across_calls():
    """Routed batches rank their tokens over ceil(T/4) blocks and the last block to
    arrive groups the pairs; the router launch zeroes the arrival counter in every
    call.  One workspace serves calls of different sizes back to back (ragged T,
    one block, 128 blocks), eagerly and replayed from a captured graph with eager
    calls of other sizes between the replays."""
    shape = synth.MoEShape("edge-rank", 256, 128, 64, 8, 128, 1, 0.0, 25)
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    or_layer = oracle_layer(shape)
    ws = w4.alloc_workspace(dev_layer, 509)

    def call(x_bits):
        T = x_bits.shape[0]
        ids = torch.full((T, shape.top_k), -7, dtype=torch.int32, device=DEV)
        wts = torch.zeros((T, shape.top_k), dtype=torch.float32, device=DEV)
        y = w4.moe_w4a16_forward(dev_layer, wl.bf16_tensor(x_bits), topk_ids=ids, topk_w=wts, ws=ws)
        return y, ids, wts

    xs = {T: tie_free_tokens(shape, or_layer, T, first=13 * T) for T in (509, 7, 4, 130, 33)}
    for T in (509, 7, 4, 130, 509):
        print(f"rank blocks T={T}", flush=True)
        y, ids, wts = call(xs[T])
        ref, rids, rw = ops.moe_forward(or_layer, xs[T])
        assert np.array_equal(ids.cpu().numpy(), rids), T
        np.testing.assert_allclose(wts.cpu().numpy(), rw, rtol=2e-6, atol=1e-7)
        assert_bf16_close(wl.bf16_bits(y), ref, f"rank blocks T={T}")
    # graph replays of a T = 33 call, eager calls of other sizes in between
    x33 = wl.bf16_tensor(xs[33])
    y33 = torch.empty((33, shape.hidden), dtype=torch.bfloat16, device=DEV)
    w4.moe_w4a16_forward(dev_layer, x33, y=y33, ws=ws)
    torch.cuda.synchronize()
    eager = y33.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            w4.moe_w4a16_forward(dev_layer, x33, y=y33, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    for T in (7, 130, 4):
        y33.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y33, eager), "graph replay"
        call(xs[T])
        torch.cuda.synchronize()
