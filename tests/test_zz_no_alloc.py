"""The no-allocation entry point (moe_w4a16_forward_noalloc) against the
workspace entry point (moe_w4a16_forward) through the C ABI: the same kernels on
the library's per-GPU scratch, so outputs, ids and weights must match bit for
bit.  Two calls in a row, the second with a smaller batch, on the batched and
the single-token paths; a batch too large for the scratch is refused before
anything runs."""

import numpy as np
import pytest
import torch

import bit_block_scaled_router_amd as w4
from bit_block_scaled_router_amd import synth, workloads as wl

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


def _both(layer, xb):
    T, K = xb.shape[0], layer.top_k
    x = wl.bf16_tensor(xb, DEV)
    out = []
    for noalloc in (False, True):
        y = torch.full((T, layer.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
        ids = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
        wts = torch.zeros((T, K), dtype=torch.float32, device=DEV)
        if noalloc:
            w4.moe_w4a16_forward_noalloc(layer, x, y, topk_ids=ids, topk_w=wts)
        else:
            w4.moe_w4a16_forward(layer, x, y=y, topk_ids=ids, topk_w=wts)
        torch.cuda.synchronize()
        out.append((wl.bf16_bits(y), ids.cpu().numpy(), wts.cpu().numpy()))
    return out


def _rows(shape, T, first):
    return np.stack([synth.x_row(shape.seed, shape.hidden, first + t) for t in range(T)])


@pytest.mark.parametrize("shape,Ts", [
    (synth.QWEN_MOE_T32, (32, 1)),        # grouped path, then the single-token path
    (synth.TINY_MOE_BF16SH, (300, 40)),   # two grouped batches, the second smaller
])
def test_noalloc_matches_workspace_entry(shape, Ts):
    layer = wl.build_moe_layer(shape, device=DEV)
    for i, T in enumerate(Ts):
        need = w4.moe_w4a16_workspace_bytes(layer, T)
        print(f"noalloc {shape.name} T={T} workspace {need} B", flush=True)
        assert need <= 8 << 20
        (y0, i0, w0), (y1, i1, w1) = _both(layer, _rows(shape, T, 100 * i))
        assert np.all(np.isfinite((y0.astype(np.uint32) << 16).view(np.float32)))
        assert np.array_equal(y0, y1) and np.array_equal(i0, i1)
        assert np.array_equal(w0.view(np.uint32), w1.view(np.uint32))


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    shape = synth.TINY_MOE
    layer = wl.build_moe_layer(shape, device=DEV)
    T = 16384
    assert w4.moe_w4a16_workspace_bytes(layer, T) > 8 << 20
    x = torch.zeros((T, shape.hidden), dtype=torch.bfloat16, device=DEV)
    y = torch.zeros_like(x)
    with pytest.raises(w4.W4Error) as e:
        w4.moe_w4a16_forward_noalloc(layer, x, y)
    assert e.value.status == w4.W4_ERR_WORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert not torch.any(y != 0)  # nothing ran
