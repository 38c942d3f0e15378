"""The layer under HIP graph capture (how bench.py times it): a captured forward,
replayed several times with other eager work and synchronisations between the
replays, gives exactly the eager result every time (the kernels are
deterministic and the library records no memset or allocation in the graph).
Covers the single-token path, the grouped paths (E2M1, NVFP4, MX) and the
multi-launch grouping of large batches."""

import numpy as np
import pytest
import torch

import bit_block_scaled_router_amd as w4
from bit_block_scaled_router_amd import synth, workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CASES = [
    ("e2m1 T=1", synth.TINY_MOE, 1),
    ("e2m1 T=40", synth.TINY_MOE, 40),
    ("nvfp4 T=40", synth.MoEShape("tiny-nvfp4", 256, 128, 8, 2, 128, 1, 0.0, 0, "nvfp4"), 40),
    ("mxfp4 T=7", synth.TINY_MOE_MX, 7),
    ("e2m1 T=2500 (three-launch grouping)", synth.TINY_MOE, 2500),
]


@pytest.mark.parametrize("name,shape,T", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, shape, T):
    print(f"graph {name}", flush=True)
    layer = wl.build_moe_layer(shape, device="cuda")
    xa = wl.bf16_tensor(np.stack([synth.x_row(3, shape.hidden, t) for t in range(T)]), "cuda")
    xb = wl.bf16_tensor(np.stack([synth.x_row(4, shape.hidden, t) for t in range(T)]), "cuda")
    ws = w4.alloc_workspace(layer, T)
    y = torch.empty_like(xa)
    ids = torch.empty((T, shape.top_k), dtype=torch.int32, device="cuda")
    w4.moe_w4a16_forward(layer, xa, y=y, topk_ids=ids, ws=ws)
    torch.cuda.synchronize()
    want, want_ids = y.clone(), ids.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            w4.moe_w4a16_forward(layer, xa, y=y, topk_ids=ids, ws=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        # other eager work on the same buffers between replays
        w4.moe_w4a16_forward(layer, xb, y=y, topk_ids=ids, ws=ws)
        torch.cuda.synchronize()
        assert not torch.equal(y, want) or T == 0
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), want.view(torch.int16)), (name, rep)
        assert torch.equal(ids, want_ids), (name, rep)
    del g
