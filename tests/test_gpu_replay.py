"""Every launch of the layer can run again on its own, on the inputs the launch
before it left (what bench.py's per-kernel timing and a profiler's replay do):
each kernel node of a captured step is replayed alone, in launch order, and the
step's output must come out as the full step made it.  A kernel that rewrote
its own input in place (the large-batch scan once turned its block histograms
into offsets in place, and a second run of it alone fed the scatter offsets far
past the pair list) or that kept state between launches (the ranking's arrival
counter) fails here instead of in a benchmark."""

import numpy as np
import pytest
import torch

import bench
import bit_block_scaled_router_amd as w4
from bit_block_scaled_router_amd import synth, workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"
SHAPE = synth.MoEShape("replay", 256, 128, 16, 4, 128, 1, 0.0, 41)


@pytest.mark.parametrize("T,stages,layout", [
    (1, 3, w4.W4_LAYOUT_GFX950_V1),      # single-token path
    (40, 5, w4.W4_LAYOUT_GFX950_V1),     # multi-block ranking + one-launch grouping
    (1200, 7, w4.W4_LAYOUT_GFX950_V1),   # three-launch grouping (4800 pairs), large-batch GEMMs
    (3, 3, w4.W4_LAYOUT_GFX950_KT16),    # K-tiled decode kernels
])
def test_each_launch_replays_alone(T, stages, layout):
    print(f"replay T={T} layout={layout}", flush=True)
    l13 = w4.W4_LAYOUT_GFX950_V1
    layer = wl.build_moe_layer(SHAPE, device=DEV, layout=l13, w2_layout=layout)
    assert w4.moe_w4a16_stage_count(layer, T) == stages
    x = wl.bf16_tensor(np.stack([synth.x_row(SHAPE.seed, SHAPE.hidden, t) for t in range(T)]))
    y = torch.empty((T, SHAPE.hidden), dtype=torch.bfloat16, device=DEV)
    ws = w4.alloc_workspace(layer, T)
    w4.moe_w4a16_forward(layer, x, y=y, ws=ws)
    torch.cuda.synchronize()
    eager = y.clone()
    g = torch.cuda.CUDAGraph(keep_graph=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            w4.moe_w4a16_forward(layer, x, y=y, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    g.instantiate()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y, eager)
    hip = bench.HipRuntime()
    chain = hip.kernel_chain(g.raw_cuda_graph())
    assert len(chain) == stages
    cur = torch.cuda.current_stream().cuda_stream
    y.zero_()
    torch.cuda.synchronize()
    for node in chain:  # each launch alone, three times, in launch order
        hip.replay_nodes_us([node], cur, reps=2)
    torch.cuda.synchronize()
    assert torch.equal(y, eager), "per-launch replays"
    y.zero_()
    torch.cuda.synchronize()
    hip.replay_nodes_us(chain, cur, reps=1)  # the whole chain copied out of the graph
    torch.cuda.synchronize()
    assert torch.equal(y, eager), "chain replay"
