"""Device-resident workloads built from the seeded synthetic weights.

The fp32 weights come from `synth` (random draws only); quantisation uses the
library's own host quantiser (w4_quantize) and the results are uploaded to
device memory as the library's canonical layout.
"""

import numpy as np

from . import synth
from . import (
    GROUP,
    FORMATS,
    MoELayer,
    QMatrix,
    W4_FMT_E2M1_F16S16,
    w4_quantize,
)


def quantize_stack(fmt, gen, groups, n, k):
    """Quantise `groups` matrices gen(g) -> fp32 [n][k] into stacked host arrays."""
    codes = np.empty((groups, n, k // 2), dtype=np.uint8)
    scales = np.empty((groups, n, k // GROUP[fmt]), dtype=np.uint16)
    for g in range(groups):
        w4_quantize(fmt, gen(g), codes[g], scales[g])
    return codes, scales


def build_moe_layer(shape, fmt=W4_FMT_E2M1_F16S16, device="cuda"):
    """Quantise and upload a whole MoE layer of `shape` (a synth.MoEShape)."""
    import torch

    c13, s13 = quantize_stack(fmt, lambda e: synth.expert_w13(shape, e), shape.num_experts,
                              2 * shape.inter, shape.hidden)
    c2, s2 = quantize_stack(fmt, lambda e: synth.expert_w2(shape, e), shape.num_experts,
                            shape.hidden, shape.inter)
    w13 = QMatrix.upload(fmt, c13, s13, device)
    w2 = QMatrix.upload(fmt, c2, s2, device)
    del c13, s13, c2, s2
    router_w = torch.from_numpy(synth.router_weight(shape).view(np.int16)).to(device)
    bias = synth.router_bias(shape)
    router_bias = torch.from_numpy(bias).to(device) if bias is not None else None
    kw = {}
    if shape.has_shared:
        sc13, ss13 = w4_quantize(fmt, synth.shared_w13(shape))
        sc2, ss2 = w4_quantize(fmt, synth.shared_w2(shape))
        kw = dict(
            shared_w13=QMatrix.upload(fmt, sc13, ss13, device),
            shared_w2=QMatrix.upload(fmt, sc2, ss2, device),
            shared_gate_w=torch.from_numpy(synth.shared_gate_weight(shape).view(np.int16)).to(device),
        )
    return MoELayer(shape.hidden, shape.inter, shape.num_experts, shape.top_k, router_w, w13, w2,
                    router_bias=router_bias, **kw)


def build_dense(shape, device="cuda"):
    """Quantise and upload a dense GEMV matrix of `shape` (a synth.GemvShape)."""
    fmt = FORMATS[shape.fmt]
    codes, scales = w4_quantize(fmt, synth.dense_weight(shape))
    return QMatrix.upload(fmt, codes, scales, device)


def bf16_tensor(bits, device="cuda"):
    """bf16 bit patterns (uint16 numpy) -> torch bfloat16 tensor on `device`."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def bf16_bits(t):
    """torch bfloat16 tensor -> uint16 numpy bit patterns (host copy)."""
    import torch

    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
