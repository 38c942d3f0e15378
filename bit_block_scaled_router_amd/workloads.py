"""Device-resident workloads built from the seeded synthetic weights.

The fp32 weights come from `synth` (random draws only); quantisation uses the
library's own host quantiser (w4_quantize) and the results are uploaded to
device memory in the canonical layout or, packed on the host by w4_pack, in the
device layout (W4_LAYOUT_GFX950_V1).
"""

import numpy as np

from . import synth
from . import (
    GROUP,
    FORMATS,
    SCALE_DTYPE,
    MoELayer,
    QMatrix,
    W4_FMT_NVFP4_E4M3S16,
    W4_FMT_BF16,
    W4_LAYOUT_CANONICAL,
    w4_quantize,
)


def quantize_stack(fmt, gen, groups, n, k):
    """Quantise `groups` matrices gen(g) -> fp32 [n][k] into stacked host arrays:
    (codes, scales) or, for NVFP4, (codes, scales, global scales fp32 [groups])."""
    codes = np.empty((groups, n, k // 2), dtype=np.uint8)
    scales = np.empty((groups, n, k // GROUP[fmt]), dtype=SCALE_DTYPE[fmt])
    gsc = np.zeros(groups, dtype=np.float32)
    for g in range(groups):
        r = w4_quantize(fmt, gen(g), codes[g], scales[g])
        if fmt == W4_FMT_NVFP4_E4M3S16:
            gsc[g] = r[2]
    return (codes, scales, gsc) if fmt == W4_FMT_NVFP4_E4M3S16 else (codes, scales)


def upload(fmt, q, device, layout=W4_LAYOUT_CANONICAL):
    """QMatrix from the output of quantize_stack / w4_quantize, in `layout`."""
    if fmt == W4_FMT_BF16:
        return QMatrix.upload_bf16(q[0], device)
    return QMatrix.upload(fmt, q[0], q[1], device, global_np=q[2] if len(q) > 2 else None, layout=layout)


def build_moe_layer(shape, fmt=None, device="cuda", layout=W4_LAYOUT_CANONICAL, w2_layout=None):
    """Quantise and upload a whole MoE layer of `shape` (a synth.MoEShape) in the
    shape's weight format (or `fmt`, a W4_FMT_* tag) and the given layout;
    w2_layout (default: layout) for the down projections (routed and shared),
    e.g. the K-tiled layout of the decode kernels."""
    import torch

    fmt = FORMATS[shape.fmt] if fmt is None else fmt

    q13 = quantize_stack(fmt, lambda e: synth.expert_w13(shape, e), shape.num_experts, 2 * shape.inter, shape.hidden)
    q2 = quantize_stack(fmt, lambda e: synth.expert_w2(shape, e), shape.num_experts, shape.hidden, shape.inter)
    w2_layout = layout if w2_layout is None else w2_layout
    w13 = upload(fmt, q13, device, layout)
    w2 = upload(fmt, q2, device, w2_layout)
    del q13, q2
    router_w = torch.from_numpy(synth.router_weight(shape).view(np.int16)).to(device)
    bias = synth.router_bias(shape)
    router_bias = torch.from_numpy(bias).to(device) if bias is not None else None
    kw = {}
    if shape.has_shared:
        sfmt = FORMATS[shape.shared_fmt] if shape.shared_fmt else fmt
        kw = dict(
            shared_w13=upload(sfmt, w4_quantize(sfmt, synth.shared_w13(shape)), device, layout),
            shared_w2=upload(sfmt, w4_quantize(sfmt, synth.shared_w2(shape)), device, w2_layout),
            shared_gate_w=torch.from_numpy(synth.shared_gate_weight(shape).view(np.int16)).to(device),
        )
    return MoELayer(shape.hidden, shape.inter, shape.num_experts, shape.top_k, router_w, w13, w2,
                    router_bias=router_bias, **kw)


def build_dense(shape, device="cuda", layout=W4_LAYOUT_CANONICAL):
    """Quantise and upload a dense GEMV matrix of `shape` (a synth.GemvShape)."""
    fmt = FORMATS[shape.fmt]
    return upload(fmt, w4_quantize(fmt, synth.dense_weight(shape)), device, layout)


def bf16_tensor(bits, device="cuda"):
    """bf16 bit patterns (uint16 numpy) -> torch bfloat16 tensor on `device`."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def bf16_bits(t):
    """torch bfloat16 tensor -> uint16 numpy bit patterns (host copy)."""
    import torch

    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
