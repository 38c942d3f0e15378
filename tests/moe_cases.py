"""Shared helpers of the GPU parity tests: oracle layers, tie-free tokens, tolerances.

Tolerances: bf16 outputs must satisfy max|gpu - oracle| <= 1e-2 * max|oracle| and
relative L1 error sum|gpu - oracle| / sum|oracle| <= 2e-3 (the mean relative
error bound of the parity bar); top-k ids and dequantised weights are bit-exact.
The mean bound is applied to outputs of at least MEAN_MIN elements: a single
round-to-nearest bf16 result alone may sit 2**-8 relative from the exact value,
so a mean over a handful of elements measures rounding luck, not the kernel.
Every element, whatever the size, must also be within one bf16 rounding
(2**-8 relative) of the oracle plus an fp32-accumulation allowance of
1e-5 * max|oracle|.

The MX path's per-element allowance is derived from the scaled MFMA's
arithmetic instead (elem_allow; test_gpu_mx states the model).
"""

import numpy as np

import oracle
from oracle import formats as F
from oracle import ops
from bit_block_scaled_router_amd import synth

MAX_REL = 1e-2
MEAN_REL = 2e-3
MEAN_MIN = 256
GAP = 1e-3  # minimum adjacent gap among the k+1 largest logits of a parity token


_OFMT = {"e2m1": F.FMT_E2M1, "int4": F.FMT_INT4, "nvfp4": F.FMT_NVFP4, "bf16": F.FMT_BF16, "mxfp4": F.FMT_MXFP4}


def oracle_layer(shape, fmt=None):
    """Oracle view of a synth layer; experts are quantised lazily by the oracle.
    fmt: oracle format of the routed experts (default: the shape's)."""
    fmt = _OFMT[shape.fmt] if fmt is None else fmt
    sfmt = _OFMT[shape.shared_fmt] if shape.shared_fmt else fmt
    kw = {}
    if shape.has_shared:
        kw = dict(shared_w13=oracle.quantize(sfmt, synth.shared_w13(shape)),
                  shared_w2=oracle.quantize(sfmt, synth.shared_w2(shape)),
                  shared_gate_w=synth.shared_gate_weight(shape), shared_fmt=sfmt)
    return ops.MoELayer(
        fmt, shape.hidden, shape.inter, shape.num_experts, shape.top_k, synth.router_weight(shape),
        lambda e: oracle.quantize(fmt, synth.expert_w13(shape, e)),
        lambda e: oracle.quantize(fmt, synth.expert_w2(shape, e)),
        router_bias=synth.router_bias(shape), **kw)


def min_gap(layer, x_bits):
    z = ops.router_logits(layer.router_w, x_bits, layer.router_bias)
    top = np.sort(z)[::-1][: layer.top_k + 1]
    return float(np.min(-np.diff(top))) if top.size > 1 else np.inf


def tie_free_tokens(shape, layer, T, first=0):
    """T activation rows; a row whose top-(k+1) logits have a gap < GAP is redrawn."""
    rows = []
    for t in range(first, first + T):
        for attempt in range(100):
            x = synth.x_row(shape.seed, shape.hidden, t, attempt)
            if min_gap(layer, x) >= GAP:
                rows.append(x)
                break
        else:
            raise RuntimeError("no tie-free draw")
    return np.stack(rows)


def assert_bf16_close(gpu_bits, ref, what="", elem_abs=1e-5, elem_allow=None):
    """Parity bounds above; elem_allow (same shape as ref) adds a derived
    per-element allowance to the one-rounding bound."""
    g = oracle.bf16_bits_to_f64(gpu_bits)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    rep = oracle.error_report(g, r)
    assert rep["max_abs"] <= MAX_REL * rep["max_ref"], (what, rep)
    if g.size >= MEAN_MIN:
        assert rep["rel_l1"] <= MEAN_REL, (what, rep)
    bound = np.abs(r) * 2.0 ** -8 + elem_abs * rep["max_ref"]
    if elem_allow is not None:
        bound = bound + elem_allow
    bad = np.abs(g - r) > bound
    assert not bad.any(), (what, int(bad.sum()), rep)
    return rep
