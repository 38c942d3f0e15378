"""Oracle: dense W4A16 GEMV and the W4A16 mixture-of-experts decode layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Every step is the plain definition, in float64, on exactly dequantised fp32
weights (oracle.formats.dequant) and exactly decoded bf16 activations:

* GEMV: y = W x, the textbook matrix-vector product ("Lynn Engine" article,
  stage P1: the packed W4A16 matvec).
* Router, in the order the lynn-engine tutorials index (note 06, "MoE router")
  gives for Qwen 3.6: softmax over ALL expert logits, then the k largest
  probabilities, then renormalise the k selected probabilities to sum to one.
  The same note states that this equals softmax over the k selected logits;
  route_topk_softmax() is that second form, used only to pin the first.
  Selected ids are sorted by descending probability with ties to the lower expert
  index (lynn-engine README, status note P35: sorted-router contract).
  An optional per-expert logit bias is added before the softmax.
* Shared expert gate: sigma = 1 / (1 + exp(-(w_sg . x))), a scalar per token
  (tutorials index: the shared expert carries a sigmoid gate; the 35B-A3B config
  block lists "shared_expert: sigmoid_gate").
* Expert FFN (SwiGLU): gu = W13 x; g = gu[:I] (gate rows), u = gu[I:] (up rows);
  h = silu(g) * u with silu(g) = g / (1 + exp(-g)); y_e = W2 h
  (lynn-engine README, status notes P28 "gate_up_silu" and P29 "down weighted sum").
* Combine: out = sum_j w_j * y_{e_j} + sigma * y_shared (P29/P45 contracts; the
  shared expert is gated by sigma and not renormalised with the routed weights).
* Tokens are independent; a batch is a loop over tokens.

Reading for the row order of W13: rows [0, I) are the gate projection and rows
[I, 2I) the up projection (the pages say "gate/up" and apply SiLU to the gate).

Parity pins (tests/test_oracle_moe.py): brute force over all k-subsets for E <= 12;
the softmax-all/top-k/renormalise == top-k/softmax equivalence stated by note 06;
k = 1 (weight exactly 1), k = E (weights = full softmax), zero shared-gate weight
(sigma exactly 0.5); E = k = 1 reduces to a dense SwiGLU built from gemv();
x = 0 gives exactly 0; one-hot x picks a column of the dequantised matrix.
"""

import numpy as np

from .formats import FMT_E2M1, FMT_MXFP4, bf16_bits_to_f64, dequant, mx_e4m3


def _as_x(x_bits):
    return bf16_bits_to_f64(x_bits)


# --------------------------------------------------------------------------- GEMV


def gemv(fmt, packed, scale_bits, x_bits, gscale=None):
    """y[N] = dequant(W)[N][K] . x[K], float64.  x given as bf16 bits; gscale is
    the global scale of an NVFP4 matrix."""
    w = dequant(fmt, packed, scale_bits, gscale).astype(np.float64)
    x = _as_x(x_bits)
    if w.shape[1] != x.shape[-1]:
        raise ValueError("K mismatch")
    return w @ x.T if x.ndim == 1 else (x @ w.T)


# --------------------------------------------------------------------------- router


def router_logits(wr_bits, x_bits, bias=None):
    wr = bf16_bits_to_f64(wr_bits)
    x = _as_x(x_bits)
    logits = wr @ x
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float32).astype(np.float64)
    return logits


def router_probs(logits):
    """Softmax over all experts (max-subtracted)."""
    z = np.asarray(logits, dtype=np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def _topk_indices(p, k):
    # descending probability, ties to the lower index
    order = np.lexsort((np.arange(p.shape[0]), -p))
    return order[:k]


def route(logits, k):
    """softmax(all) -> top-k -> renormalise.  Returns (ids int32 [k], weights f64 [k])."""
    p = router_probs(logits)
    if not 1 <= k <= p.shape[0]:
        raise ValueError("bad top_k")
    ids = _topk_indices(p, k)
    sel = p[ids]
    return ids.astype(np.int32), sel / sel.sum()


def route_topk_softmax(logits, k):
    """Second form from tutorials note 06: top-k logits, then softmax over them."""
    z = np.asarray(logits, dtype=np.float64)
    ids = np.lexsort((np.arange(z.shape[0]), -z))[:k]
    sel = z[ids]
    e = np.exp(sel - sel.max())
    return ids.astype(np.int32), e / e.sum()


def shared_gate(wsg_bits, x_bits):
    """sigma = 1 / (1 + exp(-(w_sg . x)))."""
    t = bf16_bits_to_f64(wsg_bits) @ _as_x(x_bits)
    return 1.0 / (1.0 + np.exp(-t))


# --------------------------------------------------------------------------- experts


def silu(g):
    return g / (1.0 + np.exp(-g))


def expert_ffn(w13_f32, w2_f32, x, mx_act=False):
    """SwiGLU expert on dequantised weights; x float64 [H] -> float64 [H].

    mx_act: the MXFP4 path's activations — x and the intermediate h are
    quantised to MXFP8 (formats.mx_e4m3) before their products."""
    w13 = np.asarray(w13_f32, dtype=np.float64)
    w2 = np.asarray(w2_f32, dtype=np.float64)
    inter = w13.shape[0] // 2
    if mx_act:
        x = mx_e4m3(x)[0]
    gu = w13 @ x
    g, u = gu[:inter], gu[inter:]
    h = silu(g) * u
    if mx_act:
        h = mx_e4m3(h)[0]
    return w2 @ h


class MoELayer:
    """Canonical-layout quantised layer, dequantised lazily per expert (cached).

    Fields mirror the layer description of the GPU library but are independent:
      router_w   bf16 bits [E][H];  router_bias fp32 [E] or None
      w13_codes  packed [E][2I][H/2], w13_scales bits [E][2I][H/G]
      w2_codes   packed [E][H][I/2],  w2_scales  bits [E][H][I/G]
      shared_*   same for the shared expert (groups = 1) or None
      shared_gate_w bf16 bits [H] or None
    The w13/w2 fields may be callables e -> (codes, scales) so that a test can
    quantise only the experts a token selects.  For NVFP4 every (codes, scales)
    pair carries a third element, the global scale (stacked: fp32 [E]).  The
    shared expert may use another format (shared_fmt; FMT_BF16: 1-tuples of
    bf16 bits, the pages' production choice for it).
    """

    def __init__(self, fmt, hidden, inter, num_experts, top_k, router_w, w13, w2,
                 router_bias=None, shared_w13=None, shared_w2=None, shared_gate_w=None, shared_fmt=None):
        self.fmt = fmt
        self.shared_fmt = fmt if shared_fmt is None else shared_fmt
        self.hidden = hidden
        self.inter = inter
        self.num_experts = num_experts
        self.top_k = top_k
        self.router_w = router_w
        self.router_bias = router_bias
        self._w13 = w13
        self._w2 = w2
        self.shared_w13 = shared_w13
        self.shared_w2 = shared_w2
        self.shared_gate_w = shared_gate_w
        self._cache = {}

    @property
    def has_shared(self):
        return self.shared_w13 is not None

    def _get(self, src, e):
        if callable(src):
            return tuple(src(e))
        return tuple(a[e] for a in src)

    def expert(self, e):
        if e not in self._cache:
            self._cache[e] = (dequant(self.fmt, *self._get(self._w13, e)),
                              dequant(self.fmt, *self._get(self._w2, e)))
        return self._cache[e]

    def shared(self):
        if "shared" not in self._cache:
            self._cache["shared"] = (dequant(self.shared_fmt, *self.shared_w13),
                                     dequant(self.shared_fmt, *self.shared_w2))
        return self._cache["shared"]


def moe_experts(layer, x_bits, ids, weights):
    """Experts + combine with caller-supplied routing (the P45 one-call shape).

    x_bits bf16 [T][H]; ids int [T][k]; weights [T][k].  Returns float64 [T][H].
    The shared expert (if present) is added with its sigmoid gate.
    """
    xs = np.atleast_2d(_as_x(x_bits))
    ids = np.atleast_2d(ids)
    weights = np.atleast_2d(np.asarray(weights, dtype=np.float64))
    out = np.zeros((xs.shape[0], layer.hidden), dtype=np.float64)
    for t in range(xs.shape[0]):
        x = xs[t]
        acc = np.zeros(layer.hidden, dtype=np.float64)
        mx = layer.fmt == FMT_MXFP4
        for j in range(ids.shape[1]):
            w13, w2 = layer.expert(int(ids[t, j]))
            acc += weights[t, j] * expert_ffn(w13, w2, x, mx)
        if layer.has_shared:
            sw13, sw2 = layer.shared()
            sig = shared_gate(layer.shared_gate_w, np.atleast_2d(x_bits)[t])
            acc += sig * expert_ffn(sw13, sw2, x, mx and layer.shared_fmt == FMT_MXFP4)
        out[t] = acc
    return out


def moe_forward(layer, x_bits, tokens=None):
    """Full layer: router -> softmax-all -> top-k -> renormalise -> experts -> combine.

    Returns (out float64 [T][H], ids int32 [T][k], weights float64 [T][k]).
    `tokens` optionally restricts the work to a subset of token indices (the
    returned arrays then cover only those rows, in the given order).
    """
    xb = np.atleast_2d(np.asarray(x_bits, dtype=np.uint16))
    rows = range(xb.shape[0]) if tokens is None else tokens
    outs, all_ids, all_w = [], [], []
    for t in rows:
        logits = router_logits(layer.router_w, xb[t], layer.router_bias)
        ids, w = route(logits, layer.top_k)
        outs.append(moe_experts(layer, xb[t:t + 1], ids[None], w[None])[0])
        all_ids.append(ids)
        all_w.append(w)
    return np.array(outs), np.array(all_ids, dtype=np.int32), np.array(all_w)


# --------------------------------------------------------------------------- metrics


def rel_l1(got, ref):
    """sum |got - ref| / sum |ref|: the mean relative error used for parity."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).sum()
    return float(np.abs(got - ref).sum() / den) if den > 0 else float(np.abs(got).sum())


def error_report(got, ref):
    """cosine, max_abs, rel_l2 and rel_l1 of got vs ref (the metrics the pages use)."""
    g = np.asarray(got, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    diff = g - r
    nr = np.linalg.norm(r)
    ng = np.linalg.norm(g)
    return {
        "max_abs": float(np.abs(diff).max()) if diff.size else 0.0,
        "max_ref": float(np.abs(r).max()) if r.size else 0.0,
        "rel_l2": float(np.linalg.norm(diff) / nr) if nr > 0 else float(np.linalg.norm(diff)),
        "rel_l1": rel_l1(g, r),
        "cosine": float(g @ r / (ng * nr)) if ng > 0 and nr > 0 else float(ng == nr),
    }
