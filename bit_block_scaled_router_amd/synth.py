"""Seeded synthetic inputs for the W4A16 MoE layer and dense GEMV workloads.

This module only draws random numbers; it holds none of the layer's arithmetic
(no quantisation, routing or matrix products), so that both the GPU path and the
CPU oracle can be fed from it without sharing any of the method's code.

Recipe (NumPy PCG64 streams keyed by [seed, stream, ...]):
  stream 0  activations x: fp32 N(0, 1) rounded to bf16, one row per (token, attempt)
  stream 1  router weight: fp32 N(0, 0.02) rounded to bf16, [E][H]
  stream 2  routed expert e, W13 (gate rows then up rows): fp32 N(0, 0.02), [2I][H]
  stream 3  routed expert e, W2: fp32 N(0, 0.02), [H][I]
  stream 4  shared expert W13, stream 5 shared expert W2 (same distributions)
  stream 6  shared-expert gate weight: fp32 N(0, 0.02) rounded to bf16, [H]
  stream 7  Zipf rank permutation of the experts (batched workload only)
  stream 9  dense GEMV weight [N][K]: fp32 N(0, 0.02)
Per-expert streams let a checker regenerate only the experts it needs.

The shapes follow the Qwen 3.6 35B-A3B configuration block of the lynn-engine
tutorials index (hidden 2048, 256 experts, 8 per token, a sigmoid-gated shared
expert) with an expert intermediate of 512 (lynn-engine README, status note P28:
"[top_k, 512]" gate/up output), and the 8192x2048 projection of the "Lynn
Engine" article's stage P1.  The pages' real checkpoints and activations are not
available; these draws stand in for them.
"""

from dataclasses import dataclass

import numpy as np

SIGMA_W = 0.02  # weight std (router, shared gate, experts, dense)


def _rng(*key):
    return np.random.default_rng([int(k) for k in key])


def f32_to_bf16_bits(a):
    """fp32 -> bf16 bits, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def normal_f32(shape, std, *key):
    return (_rng(*key).standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


# --------------------------------------------------------------------------- workloads


@dataclass(frozen=True)
class MoEShape:
    name: str
    hidden: int
    inter: int
    num_experts: int
    top_k: int
    shared_inter: int = 0  # 0 = no shared expert
    tokens: int = 1
    zipf_s: float = 0.0  # > 0: router logit bias -s*ln(rank)
    seed: int = 0
    fmt: str = "e2m1"  # weight format of the experts: "e2m1", "int4", "nvfp4" or "mxfp4"
    shared_fmt: str = ""  # shared expert's format ("" = fmt; "bf16" = unquantised)

    @property
    def has_shared(self):
        return self.shared_inter > 0


@dataclass(frozen=True)
class GemvShape:
    name: str
    n: int
    k: int
    fmt: str  # "e2m1", "int4" or "nvfp4"
    seed: int = 0


TINY_MOE = MoEShape("tiny-moe-h256-e8-k2-i128", 256, 128, 8, 2, 0, 1, 0.0, 0)
QWEN_MOE_T1 = MoEShape("qwen3.6-35b-a3b-moe-decode-t1", 2048, 512, 256, 8, 512, 1, 0.0, 0)
GEMV_E2M1 = GemvShape("gemv-e2m1-8192x2048", 8192, 2048, "e2m1", 0)
GEMV_INT4 = GemvShape("gemv-int4g128-8192x2048", 8192, 2048, "int4", 0)
GEMV_NVFP4 = GemvShape("gemv-nvfp4-8192x2048", 8192, 2048, "nvfp4", 0)
# lm_head-sized projection (vocabulary 248,320 x hidden 2048): 318 MB packed E2M1
GEMV_LMHEAD = GemvShape("gemv-e2m1-lmhead-248320x2048", 248320, 2048, "e2m1", 0)
QWEN_MOE_T32 = MoEShape("qwen3.6-35b-a3b-moe-batch32-zipf1.1", 2048, 512, 256, 8, 512, 32, 1.1, 0)
QWEN_MOE_T1_NVFP4 = MoEShape("qwen3.6-35b-a3b-moe-decode-t1-nvfp4", 2048, 512, 256, 8, 512, 1, 0.0, 0, "nvfp4")
QWEN_MOE_T32_NVFP4 = MoEShape("qwen3.6-35b-a3b-moe-batch32-zipf1.1-nvfp4", 2048, 512, 256, 8, 512, 32, 1.1, 0, "nvfp4")
# bf16 shared expert (the pages' production choice for it), E2M1 routed experts
QWEN_MOE_T1_BF16SH = MoEShape("qwen3.6-35b-a3b-moe-decode-t1-bf16shared", 2048, 512, 256, 8, 512, 1, 0.0, 0, "e2m1",
                              "bf16")
TINY_MOE_BF16SH = MoEShape("tiny-moe-h256-e8-k2-i128-bf16shared", 256, 128, 8, 2, 128, 1, 0.0, 0, "e2m1", "bf16")
QWEN_MOE_T32_INT4 = MoEShape("qwen3.6-35b-a3b-moe-batch32-zipf1.1-int4", 2048, 512, 256, 8, 512, 32, 1.1, 0, "int4")
QWEN_MOE_T32_BF16SH = MoEShape("qwen3.6-35b-a3b-moe-batch32-zipf1.1-bf16shared", 2048, 512, 256, 8, 512, 32, 1.1, 0,
                               "e2m1", "bf16")
# MXFP4 experts with MXFP8 activations (the scaled FP4 MFMA path)
TINY_MOE_MX = MoEShape("tiny-moe-h256-e8-k2-i128-mxfp4", 256, 128, 8, 2, 128, 1, 0.0, 0, "mxfp4")
QWEN_MOE_T1_MX = MoEShape("qwen3.6-35b-a3b-moe-decode-t1-mxfp4", 2048, 512, 256, 8, 512, 1, 0.0, 0, "mxfp4")
QWEN_MOE_T32_MX = MoEShape("qwen3.6-35b-a3b-moe-batch32-zipf1.1-mxfp4", 2048, 512, 256, 8, 512, 32, 1.1, 0, "mxfp4")
# prefill-sized batches: 2048 tokens x top-8 = 16,384 (token, slot) pairs, ~64 per
# expert (no popularity bias), the MFMA-bound regime of the grouped path
QWEN_MOE_PREFILL = MoEShape("qwen3.6-35b-a3b-moe-prefill2048", 2048, 512, 256, 8, 512, 2048, 0.0, 0)
QWEN_MOE_PREFILL_MX = MoEShape("qwen3.6-35b-a3b-moe-prefill2048-mxfp4", 2048, 512, 256, 8, 512, 2048, 0.0, 0, "mxfp4")
QWEN_MOE_PREFILL_NVFP4 = MoEShape("qwen3.6-35b-a3b-moe-prefill2048-nvfp4", 2048, 512, 256, 8, 512, 2048, 0.0, 0,
                                  "nvfp4")
QWEN_MOE_PREFILL_BF16SH = MoEShape("qwen3.6-35b-a3b-moe-prefill2048-bf16shared", 2048, 512, 256, 8, 512, 2048, 0.0, 0,
                                   "e2m1", "bf16")


# --------------------------------------------------------------------------- draws


def x_row(seed, hidden, token, attempt=0):
    """One activation row (bf16 bits [H]) for a token; `attempt` > 0 redraws it."""
    return f32_to_bf16_bits(normal_f32((hidden,), 1.0, seed, 0, token, attempt))


def router_weight(shape: MoEShape):
    return f32_to_bf16_bits(normal_f32((shape.num_experts, shape.hidden), SIGMA_W, shape.seed, 1))


def router_bias(shape: MoEShape):
    """Zipf-style popularity bias: -s * ln(rank), rank = 1 + a seeded permutation."""
    if shape.zipf_s <= 0:
        return None
    rank = 1 + _rng(shape.seed, 7).permutation(shape.num_experts)
    return (-shape.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)


def expert_w13(shape: MoEShape, e):
    return normal_f32((2 * shape.inter, shape.hidden), SIGMA_W, shape.seed, 2, e)


def expert_w2(shape: MoEShape, e):
    return normal_f32((shape.hidden, shape.inter), SIGMA_W, shape.seed, 3, e)


def shared_w13(shape: MoEShape):
    return normal_f32((2 * shape.shared_inter, shape.hidden), SIGMA_W, shape.seed, 4)


def shared_w2(shape: MoEShape):
    return normal_f32((shape.hidden, shape.shared_inter), SIGMA_W, shape.seed, 5)


def shared_gate_weight(shape: MoEShape):
    return f32_to_bf16_bits(normal_f32((shape.hidden,), SIGMA_W, shape.seed, 6))


def dense_weight(shape: GemvShape):
    return normal_f32((shape.n, shape.k), SIGMA_W, shape.seed, 9)


def dense_x(shape: GemvShape, attempt=0):
    return x_row(shape.seed, shape.k, 0, attempt)
