"""The seeded input generator: determinism, distributions, bf16 rounding."""

import numpy as np
import torch

from bit_block_scaled_router_amd import synth


def test_same_seed_same_bytes():
    s = synth.QWEN_MOE_T1
    assert np.array_equal(synth.expert_w13(s, 17), synth.expert_w13(s, 17))
    assert not np.array_equal(synth.expert_w13(s, 17), synth.expert_w13(s, 18))
    assert np.array_equal(synth.x_row(0, 2048, 3), synth.x_row(0, 2048, 3))
    assert not np.array_equal(synth.x_row(0, 2048, 3, 0), synth.x_row(0, 2048, 3, 1))


def test_bf16_rounding_matches_torch():
    v = np.random.default_rng(0).standard_normal(50000).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(v), want)


def test_distributions_and_shapes():
    s = synth.QWEN_MOE_T1
    w = synth.expert_w13(s, 0)
    assert w.shape == (1024, 2048) and w.dtype == np.float32
    assert abs(w.std() - 0.02) < 1e-3 and abs(w.mean()) < 1e-3
    assert synth.expert_w2(s, 0).shape == (2048, 512)
    assert synth.router_weight(s).shape == (256, 2048)
    assert synth.router_bias(s) is None


def test_zipf_bias_is_minus_s_log_rank():
    b = synth.router_bias(synth.QWEN_MOE_T32).astype(np.float64)
    ranks = np.sort(np.exp(-b / 1.1))
    np.testing.assert_allclose(ranks, np.arange(1, 257), rtol=1e-5)
