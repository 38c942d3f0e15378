"""Pins of the oracle's MX path: MXFP4 weights (E2M1 + E8M0 per 32) and MXFP8
activations (E4M3 + E8M0 per 32), per the OCP Microscaling v1.0 conversion.

Against: hand-worked blocks (tests/golden/mxfp4_blocks.txt), the E8M0 closed
form, brute force over all codes, the shared-exponent invariant, torch's
float8_e4m3fn (an independent E4M3 rounding), idempotence on representable
inputs."""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import ops
from conftest import read_golden_lines


def _blocks():
    out, cur = [], None
    for line in read_golden_lines("mxfp4_blocks.txt"):
        if line.startswith("block"):
            _, name, sc = line.split()
            cur = {"name": name, "scale": int(sc.split("=")[1], 16)}
            out.append(cur)
        elif line.startswith("w:"):
            cur["w"] = np.array([float(v) for v in line[2:].split()], np.float32)
        elif line.startswith("codes:"):
            cur["codes"] = np.array([int(v, 16) for v in line[6:].split()], np.uint8)
    return out


@pytest.mark.parametrize("b", _blocks(), ids=lambda b: b["name"])
def test_mxfp4_golden(b):
    codes, sb = O.quantize_mxfp4(b["w"][None])
    assert int(sb[0, 0]) == b["scale"]
    assert np.array_equal(codes[0], b["codes"])


def test_e8m0_values():
    assert O.e8m0_value(0x7F) == 1.0 and O.e8m0_value(0x80) == 2.0 and O.e8m0_value(0x7C) == 0.125
    assert O.e8m0_value(0) == 2.0 ** -127 and np.isnan(O.e8m0_value(0xFF))
    b = np.arange(255)
    assert np.array_equal(O.e8m0_value(b), np.array([2.0 ** (int(v) - 127) for v in b]))


def test_mxfp4_brute_force_and_invariant():
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((32, 256)) * 0.02 * np.exp2(rng.integers(-6, 6, (32, 1)))).astype(np.float32)
    w[3, 32:64] = 0
    codes, sb = O.quantize_mxfp4(w)
    vals = O.e2m1_value(np.arange(16))
    for r in range(w.shape[0]):
        for blk in range(w.shape[1] // 32):
            seg = w[r, 32 * blk:32 * blk + 32].astype(np.float64)
            a = np.abs(seg).max()
            if a == 0:
                assert sb[r, blk] == 0 and not codes[r, 32 * blk:32 * blk + 32].any()
                continue
            X = int(sb[r, blk]) - 127
            assert 4 <= a / 2.0 ** X < 8  # floor(log2 absmax) - 2
            for i, v in enumerate(seg):
                q = min(max(v / 2.0 ** X, -6.0), 6.0)  # clamp, then nearest
                err = np.abs(vals - q)
                c = codes[r, 32 * blk + i]
                assert err[c] == err.min()
                if vals[c] == 0:
                    assert c == 0
                if len({vals[x] for x in range(16) if err[x] == err.min()}) > 1:
                    assert (c & 7) % 2 == 0
            # the block maximum lands on magnitude 4 or 6
            assert (codes[r, 32 * blk:32 * blk + 32] & 7).max() >= 6


def test_mxfp4_dequant_exact_and_sizes():
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((8, 128)) * 0.05).astype(np.float32)
    packed, sb = O.quantize(O.FMT_MXFP4, w)
    deq = O.dequant(O.FMT_MXFP4, packed, sb)
    want = O.e2m1_value(O.unpack_nibbles(packed)) * np.repeat(O.e8m0_value(sb), 32, axis=1)
    assert np.array_equal(deq.astype(np.float64), want)
    # 8192 x 2048: 8 MiB codes + 512 KiB E8M0 scales
    assert O.scales_bytes(O.FMT_MXFP4, 1, 8192, 2048) == 8192 * 64


def test_mxfp8_activation_quantisation_matches_torch():
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((16, 256)) * np.exp2(rng.integers(-10, 10, (16, 1)))).astype(np.float32)
    x[2, :32] = 0
    q, X = O.mx_e4m3(x)
    for r in range(16):
        for blk in range(8):
            seg = x[r, 32 * blk:32 * blk + 32].astype(np.float64)
            a = np.abs(seg).max()
            if a == 0:
                assert X[r, blk] == -127 and not q[r, 32 * blk:32 * blk + 32].any()
                continue
            assert X[r, blk] == np.floor(np.log2(a)) - 8
            s = 2.0 ** X[r, blk]
            t = torch.from_numpy(np.clip(seg / s, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn)
            assert np.array_equal(q[r, 32 * blk:32 * blk + 32], t.to(torch.float64).numpy() * s)


def test_mxfp8_idempotent_and_bounds():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((4, 128))
    q, X = O.mx_e4m3(x)
    q2, X2 = O.mx_e4m3(q)
    assert np.array_equal(q, q2) and np.array_equal(X, X2)
    # relative error of an element in E4M3's normal range, below the clamp, is at
    # most 2^-4 (3 mantissa bits); elements beyond 448 * 2^X clamp to +-448 * 2^X
    s = np.repeat(np.exp2(X.astype(np.float64)), 32, axis=-1)
    r = np.abs(x) / s
    normal = (r >= 2.0 ** -6) & (r <= 448)
    assert np.all(np.abs(q - x)[normal] <= np.abs(x)[normal] * 2.0 ** -4)
    sat = r > 448
    assert sat.any() and np.array_equal(q[sat], np.sign(x[sat]) * 448 * s[sat])


def test_mx_expert_quantises_x_and_h():
    """The MX expert equals the plain SwiGLU on MXFP8-quantised x and h."""
    rng = np.random.default_rng(16)
    w13 = O.dequant(O.FMT_MXFP4, *O.quantize(O.FMT_MXFP4, (rng.standard_normal((64, 64)) * 0.1).astype(np.float32)))
    w2 = O.dequant(O.FMT_MXFP4, *O.quantize(O.FMT_MXFP4, (rng.standard_normal((64, 32)) * 0.1).astype(np.float32)))
    x = rng.standard_normal(64)
    got = ops.expert_ffn(w13, w2, x, mx_act=True)
    xq = O.mx_e4m3(x)[0]
    gu = w13.astype(np.float64) @ xq
    h = gu[:32] / (1 + np.exp(-gu[:32])) * gu[32:]
    want = w2.astype(np.float64) @ O.mx_e4m3(h)[0]
    assert np.array_equal(got, want)
    assert not np.allclose(got, ops.expert_ffn(w13, w2, x), rtol=1e-6)


def test_mxfp8_given_exponent():
    """mx_e4m3 with the shared exponents given: the computed ones reproduce the
    default result; one more (a coarser block scale) matches torch's E4M3
    rounding of v / 2^(X+1), clamped to +-448."""
    rng = np.random.default_rng(17)
    x = (rng.standard_normal((6, 128)) * np.exp2(rng.integers(-6, 6, (6, 1)))).astype(np.float64)
    q, X = O.mx_e4m3(x)
    q1, X1 = O.mx_e4m3(x, X)
    assert np.array_equal(q, q1) and np.array_equal(X, X1)
    q2, X2 = O.mx_e4m3(x, X + 1)
    assert np.array_equal(X2, X + 1)
    s = np.repeat(np.exp2((X + 1).astype(np.float64)), 32, axis=-1)
    t = torch.from_numpy(np.clip(x / s, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64)
    assert np.array_equal(q2, t.numpy() * s)
