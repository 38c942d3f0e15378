"""Pins for the oracle's format layer (codes, scales, quantiser, packing, sizes).

Every check compares the oracle with something it does not compute itself: typed
tables from the format definitions, hand-worked blocks, exhaustive search, library
conversions (torch's fp32->bf16, numpy's fp16) and invariants that any correct
quantiser must satisfy.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from conftest import read_golden_blocks, read_golden_lines


# ---------------------------------------------------------------- code tables


def test_e2m1_closed_form_matches_typed_table():
    rows = [ln.split() for ln in read_golden_lines("e2m1_table.txt")]
    assert len(rows) == 16
    for code_s, val_s in rows:
        code = int(code_s, 16)
        got = float(oracle.e2m1_value(code))
        want = float(val_s)
        assert got == want and np.signbit(got) == np.signbit(want), (code, got, want)


def test_int4_matches_twos_complement_table():
    rows = [ln.split() for ln in read_golden_lines("int4_table.txt")]
    assert len(rows) == 16
    for code_s, val_s in rows:
        assert float(oracle.int4_value(int(code_s, 16))) == float(val_s)


# ---------------------------------------------------------------- bf16


def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x3E80], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 3.3895313892515355e38, 2.0 ** -133, 0.25]
    got = oracle.bf16_bits_to_f64(bits)
    for g, w in zip(got, want):
        assert g == w and np.signbit(g) == np.signbit(w)


def test_bf16_round_ties_to_even_by_hand():
    # spacing of bf16 near 1 is 2**-7
    cases = {
        1.0 + 2.0 ** -8: 0x3F80,        # tie, lower neighbour even -> 1.0
        1.0 + 3 * 2.0 ** -8: 0x3F82,    # tie, upper neighbour even -> 1 + 2**-6
        1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,  # just above the tie -> up
        -(1.0 + 2.0 ** -8): 0xBF80,
        0.0: 0x0000,
    }
    for v, b in cases.items():
        assert int(oracle.f64_to_bf16_bits(np.array([v]))[0]) == b, v


def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(123)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
    ])
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f64_to_bf16_bits(v.astype(np.float64))
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- hand-worked blocks


@pytest.mark.parametrize("block", read_golden_blocks("e2m1_blocks.txt"), ids=lambda b: b[0])
def test_e2m1_quantize_golden_blocks(block):
    name, scale_bits, w, codes = block
    w = np.array(w, dtype=np.float32)[None, :]
    c, s = oracle.quantize_e2m1(w)
    assert int(s.view(np.uint16)[0, 0]) == scale_bits
    assert c[0].tolist() == codes


def test_int4_quantize_golden_block():
    (name, scale_bits, w, codes), = read_golden_blocks("int4_blocks.txt")
    full = np.zeros((1, 128), dtype=np.float32)
    full[0, :16] = w
    c, s = oracle.quantize_int4(full)
    assert int(s.view(np.uint16)[0, 0]) == scale_bits
    assert c[0, :16].tolist() == codes
    assert not c[0, 16:].any()


# ---------------------------------------------------------------- exhaustive search


def _brute_force_codes(fmt, w32, scale_f16):
    """Per element, try all 16 codes and keep the nearest to w/s (fp32 division).

    Ties between two codes go to the even code; negative zero is never chosen
    (code 8 decodes to -0.0 and would tie with code 0)."""
    group = F.group_size(fmt)
    values = F._decode(fmt, np.arange(16))
    out = np.zeros(w32.shape, dtype=np.uint8)
    s32 = scale_f16.astype(np.float32)
    for i in range(w32.shape[0]):
        for j in range(w32.shape[1]):
            s = s32[i, j // group]
            if s == 0:
                continue
            r = np.float32(w32[i, j]) / s
            best = None
            for c in range(16):
                if fmt == F.FMT_E2M1 and c == 8:
                    continue
                d = abs(float(r) - float(values[c]))
                key = (d, 0 if c % 2 == 0 else 1)
                if fmt == F.FMT_INT4:
                    # int4 rounds half to even on the integer value, which is the
                    # even code too (two's complement keeps the parity)
                    key = (d, int(values[c]) % 2)
                if best is None or key < best[0]:
                    best = (key, c)
            out[i, j] = best[1]
    return out


def _near_midpoint_blocks(fmt, rng, nblocks):
    """Blocks whose ratios sit on, and one fp32 ulp around, every midpoint."""
    group = F.group_size(fmt)
    if fmt == F.FMT_E2M1:
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
        top = 6.0
    else:
        mids = np.arange(-7.5, 7.5, 1.0)
        top = 7.0
    w = np.zeros((nblocks, group), dtype=np.float32)
    for b in range(nblocks):
        s = np.float32(2.0 ** rng.integers(-8, 3))
        vals = rng.choice(mids, group - 1) * rng.choice([-1, 1], group - 1)
        vals = vals.astype(np.float32) * s
        nudge = rng.integers(-1, 2, group - 1)
        vals = np.nextafter(vals, np.where(nudge > 0, np.inf, -np.inf).astype(np.float32)) \
            * (nudge != 0) + vals * (nudge == 0)
        w[b, 0] = top * s  # absmax -> scale exactly s
        w[b, 1:] = vals
    return w


@pytest.mark.parametrize("fmt", [F.FMT_E2M1, F.FMT_INT4])
def test_quantizer_equals_exhaustive_search(fmt):
    rng = np.random.default_rng(7)
    group = F.group_size(fmt)
    w = np.concatenate([
        _near_midpoint_blocks(fmt, rng, 12).reshape(-1, group),
        (rng.standard_normal((6, group)) * 0.02).astype(np.float32),
        (rng.standard_normal((2, group)) * 1e-6).astype(np.float32),  # subnormal scales
    ]).reshape(4, -1)
    q = oracle.quantize_e2m1 if fmt == F.FMT_E2M1 else oracle.quantize_int4
    codes, s = q(w)
    assert np.array_equal(codes, _brute_force_codes(fmt, w, s))


# ---------------------------------------------------------------- invariants


@pytest.mark.parametrize("fmt", [F.FMT_E2M1, F.FMT_INT4])
def test_quantizer_invariants(fmt):
    rng = np.random.default_rng(11)
    group = F.group_size(fmt)
    qmax = 6.0 if fmt == F.FMT_E2M1 else 7.0
    w = (rng.standard_normal((64, 8 * group)) * 0.02).astype(np.float32)
    w[3, :group] = 0.0  # a zero block
    q = oracle.quantize_e2m1 if fmt == F.FMT_E2M1 else oracle.quantize_int4
    codes, s = q(w)
    vals = F._decode(fmt, codes)
    s32 = s.astype(np.float64)
    a = np.abs(w.reshape(64, 8, group)).max(axis=2).astype(np.float64)
    # the scale is absmax / qmax up to fp16 rounding (relative 2**-11 for normal values)
    normal = s32 >= 2.0 ** -14
    assert np.all(np.abs(s32 - a / qmax)[normal] <= (a / qmax)[normal] * 2.0 ** -11)
    # every non-zero block holds a code of maximum magnitude
    blk = np.abs(vals.reshape(64, 8, group)).max(axis=2)
    assert np.all(blk[(a > 0) & normal] == qmax)
    assert np.all(blk[a == 0] == 0) and np.all(s32[a == 0] == 0)
    # error within half a grid step of the code value (plus fp32 division rounding)
    deq = F.dequant(fmt, F.pack_nibbles(codes), s.view(np.uint16)).astype(np.float64)
    r = np.abs(w.astype(np.float64)) / np.repeat(np.where(s32 > 0, s32, 1), group, axis=1)
    if fmt == F.FMT_E2M1:
        half = np.where(r < 2, 0.25, np.where(r < 4, 0.5, 1.0))
    else:
        half = np.full_like(r, 0.5)
    bound = (half + r * 2.0 ** -23) * np.repeat(s32, group, axis=1)
    assert np.all(np.abs(deq - w) <= bound)
    # negative zero and (for normal int4 scales) -8 are never emitted
    if fmt == F.FMT_E2M1:
        assert not np.any(codes == 8)
    else:
        assert not np.any(codes[np.repeat(normal, group, axis=1)] == 8)


@pytest.mark.parametrize("fmt", [F.FMT_E2M1, F.FMT_INT4])
def test_quantizer_power_of_two_covariance(fmt):
    """Scaling w by 2**m scales every fp16 scale by 2**m and leaves the codes alone."""
    rng = np.random.default_rng(5)
    group = F.group_size(fmt)
    w = (rng.standard_normal((16, 4 * group)) * 0.02).astype(np.float32)
    q = oracle.quantize_e2m1 if fmt == F.FMT_E2M1 else oracle.quantize_int4
    c0, s0 = q(w)
    for m in (-3, 1, 4):
        c1, s1 = q(w * np.float32(2.0 ** m))
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1.astype(np.float64), s0.astype(np.float64) * 2.0 ** m)


def test_quantizer_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.quantize_e2m1(np.full((1, 16), np.inf, dtype=np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_e2m1(np.full((1, 16), 4e5, dtype=np.float32))  # 4e5/6 > fp16 max
    with pytest.raises(ValueError):
        oracle.quantize_int4(np.zeros((1, 64), dtype=np.float32))  # K not a multiple of 128


# ---------------------------------------------------------------- packing and sizes


def test_pack_nibble_order_by_hand():
    # element 0 -> low nibble, element 1 -> high nibble
    assert oracle.pack_nibbles(np.array([[0x1, 0x2, 0xF, 0x0]], dtype=np.uint8)).tolist() == [[0x21, 0x0F]]


def test_pack_unpack_identity_all_bytes():
    b = np.arange(256, dtype=np.uint8)[None, :]
    assert np.array_equal(oracle.pack_nibbles(oracle.unpack_nibbles(b)), b)
    nib = oracle.unpack_nibbles(b)
    assert np.array_equal(nib[0, 0::2], np.arange(256) & 0xF)
    assert np.array_equal(nib[0, 1::2], np.arange(256) >> 4)


def test_packed_size_matches_stage_p1():
    (line,) = read_golden_lines("layout_sizes.txt")
    n, k, bf16_mib, packed_mib, ratio = line.split()
    n, k = int(n), int(k)
    total = oracle.codes_bytes(F.FMT_E2M1, 1, n, k) + oracle.scales_bytes(F.FMT_E2M1, 1, n, k)
    assert total == 10_485_760
    assert f"{total / 2**20:.2f}" == packed_mib
    assert f"{n * k * 2 / 2**20:.2f}" == bf16_mib
    assert f"{n * k * 2 / total:.2f}" == ratio


# ---------------------------------------------------------------- dequant


def test_dequant_golden_blocks_and_exactness():
    table = {int(c, 16): float(v) for c, v in (ln.split() for ln in read_golden_lines("e2m1_table.txt"))}
    for name, scale_bits, w, codes in read_golden_blocks("e2m1_blocks.txt"):
        packed = oracle.pack_nibbles(np.array([codes], dtype=np.uint8))
        sb = np.array([[scale_bits]], dtype=np.uint16)
        got = oracle.dequant(F.FMT_E2M1, packed, sb)
        s = float(np.array([scale_bits], dtype=np.uint16).view(np.float16)[0])
        assert got[0].tolist() == [table[c] * s for c in codes]


def test_dequant_exact_over_all_codes_and_extreme_scales():
    # every code against the largest, smallest normal and smallest subnormal fp16 scale
    codes = np.tile(np.arange(16, dtype=np.uint8), 3)[None, :]
    scales = np.array([[0x7BFF, 0x0400, 0x0001]], dtype=np.uint16)  # 65504, 2**-14, 2**-24
    got = oracle.dequant(F.FMT_E2M1, oracle.pack_nibbles(codes), scales).astype(np.float64)
    vals = oracle.e2m1_value(np.arange(16))
    want = np.concatenate([vals * 65504.0, vals * 2.0 ** -14, vals * 2.0 ** -24])
    assert np.array_equal(got[0], want)
