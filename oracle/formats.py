"""Oracle: 4-bit weight formats (codes, scales, quantize, pack, dequant).

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests, the smoke
check and the benchmark's CPU baseline, never by the product path.

Everything here is written from the definitions, in float32/float64 NumPy:

* E2M1 (4-bit float: 1 sign, 2 exponent, 1 mantissa bit, bias 1, no inf/NaN) as
  defined by the OCP Microscaling (MX) v1.0 specification's FP4 element type.  The
  pages only name the format: "Lynn Engine" article, "Native NVFP4 quantization
  support" (W4A16: 4-bit weights, bf16 activations) and "Kernel optimisation
  history", stage P1 (packed E2M1 plus an FP16 scale, read by the matvec directly).
* One FP16 scale per 16 consecutive K elements ("Lynn Engine" article, stage P1;
  the 8192x2048 projection shrinking from 32.00 MiB to 10.00 MiB fixes both the
  block of 16 and the 2-byte scale).
* Signed int4 with one FP16 scale per group of 128 along K: "cuda_inf" article,
  section "2. INT4 weight quantization".
* MXFP4 (OCP Microscaling v1.0, the vendor format the README notes P17/P54 and
  R5-B bridge to, "e8m0/group32"): E2M1 codes with one E8M0 scale (a power of
  two, 2^(byte - 127); byte 0xFF is NaN) per 32 K elements.  Shared exponent and
  element rounding follow the MX specification's conversion: X =
  floor(log2(absmax)) - emax_elem (emax_elem = 2 for E2M1, 8 for E4M3), elements
  round to nearest even after division by 2^X and clamp to the largest normal.
  The MX path computes with MXFP8 activations (E4M3 elements, E8M0 per 32): the
  layer input and the SwiGLU intermediate are quantised that way before each
  scaled MFMA, so it is a W4A8 variant with its own parity reference.
* NVFP4 proper: E2M1 codes, one unsigned E4M3 (UE4M3) scale per 16 K elements and
  one fp32 global scale per matrix.  The lynn-engine README names this variant
  (status notes P17/P54 "per-16/e4m3" scales, R5-C0 "UE4M3" block-16 scales,
  P29 a down projection taking "packed/scale/global"); E4M3 is the OCP 8-bit
  float (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
  infinities, S.1111.111 = NaN, largest finite 448).

Readings taken where the pages are silent (each one is also listed in the design
notes of the repository):
  - scale = RNE_fp16(fp32(absmax) / 6) for E2M1 and / 7 for int4; the division is
    an IEEE fp32 division and the fp32 quotient is then rounded to fp16;
  - element code = nearest representable value to fp32(w) / fp32(scale) (IEEE fp32
    division), ties to the even code, saturating; int4 rounds half to even and
    clips to [-8, 7];
  - an all-zero block gets scale 0 and all codes 0; a negative value that rounds
    to magnitude zero is encoded as +0 (code 0x0), so code 0x8 is never emitted;
  - a block whose fp16 scale would be infinite, or any non-finite input, is an
    error (ValueError here);
  - nibble order: element 2j in the low nibble, 2j+1 in the high nibble of byte j;
  - int4 nibbles are two's complement.
  - NVFP4 (the pages give no recipe; this is the common one, which puts the
    largest block scale at the top of the E4M3 range): g = fp32(absmax(W)) /
    fp32(6 * 448) per matrix; block scale s = UE4M3 round-to-nearest-even of
    fp32(fp32(absmax_block) / 6) / g, saturating at 448; element code = nearest
    E2M1 value to fp32(w) / fp32(value(s) * g) as for the FP16-scale format; an
    all-zero matrix gets g = 0 with zero scales and codes; a block whose scale
    rounds to zero gets zero codes.  Value of an element: code * s * g.

Parity pins (tests/test_oracle_formats.py): the E2M1 closed form against a literal
table typed from the OCP MX definition; int4 against two's complement; the
quantizer against exhaustive search over all 16 codes and its invariants (every
non-zero block with a normal scale holds a code of maximum magnitude, the error
bound of half a grid step, scaling covariance under powers of two); hand-worked
golden blocks; the 10.00 MiB / 3.20x size from stage P1; pack/unpack identity over
all 256 byte values.
"""

import numpy as np

FMT_E2M1 = 1  # E2M1 codes, FP16 scale per 16 K elements
FMT_INT4 = 2  # two's-complement int4 codes, FP16 scale per 128 K elements
FMT_NVFP4 = 3  # E2M1 codes, UE4M3 scale per 16 K elements, fp32 scale per matrix
FMT_BF16 = 4  # unquantised bf16 weights (the shared expert's production format in the pages)
FMT_MXFP4 = 5  # E2M1 codes, E8M0 scale per 32 K elements (OCP MX); activations MXFP8
MX_BLOCK = 32

E2M1_GROUP = 16
INT4_GROUP = 128

_GROUP = {FMT_E2M1: E2M1_GROUP, FMT_INT4: INT4_GROUP, FMT_NVFP4: E2M1_GROUP, FMT_MXFP4: MX_BLOCK}
_SCALE_BYTES = {FMT_E2M1: 2, FMT_INT4: 2, FMT_NVFP4: 1, FMT_MXFP4: 1}

E4M3_MAX = 448.0


def group_size(fmt):
    if fmt not in _GROUP:
        raise ValueError(f"unknown format {fmt}")
    return _GROUP[fmt]


# --------------------------------------------------------------------------- bf16


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v):
    """float64 -> bf16 bits, rounding to nearest, ties to even, in one step.

    bf16 keeps 8 significant bits and the fp32 exponent range (normal values down
    to 2**-126, subnormal spacing 2**-133).  Inputs here are finite.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite value")
    m, e = np.frexp(v)  # v = m * 2**e, 0.5 <= |m| < 1
    # spacing of bf16 values near v: 2**(e-8) for normal values, 2**-133 below.
    step_exp = np.maximum(e - 8, -133)
    q = np.rint(np.ldexp(v, -step_exp))  # round half to even
    r = np.ldexp(q, step_exp)
    if np.any(np.abs(r) > 3.3895313892515355e38):
        raise ValueError("bf16 overflow")
    # r is exactly representable in bf16, hence in fp32 with a zero low half
    u = r.astype(np.float32).view(np.uint32)
    assert np.all((u & np.uint32(0xFFFF)) == 0)
    return (u >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------- codes


def e2m1_value(code):
    """Decode an E2M1 code (0..15) from its bit fields.

    sign = bit 3, exponent = bits 2..1 (bias 1), mantissa = bit 0.  Exponent 0 is
    subnormal: magnitude = mantissa * 0.5.  Otherwise 2**(exponent-1) * (1 + m/2).
    Code 8 is negative zero.
    """
    c = np.asarray(code, dtype=np.int64)
    sign = (c >> 3) & 1
    exp = (c >> 1) & 3
    man = c & 1
    mag = np.where(exp == 0, man * 0.5, np.ldexp(1.0 + man * 0.5, exp - 1))
    return np.where(sign == 1, -mag, mag).astype(np.float64)


def int4_value(code):
    """Decode a two's-complement 4-bit code (0..15) to an integer in [-8, 7]."""
    c = np.asarray(code, dtype=np.int64)
    return (c - 16 * (c >= 8)).astype(np.float64)


def e4m3_value(byte):
    """OCP E4M3 byte -> float64 (closed form): sign s, exponent e (4 bits, bias 7),
    mantissa m (3 bits); e = 0 is subnormal m/8 * 2**-6; S.1111.111 is NaN."""
    b = np.asarray(byte, dtype=np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    return np.where((b & 0x7F) == 0x7F, np.nan, sign * mag)


# the 127 finite non-negative E4M3 values, in code order 0x00..0x7E (increasing)
_UE4M3 = e4m3_value(np.arange(0x7F))


def f32_to_ue4m3(v):
    """Non-negative fp32 values -> UE4M3 bytes: nearest representable value, ties
    to the even code (round to nearest even), saturating at 448."""
    return _ue4m3_rne(np.asarray(v, dtype=np.float32).astype(np.float64))


def _ue4m3_rne(x):
    """Non-negative float64 values -> UE4M3 bytes, round to nearest even (no
    intermediate rounding), saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(x < 0) or not np.all(np.isfinite(x)):
        raise ValueError("UE4M3 input must be finite and non-negative")
    x = np.minimum(x, E4M3_MAX)
    i = np.clip(np.searchsorted(_UE4M3, x, side="left"), 1, 0x7E)  # _UE4M3[i-1] < x <= _UE4M3[i]
    lo, hi = _UE4M3[i - 1], _UE4M3[i]
    dl, dh = x - lo, hi - x  # exact in float64
    pick_hi = (dh < dl) | ((dh == dl) & (i % 2 == 0))
    return np.where(pick_hi, i, i - 1).astype(np.uint8)


def e8m0_value(byte):
    """OCP E8M0 scale byte -> float64: 2^(byte - 127); 0xFF is NaN."""
    b = np.asarray(byte, dtype=np.int64)
    return np.where(b == 0xFF, np.nan, np.exp2(b.astype(np.float64) - 127.0))


def _mx_exponent(amax, emax_elem):
    """Shared MX exponent of a block: floor(log2(amax)) - emax_elem, amax > 0
    (exact: frexp gives amax = f 2^e with f in [0.5, 1), floor(log2) = e - 1),
    limited to the E8M0 range [-127, 127]."""
    _, e = np.frexp(np.asarray(amax, dtype=np.float64))
    return np.clip(e.astype(np.int64) - 1 - emax_elem, -127, 127)


def quantize_mxfp4(w):
    """fp32 weights [N][K] -> (codes [N][K] uint8 0..15, E8M0 scale bytes [N][K/32]).

    Per 32-element block (OCP MX v1.0 conversion): X = floor(log2(absmax)) - 2;
    element = nearest E2M1 value to w / 2^X (exact division), ties to the even
    code, saturating at 6; an all-zero block gets X = -127 (byte 0) and zero codes;
    -0 is never emitted."""
    w32 = _check_input(w, MX_BLOCK)
    n, k = w32.shape
    blk = np.abs(w32.reshape(n, k // MX_BLOCK, MX_BLOCK)).max(axis=2).astype(np.float64)
    X = np.where(blk > 0, _mx_exponent(np.where(blk > 0, blk, 1.0), 2), -127)
    r = w32.astype(np.float64) / np.exp2(np.repeat(X, MX_BLOCK, axis=1).astype(np.float64))
    mag = _nearest_e2m1_magnitude_code(np.abs(r))
    neg = (r < 0) & (mag != 0)
    codes = (mag + 8 * neg).astype(np.uint8)
    return codes, (X + 127).astype(np.uint8)


def mx_e4m3(v, X=None):
    """MXFP8 (E4M3 elements, E8M0 per 32) quantisation of activations along the
    last axis, returned dequantised (float64, exact) with the scale exponents.

    Per block: X = floor(log2(absmax)) - 8; q = E4M3 round-to-nearest-even of
    clamp(v / 2^X, +-448) (sign of zero kept); value = q * 2^X.  A zero block has
    X = -127 and zero values.  X (int array, one per block) may be given to
    quantise under another shared exponent (the other side of an absmax that
    sits on a power of two)."""
    a = np.asarray(v, dtype=np.float64)
    shp = a.shape
    if shp[-1] % MX_BLOCK:
        raise ValueError("length not a multiple of 32")
    b = a.reshape(shp[:-1] + (shp[-1] // MX_BLOCK, MX_BLOCK))
    amax = np.abs(b).max(axis=-1)
    if X is None:
        X = np.where(amax > 0, _mx_exponent(np.where(amax > 0, amax, 1.0), 8), -127)
    X = np.asarray(X, dtype=np.int64)
    r = np.clip(b / np.exp2(X.astype(np.float64))[..., None], -E4M3_MAX, E4M3_MAX)
    q = e4m3_value(_ue4m3_rne(np.abs(r))) * np.where(np.signbit(r), -1.0, 1.0)
    return (q * np.exp2(X.astype(np.float64))[..., None]).reshape(shp), X


def _decode(fmt, code):
    if fmt in (FMT_E2M1, FMT_NVFP4, FMT_MXFP4):
        return e2m1_value(code)
    if fmt == FMT_INT4:
        return int4_value(code)
    raise ValueError(f"unknown format {fmt}")


# E2M1 magnitudes in code order 0..7 (from the closed form).
_E2M1_MAG = e2m1_value(np.arange(8))


# --------------------------------------------------------------------------- quantize


def _block_scales(w32, group, qmax):
    """fp16 scale per block: RNE_fp16(fp32 absmax / fp32 qmax)."""
    n, k = w32.shape
    a = np.abs(w32.reshape(n, k // group, group)).max(axis=2)  # exact in fp32
    q = a / np.float32(qmax)  # IEEE fp32 division
    with np.errstate(over="ignore"):
        s = q.astype(np.float16)  # numpy rounds fp32 -> fp16 to nearest-even
    if not np.all(np.isfinite(s)):
        raise ValueError("block scale overflows fp16")
    return s


def _check_input(w, group):
    w32 = np.asarray(w, dtype=np.float32)
    if w32.ndim != 2:
        raise ValueError("weights must be 2-D [N][K]")
    if w32.shape[1] % group != 0:
        raise ValueError(f"K={w32.shape[1]} is not a multiple of {group}")
    if not np.all(np.isfinite(w32)):
        raise ValueError("non-finite weight")
    return w32


def _nearest_e2m1_magnitude_code(r_abs):
    """Index (0..7) of the E2M1 magnitude nearest to r_abs (>= 0), ties to even.

    Above 6 every value saturates to 6 (code 7), which is also the nearest.
    """
    d = np.abs(r_abs[..., None].astype(np.float64) - _E2M1_MAG)  # exact differences
    dmin = d.min(axis=-1, keepdims=True)
    cand = d == dmin
    idx = np.argmax(cand, axis=-1)  # lowest candidate
    # two candidates can tie only as neighbours i, i+1: keep the even one
    two = cand.sum(axis=-1) > 1
    idx = np.where(two & (idx % 2 == 1), idx + 1, idx)
    return idx


def quantize_e2m1(w):
    """fp32 weights [N][K] -> (codes [N][K] uint8 in 0..15, scales [N][K/16] fp16)."""
    w32 = _check_input(w, E2M1_GROUP)
    n, k = w32.shape
    s = _block_scales(w32, E2M1_GROUP, 6)
    s32 = np.repeat(s.astype(np.float32), E2M1_GROUP, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s32 != 0, w32 / np.where(s32 != 0, s32, np.float32(1)), np.float32(0))
    mag = _nearest_e2m1_magnitude_code(np.abs(r))
    neg = (r < 0) & (mag != 0)
    codes = (mag + 8 * neg).astype(np.uint8)
    return codes, s


def quantize_int4(w):
    """fp32 weights [N][K] -> (codes [N][K] uint8 nibbles, scales [N][K/128] fp16)."""
    w32 = _check_input(w, INT4_GROUP)
    s = _block_scales(w32, INT4_GROUP, 7)
    s32 = np.repeat(s.astype(np.float32), INT4_GROUP, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s32 != 0, w32 / np.where(s32 != 0, s32, np.float32(1)), np.float32(0))
    q = np.clip(np.rint(r.astype(np.float64)), -8, 7).astype(np.int64)  # half to even
    codes = (q & 0xF).astype(np.uint8)
    return codes, s


def quantize_nvfp4(w):
    """fp32 weights [N][K] (one matrix) -> (codes [N][K] uint8 in 0..15,
    UE4M3 scale bytes [N][K/16] uint8, global scale np.float32)."""
    w32 = _check_input(w, E2M1_GROUP)
    n, k = w32.shape
    amax = np.abs(w32).max() if w32.size else np.float32(0)
    if amax == 0:
        return (np.zeros((n, k), np.uint8), np.zeros((n, k // E2M1_GROUP), np.uint8), np.float32(0))
    g = np.float32(amax) / np.float32(6 * 448)  # IEEE fp32 division
    a_blk = np.abs(w32.reshape(n, k // E2M1_GROUP, E2M1_GROUP)).max(axis=2)
    u = (a_blk / np.float32(6)) / g  # two fp32 divisions
    sb = f32_to_ue4m3(u)
    d = (e4m3_value(sb).astype(np.float32) * g).astype(np.float32)  # fp32 product
    d_full = np.repeat(d, E2M1_GROUP, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(d_full != 0, w32 / np.where(d_full != 0, d_full, np.float32(1)), np.float32(0))
    mag = _nearest_e2m1_magnitude_code(np.abs(r))
    neg = (r < 0) & (mag != 0)
    codes = (mag + 8 * neg).astype(np.uint8)
    return codes, sb, np.float32(g)


def quantize(fmt, w):
    """Quantize fp32 [N][K] to the canonical layout.

    E2M1 / int4: (packed codes [N][K/2] uint8, scale bits [N][K/G] uint16).
    NVFP4: (packed codes, UE4M3 scale bytes [N][K/16] uint8, global scale fp32).
    bf16: (bf16 bits [N][K] uint16,), each weight rounded to nearest even.
    """
    if fmt == FMT_BF16:
        return (f64_to_bf16_bits(np.asarray(w, dtype=np.float32).astype(np.float64)),)
    if fmt == FMT_E2M1:
        c, s = quantize_e2m1(w)
    elif fmt == FMT_INT4:
        c, s = quantize_int4(w)
    elif fmt == FMT_NVFP4:
        c, sb, g = quantize_nvfp4(w)
        return pack_nibbles(c), sb, g
    elif fmt == FMT_MXFP4:
        c, sb = quantize_mxfp4(w)
        return pack_nibbles(c), sb
    else:
        raise ValueError(f"unknown format {fmt}")
    return pack_nibbles(c), s.view(np.uint16)


# --------------------------------------------------------------------------- layout


def pack_nibbles(codes):
    """[..][K] nibbles -> [..][K/2] bytes: element 2j low nibble, 2j+1 high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[-1] % 2:
        raise ValueError("odd K")
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """[..][K/2] bytes -> [..][K] nibbles (inverse of pack_nibbles)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def codes_bytes(fmt, groups, n, k):
    """Bytes of packed codes for `groups` matrices of [n][k]: half a byte per element."""
    group_size(fmt)
    return groups * n * k // 2


def scales_bytes(fmt, groups, n, k):
    """Bytes of block scales: two bytes (FP16) per block of 16 (E2M1) or 128 (int4)
    elements, one byte (UE4M3) per block of 16 (NVFP4).  NVFP4 adds one fp32
    global scale per matrix, not counted here."""
    return groups * n * (k // group_size(fmt)) * _SCALE_BYTES[fmt]


# --------------------------------------------------------------------------- dequant


def dequant(fmt, packed, scale_bits=None, gscale=None):
    """Canonical codes [N][K/2] + block scales [N][K/G] -> fp32 [N][K].

    Each product value(code) * fp32(scale) is exact in fp32: an E2M1 value has at
    most 2 significant bits, an int4 value at most 4, an fp16 scale 11, and the
    smallest non-zero product (0.5 * 2**-24) is far above fp32's subnormal range.
    NVFP4 (scale_bits = UE4M3 bytes, gscale = the matrix's fp32 global scale):
    value(code) * value(scale) has at most 6 significant bits and is exact; the
    element is that product times g, rounded once to fp32.
    """
    if fmt == FMT_BF16:  # packed = bf16 bits [N][K]; exact in fp32
        return bf16_bits_to_f64(packed).astype(np.float32)
    g = group_size(fmt)
    nib = unpack_nibbles(packed)
    vals = _decode(fmt, nib).astype(np.float32)
    if fmt == FMT_MXFP4:  # value(code) * 2^(byte - 127): exact in fp32 for the bytes the quantiser emits
        s_full = np.repeat(e8m0_value(np.asarray(scale_bits, dtype=np.uint8)), g, axis=-1)
        out = vals.astype(np.float64) * s_full
        assert np.array_equal(out.astype(np.float32).astype(np.float64), out)
        return out.astype(np.float32)
    if fmt == FMT_NVFP4:
        if gscale is None:
            raise ValueError("NVFP4 needs the global scale")
        sb = np.asarray(scale_bits, dtype=np.uint8)
        s_full = np.repeat(e4m3_value(sb), g, axis=-1)
        if s_full.shape != vals.shape:
            raise ValueError("codes and scales disagree in shape")
        cs = vals.astype(np.float64) * s_full  # exact
        assert np.array_equal(cs.astype(np.float32).astype(np.float64), cs)
        return (cs * np.float64(np.float32(gscale))).astype(np.float32)  # one rounding
    s = np.asarray(scale_bits, dtype=np.uint16).view(np.float16).astype(np.float32)
    s_full = np.repeat(s, g, axis=-1)
    if s_full.shape != vals.shape:
        raise ValueError("codes and scales disagree in shape")
    out = vals * s_full
    # the float64 product is the exact one; it must equal the fp32 product
    assert np.array_equal(out.astype(np.float64), vals.astype(np.float64) * s_full.astype(np.float64))
    return out
