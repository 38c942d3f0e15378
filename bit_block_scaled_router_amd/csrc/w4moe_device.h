// Device helpers for the gfx950 W4A16 kernels: bit conversions, in-register
// decode of the 4-bit codes, 32-element chunk dot products and fixed-order
// cross-lane reductions.
//
// Lane geometry used by every weight-streaming kernel.  A matrix row of K
// elements is covered by L lanes (L = min(64, next power of two of K/32)); each
// lane owns 32 consecutive elements per step = 16 bytes of packed codes (one
// 128-bit load) and, for E2M1, exactly two FP16 scale blocks (one 32-bit load).
// A wave therefore covers 64/L rows per load and streams 1 KiB of contiguous
// canonical codes when K is a power of two <= 2048.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4k {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int FMT_E2M1 = 1;
constexpr int FMT_INT4 = 2;
constexpr int FMT_NVFP4 = 3;  // E2M1 codes, UE4M3 scale byte per 16, fp32 global scale per matrix
constexpr int FMT_MXFP4 = 5;  // E2M1 codes, E8M0 scale byte per 32

// bytes per block scale
template <int FMT>
constexpr uint32_t scale_bytes() {
    return (FMT == FMT_NVFP4 || FMT == FMT_MXFP4) ? 1u : 2u;
}

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN-ish).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(b & 0xFFFFu));
}

// a0*b0 + a1*b1 + acc over bf16 pairs, fp32 accumulate (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2(bf16x2 a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, as_bf16x2(b), acc, false);
}

// Two E2M1 codes (byte B of c: low nibble -> element 0) to two exact bf16.
template <int B>
__device__ __forceinline__ bf16x2 e2m1x2_bf16(uint32_t c) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, B);
}
template <int B>
__device__ __forceinline__ f32x2 e2m1x2_f32(uint32_t c) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, B);
}

// int4 decode.  u = nibble ^ 8 is q + 8 in [0, 15].  Spread into bytes, a byte
// u read as an OCP E4M3 code is exactly u * 2^-9 (subnormal for u < 8, exponent
// 1 otherwise), so the hardware fp8 conversion with scale 2^9 yields u exactly.
// lo holds nibbles 0,2,4,6 and hi nibbles 1,3,5,7 of the dword, one per byte.
__device__ __forceinline__ void int4_split(uint32_t c, uint32_t &lo, uint32_t &hi) {
    const uint32_t u = c ^ 0x88888888u;
    lo = u & 0x0F0F0F0Fu;
    hi = (u >> 4) & 0x0F0F0F0Fu;
}
template <bool W>
__device__ __forceinline__ bf16x2 u4x2_bf16(uint32_t bytes) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(bytes, 512.0f, W);
}
template <bool W>
__device__ __forceinline__ f32x2 u4x2_f32(uint32_t bytes) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(bytes, 512.0f, W);
}

// 8 int4 codes of one dword (element i in nibble i) -> their offset values
// u = q + 8 in [0, 15], exact in bf16, in element order (an MFMA operand).
__device__ __forceinline__ bf16x8 u4x8_bf16(uint32_t c) {
    uint32_t lo, hi;
    int4_split(c, lo, hi);                                          // lo: elements 0,2,4,6; hi: 1,3,5,7
    const uint32_t a = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // elements 0 1 2 3, one per byte
    const uint32_t b = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // elements 4 5 6 7
    const bf16x2 p0 = u4x2_bf16<false>(a), p1 = u4x2_bf16<true>(a), p2 = u4x2_bf16<false>(b), p3 = u4x2_bf16<true>(b);
    return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// bf16 8.0 in all eight elements: the int4 offset as an MFMA operand.
__device__ __forceinline__ bf16x8 bf16x8_splat8() {
    return __builtin_bit_cast(bf16x8, make_uint4(0x41004100u, 0x41004100u, 0x41004100u, 0x41004100u));
}

// ---------------------------------------------------------------- reductions

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Sum over aligned groups of L lanes (L a power of two <= 64), in a fixed order.
// L <= 16: butterfly within the row, every lane of the group gets the sum.
// L = 32, 64: the row sums are then combined with row broadcasts and the sum
// is valid in the LAST lane of each group (lane % L == L - 1).  Use
// group_leader<L>() to pick the lane that owns the result.  All 64 lanes must
// be active.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (L >= 2) v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (L >= 4) v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (L >= 8) v += dpp_f32<0x141>(v);  // row_half_mirror: the other quad
    if constexpr (L >= 16) v += dpp_f32<0x140>(v); // row_mirror: the other half-row
    if constexpr (L >= 32) {                       // row_bcast:15 into rows 1 and 3
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    }
    if constexpr (L >= 64) {                       // row_bcast:31 into row 3
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0x8, 0xF, false));
    }
    return v;
}

template <int L>
__device__ __forceinline__ bool group_leader(int lane) {
    return (lane & (L - 1)) == L - 1;
}

// Maximum over the wave, returned to every lane (wave-uniform).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<0xB1>(v));
    v = max(v, dpp_u32<0x4E>(v));
    v = max(v, dpp_u32<0x141>(v));
    v = max(v, dpp_u32<0x140>(v));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0x8, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Global wave index, marked wave-uniform (a scalar register) so that pointers
// and buffer resources derived from it need no per-lane handling.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)));
}

// Wave-uniform loads through the scalar cache (constant address space): used
// for routing ids and weights so that they do not queue behind vector loads.
typedef const __attribute__((address_space(4))) int32_t c4_i32;
typedef const __attribute__((address_space(4))) float c4_f32;
__device__ __forceinline__ int32_t ld_uniform(const int32_t *p, int idx) {
    return ((c4_i32 *)p)[__builtin_amdgcn_readfirstlane(idx)];
}
__device__ __forceinline__ float ld_uniform(const float *p, int idx) {
    return ((c4_f32 *)p)[__builtin_amdgcn_readfirstlane(idx)];
}

// ---------------------------------------------------------------- buffer loads

// Raw buffer resources: a load whose byte offset lies at or beyond the
// resource's size returns zero instead of touching memory, so masked lanes
// need no branch.  Sizes are below 2 GiB per resource.
constexpr uint32_t OOB = 0x80000000u;

struct Buf {
    __amdgpu_buffer_rsrc_t r;
};

__device__ __forceinline__ Buf make_buf(const void *p, uint32_t bytes) {
    return Buf{__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000)};
}

__device__ __forceinline__ uint4 ld128(Buf b, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(b.r, off, 0, 0));
}
__device__ __forceinline__ uint32_t ld32(Buf b, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(b.r, off, 0, 0);
}
__device__ __forceinline__ uint32_t ld8(Buf b, uint32_t off) {
    return (uint32_t)(uint8_t)__builtin_amdgcn_raw_buffer_load_b8(b.r, off, 0, 0);
}
__device__ __forceinline__ uint32_t ld16(Buf b, uint32_t off) {
    return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(b.r, off, 0, 0);
}

// ---------------------------------------------------------------- MXFP8

// MXFP8 quantisation of activations: shared exponent of a block with maximum
// magnitude `amax`: floor(log2 amax) - 8 (E4M3's largest exponent), limited to
// [-127, 127]; -127 for an all-zero block.
__device__ __forceinline__ int mx8_exponent(float amax) {
    if (!(amax > 0.f)) return -127;
    int X = __builtin_amdgcn_frexp_expf(amax) - 1 - 8;  // amax = m 2^e, m in [0.5, 1)
    return X < -127 ? -127 : (X > 127 ? 127 : X);
}

// Four activations -> four E4M3 bytes of v / 2^X, clamped to +-448, round to
// nearest even (the conversion instruction with unit scale).
__device__ __forceinline__ uint32_t mx8_pack4(float a, float b, float c, float d, int X) {
    auto cl = [&](float v) { return fminf(fmaxf(__builtin_amdgcn_ldexpf(v, -X), -448.f), 448.f); };
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    s16x2 w = {0, 0};
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, cl(a), cl(b), 1.0f, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, cl(c), cl(d), 1.0f, true);
    return __builtin_bit_cast(uint32_t, w);
}

// One MXFP8 block of 32 fp32 values (float4 q holds elements 4q .. 4q+3), in
// place: each value becomes its E4M3 element E4M3(v / 2^X) (exact in fp32);
// returns the block's shared exponent X.
__device__ __forceinline__ int mx8_block_f32(float4 *v) {
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q)
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[q].x), fabsf(v[q].y)), fmaxf(fabsf(v[q].z), fabsf(v[q].w))));
    const int X = mx8_exponent(amax);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint32_t w = mx8_pack4(v[q].x, v[q].y, v[q].z, v[q].w, X);
        const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
        const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
        v[q] = make_float4(a.x, a.y, b.x, b.y);
    }
    return X;
}

// ---------------------------------------------------------------- activations

// Activation slice of one lane for one step: 32 bf16 values as 16 dwords.  For
// int4 the pairs are regrouped to match the byte order of int4_split and the
// slice sum is kept for the +8 offset correction.
template <int FMT>
struct XSlice {
    uint4 v[4];
    float sum;
    int X;  // MXFP4 layers: shared exponent of the slice's MXFP8 block
};

// Load the slice at byte offset `off` of the activation buffer (OOB -> zeros).
template <int FMT>
__device__ __forceinline__ void load_xslice(XSlice<FMT> &xs, Buf xb, uint32_t off) {
#pragma unroll
    for (int i = 0; i < 4; ++i) xs.v[i] = ld128(xb, off + 16u * i);
}

template <int FMT>
__device__ __forceinline__ void prep_xslice(XSlice<FMT> &xs) {
    if constexpr (FMT == FMT_INT4) {
        // element pairs (0,1),(2,3),(4,5),(6,7) -> (0,2),(4,6),(1,3),(5,7)
        float s = 0.f;
        const uint32_t ones = 0x3F803F80u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 a = xs.v[i];
            s = dot2(as_bf16x2(a.x), ones, s);
            s = dot2(as_bf16x2(a.y), ones, s);
            s = dot2(as_bf16x2(a.z), ones, s);
            s = dot2(as_bf16x2(a.w), ones, s);
            uint4 b;
            b.x = __builtin_amdgcn_perm(a.y, a.x, 0x05040100u);  // (x0, x2)
            b.y = __builtin_amdgcn_perm(a.w, a.z, 0x05040100u);  // (x4, x6)
            b.z = __builtin_amdgcn_perm(a.y, a.x, 0x07060302u);  // (x1, x3)
            b.w = __builtin_amdgcn_perm(a.w, a.z, 0x07060302u);  // (x5, x7)
            xs.v[i] = b;
        }
        xs.sum = s;
    } else if constexpr (FMT == FMT_MXFP4) {
        // the slice is one MXFP8 block: each bf16 becomes its E4M3 element
        // (at most 4 significant bits, exact in bf16) and X is kept for the scale
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t d[4] = {xs.v[i].x, xs.v[i].y, xs.v[i].z, xs.v[i].w};
#pragma unroll
            for (int m = 0; m < 4; ++m)
                amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(d[m] << 16)), fabsf(__uint_as_float(d[m] & 0xFFFF0000u))));
        }
        const int X = mx8_exponent(amax);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t d[4] = {xs.v[i].x, xs.v[i].y, xs.v[i].z, xs.v[i].w};
#pragma unroll
            for (int m = 0; m < 4; m += 2) {
                const uint32_t w = mx8_pack4(__uint_as_float(d[m] << 16), __uint_as_float(d[m] & 0xFFFF0000u),
                                             __uint_as_float(d[m + 1] << 16), __uint_as_float(d[m + 1] & 0xFFFF0000u), X);
                const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
                const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
                d[m] = __builtin_amdgcn_perm(__float_as_uint(a.y), __float_as_uint(a.x), 0x07060302u);
                d[m + 1] = __builtin_amdgcn_perm(__float_as_uint(b.y), __float_as_uint(b.x), 0x07060302u);
            }
            xs.v[i] = make_uint4(d[0], d[1], d[2], d[3]);
        }
        xs.sum = 0.f;
        xs.X = X;
    } else {
        xs.sum = 0.f;
    }
}

// ---------------------------------------------------------------- chunk dots

// E2M1: 8 codes of one dword against 8 bf16 activations.
__device__ __forceinline__ float e2m1_dot8(uint32_t c, uint4 x, float acc) {
    acc = dot2(e2m1x2_bf16<0>(c), x.x, acc);
    acc = dot2(e2m1x2_bf16<1>(c), x.y, acc);
    acc = dot2(e2m1x2_bf16<2>(c), x.z, acc);
    acc = dot2(e2m1x2_bf16<3>(c), x.w, acc);
    return acc;
}

// int4 (offset form u = q + 8): 8 codes of one dword against 8 regrouped bf16.
__device__ __forceinline__ float u4_dot8(uint32_t c, uint4 x, float acc) {
    uint32_t lo, hi;
    int4_split(c, lo, hi);
    acc = dot2(u4x2_bf16<false>(lo), x.x, acc);
    acc = dot2(u4x2_bf16<true>(lo), x.y, acc);
    acc = dot2(u4x2_bf16<false>(hi), x.z, acc);
    acc = dot2(u4x2_bf16<true>(hi), x.w, acc);
    return acc;
}

// The two block scales of a lane's 32 elements (E2M1: two FP16 in the dword,
// NVFP4: two UE4M3 bytes in its low half, decoded by the gfx950 fp8 -> fp32
// conversion with unit scale).
template <int FMT>
__device__ __forceinline__ f32x2 block_scales2(uint32_t sc) {
    if constexpr (FMT == FMT_NVFP4) {
        return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sc, 1.0f, false);
    } else if constexpr (FMT == FMT_MXFP4) {  // one E8M0 byte for all 32 elements
        const float s = __builtin_amdgcn_ldexpf(1.0f, (int)(sc & 0xFFu) - 127);
        return f32x2{s, s};
    } else {
        return f32x2{f16_bits_to_f32(sc), f16_bits_to_f32(sc >> 16)};
    }
}

// 32 bf16 weights (4 x 16 bytes) of one lane against its bf16 activations
// (the unpermuted slice: load_xslice without prep_xslice).
template <int FMT>
__device__ __forceinline__ float bf16w_dot_bf16(const uint4 *w, const XSlice<FMT> &xs, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc = dot2(as_bf16x2(w[i].x), xs.v[i].x, acc);
        acc = dot2(as_bf16x2(w[i].y), xs.v[i].y, acc);
        acc = dot2(as_bf16x2(w[i].z), xs.v[i].z, acc);
        acc = dot2(as_bf16x2(w[i].w), xs.v[i].w, acc);
    }
    return acc;
}

// 32 bf16 weights of one lane against its 32 fp32 activations h[8] (float4 q
// holds elements 4q..4q+3).
__device__ __forceinline__ float bf16w_dot_f32(const uint4 *w, const float4 *h, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t d[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = 8 * i + 2 * m;  // elements e, e+1
            const float4 hq = h[e >> 2];
            const float h0 = (e & 3) ? hq.z : hq.x, h1 = (e & 3) ? hq.w : hq.y;
            acc = fmaf(__uint_as_float(d[m] << 16), h0, acc);
            acc = fmaf(__uint_as_float(d[m] & 0xFFFF0000u), h1, acc);
        }
    }
    return acc;
}

// One lane's 32 elements (16 bytes of codes + its scales) against bf16
// activations, added to acc in a fixed order.  E2M1: the dword `sc` holds the
// two FP16 scales of the lane's two blocks (low half = first block).  int4: the
// low half of `sc` is the group's scale.
template <int FMT>
__device__ __forceinline__ float chunk_dot_bf16(uint4 c, uint32_t sc, const XSlice<FMT> &xs, float acc) {
    if constexpr (FMT == FMT_E2M1 || FMT == FMT_NVFP4) {
        float p0 = e2m1_dot8(c.x, xs.v[0], 0.f);
        p0 = e2m1_dot8(c.y, xs.v[1], p0);
        float p1 = e2m1_dot8(c.z, xs.v[2], 0.f);
        p1 = e2m1_dot8(c.w, xs.v[3], p1);
        const f32x2 s = block_scales2<FMT>(sc);
        acc = fmaf(p0, s.x, acc);
        acc = fmaf(p1, s.y, acc);
    } else if constexpr (FMT == FMT_MXFP4) {
        // one block: E2M1 codes x E4M3 activations (exact products), then both
        // shared exponents at once (the E8M0 byte and the slice's X)
        float p = e2m1_dot8(c.x, xs.v[0], 0.f);
        p = e2m1_dot8(c.y, xs.v[1], p);
        p = e2m1_dot8(c.z, xs.v[2], p);
        p = e2m1_dot8(c.w, xs.v[3], p);
        acc += __builtin_amdgcn_ldexpf(p, (int)(sc & 0xFFu) - 127 + xs.X);
    } else {
        float p = u4_dot8(c.x, xs.v[0], 0.f);
        p = u4_dot8(c.y, xs.v[1], p);
        p = u4_dot8(c.z, xs.v[2], p);
        p = u4_dot8(c.w, xs.v[3], p);
        p = fmaf(-8.f, xs.sum, p);
        acc = fmaf(p, f16_bits_to_f32(sc), acc);
    }
    return acc;
}

// Same against fp32 activations h[32] (the down projection's SiLU(gate)*up).
// hs = sum of the 32 activations (int4 offset correction).  MXFP4: h holds the
// E4M3 elements of one MXFP8 block and hx its shared exponent.
template <int FMT>
__device__ __forceinline__ float chunk_dot_f32(uint4 c, uint32_t sc, const float4 *h, float hs, float acc,
                                               int hx = 0) {
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    if constexpr (FMT == FMT_MXFP4) {
        float q = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {  // dword d: elements 8d .. 8d+7
            const float4 h0 = h[2 * d], h1 = h[2 * d + 1];
            f32x2 w;
            w = e2m1x2_f32<0>(cw[d]); q = fmaf(w.x, h0.x, q); q = fmaf(w.y, h0.y, q);
            w = e2m1x2_f32<1>(cw[d]); q = fmaf(w.x, h0.z, q); q = fmaf(w.y, h0.w, q);
            w = e2m1x2_f32<2>(cw[d]); q = fmaf(w.x, h1.x, q); q = fmaf(w.y, h1.y, q);
            w = e2m1x2_f32<3>(cw[d]); q = fmaf(w.x, h1.z, q); q = fmaf(w.y, h1.w, q);
        }
        acc += __builtin_amdgcn_ldexpf(q, (int)(sc & 0xFFu) - 127 + hx);
    } else if constexpr (FMT == FMT_E2M1 || FMT == FMT_NVFP4) {
        float p[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            float q = 0.f;
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const uint32_t cd = cw[2 * b + d];
                const float4 h0 = h[4 * b + 2 * d], h1 = h[4 * b + 2 * d + 1];
                f32x2 w;
                w = e2m1x2_f32<0>(cd); q = fmaf(w.x, h0.x, q); q = fmaf(w.y, h0.y, q);
                w = e2m1x2_f32<1>(cd); q = fmaf(w.x, h0.z, q); q = fmaf(w.y, h0.w, q);
                w = e2m1x2_f32<2>(cd); q = fmaf(w.x, h1.x, q); q = fmaf(w.y, h1.y, q);
                w = e2m1x2_f32<3>(cd); q = fmaf(w.x, h1.z, q); q = fmaf(w.y, h1.w, q);
            }
            p[b] = q;
        }
        const f32x2 s = block_scales2<FMT>(sc);
        acc = fmaf(p[0], s.x, acc);
        acc = fmaf(p[1], s.y, acc);
    } else {
        float q = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t lo, hi;
            int4_split(cw[d], lo, hi);
            const float4 h0 = h[2 * d], h1 = h[2 * d + 1];  // elements 8d..8d+7
            f32x2 w;
            w = u4x2_f32<false>(lo); q = fmaf(w.x, h0.x, q); q = fmaf(w.y, h0.z, q);  // 0, 2
            w = u4x2_f32<true>(lo);  q = fmaf(w.x, h1.x, q); q = fmaf(w.y, h1.z, q);  // 4, 6
            w = u4x2_f32<false>(hi); q = fmaf(w.x, h0.y, q); q = fmaf(w.y, h0.w, q);  // 1, 3
            w = u4x2_f32<true>(hi);  q = fmaf(w.x, h1.y, q); q = fmaf(w.y, h1.w, q);  // 5, 7
        }
        q = fmaf(-8.f, hs, q);
        acc = fmaf(q, f16_bits_to_f32(sc), acc);
    }
    return acc;
}

// Byte offset, within a row's scales, of the scale(s) of the 32-element lane
// chunk starting at K index k0 (E2M1: two FP16 at block k0/16; NVFP4: two UE4M3
// bytes; MXFP4: one E8M0 byte at block k0/32; int4: one FP16 at group k0/128).
template <int FMT>
__device__ __forceinline__ uint32_t scale_col(int k0) {
    return FMT == FMT_INT4 ? (uint32_t)(k0 >> 7) * 2u
           : FMT == FMT_MXFP4 ? (uint32_t)(k0 >> 5)
                              : (uint32_t)(k0 >> 4) * scale_bytes<FMT>();
}

template <int FMT>
__device__ __forceinline__ uint32_t ld_scales(Buf b, uint32_t off) {
    if constexpr (FMT == FMT_E2M1)
        return ld32(b, off);
    else if constexpr (FMT == FMT_MXFP4)
        return ld8(b, off);  // one E8M0 byte
    else
        return ld16(b, off);  // int4: one FP16; NVFP4: two UE4M3 bytes
}


// ---------------------------------------------------------------- top-k

// Order-preserving map of a finite float to uint32 (larger float -> larger key;
// every finite value maps above 0, which marks a removed entry).
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave ranks E <= 64*PL logits (+ bias) by descending value, ties to the
// lower expert id, for `rounds` rounds, for NT tokens at once (their rounds
// interleave: independent reductions hide each other's latency).  Ranking by
// logit equals ranking by softmax probability (exp is increasing).  Lane l
// holds experts l*PL .. l*PL+PL-1, so "lowest lane, then lowest slot" is the
// lowest id.  A round takes each lane's best remaining entry (first index on
// equal keys), the wave maximum of those and the lowest lane holding it; that
// lane removes the entry.  Lane j < rounds receives token n's j-th id and its
// (biased) logit in my_id[n], my_val[n]; token 0's id of round `want` is
// returned to every lane.  Tokens n >= nvalid read nothing (their results are
// meaningless).
template <int PL, int NT>
__device__ __forceinline__ int wave_topk_n(const float *const *lg, const float *__restrict__ bias, int E, int nvalid,
                                           int rounds, int want, int *my_id, float *my_val) {
    const int lane = threadIdx.x & 63;
    const Buf bb = make_buf(bias, bias ? (uint32_t)E * 4u : 0u);
    uint32_t key[NT][PL];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const Buf lb = make_buf(lg[n], n < nvalid ? (uint32_t)E * 4u : 0u);
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            const int e = lane * PL + i;
            const uint32_t off = e < E ? (uint32_t)e * 4u : OOB;
            const float v = __uint_as_float(ld32(lb, off)) + __uint_as_float(ld32(bb, off));
            key[n][i] = e < E ? order_key(v) : 0u;
        }
        my_id[n] = -1;
        my_val[n] = 0.f;
    }
    int sel = 0;
    for (int j = 0; j < rounds; ++j) {
        uint32_t best[NT];
        int bi[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            best[n] = key[n][0];
            bi[n] = 0;
#pragma unroll
            for (int i = 1; i < PL; ++i) {
                const bool gt = key[n][i] > best[n];
                best[n] = gt ? key[n][i] : best[n];
                bi[n] = gt ? i : bi[n];
            }
        }
        uint32_t m[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) m[n] = wave_max_u32(best[n]);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const uint64_t mask = __ballot(best[n] == m[n]);
            const int winner = __ffsll((unsigned long long)mask) - 1;
            const int wid = __builtin_amdgcn_readlane(lane * PL + bi[n], winner);
            const bool pop = lane == winner;
#pragma unroll
            for (int i = 0; i < PL; ++i) key[n][i] = (pop && i == bi[n]) ? 0u : key[n][i];
            const bool mine = lane == j;
            my_id[n] = mine ? wid : my_id[n];
            my_val[n] = mine ? __uint_as_float((m[n] & 0x80000000u) ? (m[n] & 0x7FFFFFFFu) : ~m[n]) : my_val[n];
            if (n == 0) sel = j == want ? wid : sel;
        }
    }
    return sel;
}

// One token (lane j < rounds receives the j-th id and logit; the id of round
// `want` is returned to every lane).
template <int PL>
__device__ __forceinline__ int wave_topk(const float *__restrict__ lg, const float *__restrict__ bias, int E,
                                         int rounds, int want, int &my_id, float &my_val) {
    const float *l[1] = {lg};
    return wave_topk_n<PL, 1>(l, bias, E, 1, rounds, want, &my_id, &my_val);
}

// Inclusive prefix sum over the 64 lanes in lane order: shifts within each row
// of 16 lanes, then the row totals by row broadcasts.  All lanes active.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
    return v;
}

// ---------------------------------------------------------------- MFMA helpers

typedef float f32x4 __attribute__((ext_vector_type(4)));

// D += A(16x32) B(32x16), bf16 in, fp32 accumulate.  Lane i holds
// A[i%16][8(i/16)..+8], B[8(i/16)..+8][i%16] and D[4(i/16)+j][i%16], j < 4.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two floats whose values are exact in bf16 -> packed bf16x2 (upper halves).
__device__ __forceinline__ uint32_t pack_bf16_exact(float a, float b) {
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// Exact two-term split of an FP16 scale s (held in fp32): s_hi keeps the top 6
// significant bits, s_lo = s - s_hi has at most 5.  An E2M1 value has at most 2
// significant bits, so code*s_hi (<= 8 bits) and code*s_lo (<= 7 bits) are both
// exact in bf16 and code*s = code*s_hi + code*s_lo exactly.
__device__ __forceinline__ void split_scale(float s, float &s_hi, float &s_lo) {
    s_hi = __uint_as_float(__float_as_uint(s) & 0xFFFC0000u);
    s_lo = s - s_hi;
}

// 8 E2M1 codes of one dword (elements 0..7) times a split scale -> bf16x8 hi/lo.
__device__ __forceinline__ void e2m1x8_split(uint32_t c, float s_hi, float s_lo, bf16x8 &hi, bf16x8 &lo) {
    uint32_t h[4], l[4];
    f32x2 v;
    v = e2m1x2_f32<0>(c); h[0] = pack_bf16_exact(v.x * s_hi, v.y * s_hi); l[0] = pack_bf16_exact(v.x * s_lo, v.y * s_lo);
    v = e2m1x2_f32<1>(c); h[1] = pack_bf16_exact(v.x * s_hi, v.y * s_hi); l[1] = pack_bf16_exact(v.x * s_lo, v.y * s_lo);
    v = e2m1x2_f32<2>(c); h[2] = pack_bf16_exact(v.x * s_hi, v.y * s_hi); l[2] = pack_bf16_exact(v.x * s_lo, v.y * s_lo);
    v = e2m1x2_f32<3>(c); h[3] = pack_bf16_exact(v.x * s_hi, v.y * s_hi); l[3] = pack_bf16_exact(v.x * s_lo, v.y * s_lo);
    hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
    lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

// 8 E2M1 codes of one dword (elements 0..7) times a scale whose product with
// every code is exact in bf16 (an NVFP4 UE4M3 block scale: at most 4
// significant bits, a code at most 2) -> bf16x8.
__device__ __forceinline__ bf16x8 e2m1x8_scaled(uint32_t c, float s) {
    uint32_t h[4];
    f32x2 v;
    v = e2m1x2_f32<0>(c); h[0] = pack_bf16_exact(v.x * s, v.y * s);
    v = e2m1x2_f32<1>(c); h[1] = pack_bf16_exact(v.x * s, v.y * s);
    v = e2m1x2_f32<2>(c); h[2] = pack_bf16_exact(v.x * s, v.y * s);
    v = e2m1x2_f32<3>(c); h[3] = pack_bf16_exact(v.x * s, v.y * s);
    return __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Scaled FP4 x FP8 MFMA (gfx950 v_mfma_scale_f32_16x16x128_f8f6f4): D += A B with
// A 16 rows x 128 K of E2M1 codes and B 128 K x 16 columns of E4M3 values, each
// block of 32 K elements scaled by its E8M0 byte.  Lane l (g = l / 16): A holds
// row l % 16, K = 32 g .. 32 g + 31 (16 bytes, low nibble = even element) and
// that block's scale `sa`; B holds column l % 16, K = 16 g .. 16 g + 15 (b_lo) and
// 64 + 16 g .. 64 + 16 g + 15 (b_hi), plus the column's scale of block g (`sb`);
// D[4 g + j][l % 16] in component j (operand mapping measured on the device).
__device__ __forceinline__ f32x4 mfma_mx(uint4 a, uint4 b_lo, uint4 b_hi, uint32_t sa, uint32_t sb, f32x4 c) {
    const i32x8 A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const i32x8 B = {(int)b_lo.x, (int)b_lo.y, (int)b_lo.z, (int)b_lo.w,
                     (int)b_hi.x, (int)b_hi.y, (int)b_hi.z, (int)b_hi.w};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 0, 0, (int)sa, 0, (int)sb);
}

// One fp32 value -> bf16 hi (truncated) + bf16 lo (residual, rounded to
// nearest): hi + lo carries about 16 significant bits of v.
__device__ __forceinline__ void split_bf16(float v, uint16_t &hi, uint16_t &lo) {
    const float h = __uint_as_float(__float_as_uint(v) & 0xFFFF0000u);
    hi = (uint16_t)(__float_as_uint(v) >> 16);
    lo = f32_to_bf16_rne(v - h);
}

// 8 fp32 activations -> bf16 hi (truncated) + lo (residual rounded to nearest);
// hi + lo carries about 16 significant bits.
__device__ __forceinline__ void f32x8_split(float4 a, float4 b, bf16x8 &hi, bf16x8 &lo) {
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float h0 = __uint_as_float(__float_as_uint(v[2 * i]) & 0xFFFF0000u);
        const float h1 = __uint_as_float(__float_as_uint(v[2 * i + 1]) & 0xFFFF0000u);
        h[i] = pack_bf16_exact(h0, h1);
        l[i] = (uint32_t)f32_to_bf16_rne(v[2 * i] - h0) | ((uint32_t)f32_to_bf16_rne(v[2 * i + 1] - h1) << 16);
    }
    hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
    lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

}  // namespace w4k
