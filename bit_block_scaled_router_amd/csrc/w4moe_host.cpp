// Host side of the w4moe C ABI: status strings, the thread-local error message,
// size formulas, the offline quantiser and nibble packing.  Nothing here touches
// the GPU.  Rules are those of include/w4moe.h; sources: "Lynn Engine" article,
// "Kernel optimisation history" stage P1 (E2M1 + FP16 scale per 16 K elements),
// the "cuda_inf" article, "2. INT4 weight quantization" (int4, group 128), and
// the lynn-engine README notes P17/P29/R5-C0 (UE4M3 per-16 scales and a global
// scale: the NVFP4 variant).
#include "w4moe_internal.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

namespace w4 {

static thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

void clear_error() { g_err[0] = 0; }

int group_of(int32_t format) {
    switch (format) {
    case W4_FMT_E2M1_F16S16: return 16;
    case W4_FMT_INT4_F16S128: return 128;
    case W4_FMT_NVFP4_E4M3S16: return 16;
    case W4_FMT_BF16: return 32;  // no scale blocks; k must be a multiple of 32
    case W4_FMT_MXFP4_E8M0S32: return 32;
    default: return 0;
    }
}

int check_shape(int32_t format, int32_t layout, int64_t groups, int64_t n, int64_t k) {
    const int g = group_of(format);
    if (!g) return fail(W4_ERR_LAYOUT, "unknown format tag %d", (int)format);
    if (layout != W4_LAYOUT_CANONICAL && layout != W4_LAYOUT_GFX950_V1 && layout != W4_LAYOUT_GFX950_KT16)
        return fail(W4_ERR_LAYOUT, "unknown layout tag %d", (int)layout);
    if (layout == W4_LAYOUT_GFX950_KT16 && format != W4_FMT_E2M1_F16S16 && format != W4_FMT_NVFP4_E4M3S16)
        return fail(W4_ERR_UNSUPPORTED, "the K-tiled layout holds E2M1 or NVFP4 matrices (one scale per 16-wide tile)");
    if (groups < 1 || n < 1 || k < 1) return fail(W4_ERR_INVALID_ARG, "groups/n/k must be >= 1");
    const int64_t kmul = format == W4_FMT_INT4_F16S128 ? 128 : 32;
    if (k % kmul) return fail(W4_ERR_INVALID_ARG, "k=%lld must be a multiple of %lld", (long long)k, (long long)kmul);
    if (groups > (int64_t(1) << 20) || n > (int64_t(1) << 31) || k > (int64_t(1) << 24))
        return fail(W4_ERR_INVALID_ARG, "matrix dimensions out of range");
    return W4_OK;
}

size_t scale_bytes_per_row(int32_t format, int64_t k) {
    if (format == W4_FMT_BF16) return 0;
    const size_t b = (format == W4_FMT_NVFP4_E4M3S16 || format == W4_FMT_MXFP4_E8M0S32) ? 1 : 2;
    return (size_t)(k / group_of(format)) * b;
}

size_t code_bytes_per_row(int32_t format, int64_t k) { return format == W4_FMT_BF16 ? (size_t)k * 2 : (size_t)k / 2; }

size_t v1_row_bytes(int32_t format, int64_t k) {
    const size_t b = code_bytes_per_row(format, k) + scale_bytes_per_row(format, k);
    return (b + 15) / 16 * 16;
}

size_t kt16_tile_bytes(int32_t format, int64_t n) {
    const size_t sb = format == W4_FMT_NVFP4_E4M3S16 ? 1 : 2;
    return ((size_t)n * (8 + sb) + 15) / 16 * 16;
}

// ---------------------------------------------------------------- fp16 / E2M1

// fp32 -> fp16 bits, round to nearest even; the compiler's _Float16 conversion
// follows the IEEE default rounding mode.
static inline uint16_t f32_to_f16_bits(float v) {
    _Float16 h = (_Float16)v;
    uint16_t b;
    std::memcpy(&b, &h, 2);
    return b;
}

static inline float f16_bits_to_f32(uint16_t b) {
    _Float16 h;
    std::memcpy(&h, &b, 2);
    return (float)h;
}

// Non-negative fp32 -> UE4M3 byte (OCP E4M3 with sign 0: exponent bias 7, 3
// mantissa bits, subnormals m * 2^-9), round to nearest even, saturating at 448
// (code 0x7E; 0x7F is NaN and never produced).
static inline uint8_t f32_to_ue4m3(float x) {
    if (!(x < 448.0f)) return 0x7E;
    if (x < 0.015625f) {  // below 2^-6: subnormal grid of 2^-9 (exact scaling)
        const float m = std::nearbyint(x * 512.0f);  // 0..8; 8 is the first normal
        return (uint8_t)m;
    }
    int e;
    const float f = std::frexp(x, &e);             // x = f * 2^e, f in [0.5, 1)
    float m = std::nearbyint((2.0f * f - 1.0f) * 8.0f);  // exact operand, ties to even
    int be = e - 1 + 7;
    if (m == 8.0f) m = 0.0f, ++be;
    const int code = (be << 3) | (int)m;
    return (uint8_t)(code > 0x7E ? 0x7E : code);
}

static inline float ue4m3_to_f32(uint8_t c) {
    const int be = (c >> 3) & 0xF, m = c & 7;
    return be == 0 ? std::ldexp((float)m, -9) : std::ldexp(1.0f + (float)m / 8.0f, be - 7);
}

// Nearest E2M1 magnitude code (0..7) to r >= 0, ties to the even code.
// Magnitudes by code: 0, 0.5, 1, 1.5, 2, 3, 4, 6; the midpoints between
// neighbours are 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.  On a midpoint the even
// code wins, so a midpoint below an even code belongs to the upper interval.
static inline int e2m1_mag_code(float r) {
    if (r <= 0.25f) return 0;   // 0.25 ties to code 0
    if (r < 0.75f) return 1;    // 0.75 ties to code 2
    if (r <= 1.25f) return 2;   // 1.25 ties to code 2
    if (r < 1.75f) return 3;    // 1.75 ties to code 4
    if (r <= 2.5f) return 4;    // 2.5 ties to code 4
    if (r < 3.5f) return 5;     // 3.5 ties to code 6
    if (r <= 5.0f) return 6;    // 5 ties to code 6
    return 7;                   // saturate
}

// gscale: the matrix's NVFP4 global scale (unused for the FP16-scale formats).
static void quantize_rows(int32_t format, const float *w, int64_t r0, int64_t r1, int64_t k,
                          uint8_t *codes, void *scales, float gscale) {
    const int g = group_of(format);
    const float qmax = format == W4_FMT_INT4_F16S128 ? 7.0f : 6.0f;
    const int64_t nb = k / g;
    for (int64_t r = r0; r < r1; ++r) {
        const float *wr = w + r * k;
        uint8_t *cr = codes + r * (k / 2);
        for (int64_t b = 0; b < nb; ++b) {
            const float *wb = wr + b * g;
            float a = 0.f;
            for (int i = 0; i < g; ++i) a = std::fmax(a, std::fabs(wb[i]));
            float s;  // the divisor of the codes
            if (format == W4_FMT_MXFP4_E8M0S32) {  // shared exponent floor(log2 a) - 2
                int X = -127;
                if (a > 0.f) {
                    int e;
                    std::frexp(a, &e);  // a = f 2^e, f in [0.5, 1): floor(log2 a) = e - 1
                    X = e - 1 - 2;
                    X = X < -127 ? -127 : (X > 127 ? 127 : X);
                }
                static_cast<uint8_t *>(scales)[r * nb + b] = (uint8_t)(X + 127);
                s = a > 0.f ? std::ldexp(1.0f, X) : 0.f;  // power of two: the division below is exact
            } else if (format == W4_FMT_NVFP4_E4M3S16) {
                const uint8_t sb = gscale != 0.f ? f32_to_ue4m3((a / 6.0f) / gscale) : 0;
                static_cast<uint8_t *>(scales)[r * nb + b] = sb;
                s = ue4m3_to_f32(sb) * gscale;  // fp32 product
            } else {
                const uint16_t sb = f32_to_f16_bits(a / qmax);
                static_cast<uint16_t *>(scales)[r * nb + b] = sb;
                s = f16_bits_to_f32(sb);
            }
            for (int i = 0; i < g; i += 2) {
                uint8_t c2[2];
                for (int j = 0; j < 2; ++j) {
                    uint8_t c = 0;
                    if (s != 0.f) {
                        const float q = wb[i + j] / s;  // IEEE fp32 division
                        if (format != W4_FMT_INT4_F16S128) {
                            const int m = e2m1_mag_code(std::fabs(q));
                            c = (uint8_t)(m | ((q < 0.f && m != 0) ? 8 : 0));
                        } else {
                            float t = std::nearbyint(q);  // half to even (default mode)
                            t = std::fmin(7.f, std::fmax(-8.f, t));
                            c = (uint8_t)(((int)t) & 0xF);
                        }
                    }
                    c2[j] = c;
                }
                cr[(b * g + i) / 2] = (uint8_t)(c2[0] | (c2[1] << 4));
            }
        }
    }
}

}  // namespace w4

using namespace w4;

extern "C" {

const char *w4_status_string(int status) {
    switch (status) {
    case W4_OK: return "W4_OK";
    case W4_ERR_INVALID_ARG: return "W4_ERR_INVALID_ARG";
    case W4_ERR_LAYOUT: return "W4_ERR_LAYOUT";
    case W4_ERR_ALIGNMENT: return "W4_ERR_ALIGNMENT";
    case W4_ERR_UNSUPPORTED: return "W4_ERR_UNSUPPORTED";
    case W4_ERR_WORKSPACE: return "W4_ERR_WORKSPACE";
    case W4_ERR_NONFINITE: return "W4_ERR_NONFINITE";
    case W4_ERR_RANGE: return "W4_ERR_RANGE";
    case W4_ERR_HIP: return "W4_ERR_HIP";
    default: return "W4_ERR_UNKNOWN";
    }
}

const char *w4_last_error(void) { return g_err; }

const char *w4_version(void) { return "w4moe 0.1 gfx950"; }

size_t w4_codes_bytes(int32_t format, int32_t layout, int64_t groups, int64_t n, int64_t k) {
    if (check_shape(format, layout, groups, n, k) != W4_OK) return 0;
    const size_t rows = (size_t)groups * (size_t)n;
    if (layout == W4_LAYOUT_GFX950_V1) return rows * v1_row_bytes(format, k);
    if (layout == W4_LAYOUT_GFX950_KT16) return (size_t)groups * (size_t)(k / 16) * kt16_tile_bytes(format, n);
    return rows * code_bytes_per_row(format, k);
}

size_t w4_scales_bytes(int32_t format, int32_t layout, int64_t groups, int64_t n, int64_t k) {
    if (check_shape(format, layout, groups, n, k) != W4_OK) return 0;
    if (layout != W4_LAYOUT_CANONICAL) return 0;  // the scales travel inside the row or tile records
    return (size_t)groups * (size_t)n * scale_bytes_per_row(format, k);
}

int w4_quantize(int32_t format, const float *w, int64_t n, int64_t k, uint8_t *codes, void *scales,
                float *global_scale) {
    clear_error();
    int st = check_shape(format, W4_LAYOUT_CANONICAL, 1, n, k);
    if (st) return st;
    if (format == W4_FMT_BF16) {  // plain round to nearest even, no scales
        if (!w || !codes) return fail(W4_ERR_INVALID_ARG, "null pointer");
        for (int64_t i = 0; i < n * k; ++i)
            if (!std::isfinite(w[i])) return fail(W4_ERR_NONFINITE, "non-finite weight at index %lld", (long long)i);
        uint16_t *out = reinterpret_cast<uint16_t *>(codes);
        for (int64_t i = 0; i < n * k; ++i) {
            uint32_t u;
            std::memcpy(&u, &w[i], 4);
            out[i] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
        }
        return W4_OK;
    }
    if (!w || !codes || !scales) return fail(W4_ERR_INVALID_ARG, "null pointer");
    const bool nv = format == W4_FMT_NVFP4_E4M3S16;
    if (nv && !global_scale) return fail(W4_ERR_INVALID_ARG, "NVFP4 needs a global_scale output");
    const int g = group_of(format);
    const float qmax = format == W4_FMT_INT4_F16S128 ? 7.0f : 6.0f;
    // validate everything before writing anything
    const int64_t total = n * k;
    for (int64_t i = 0; i < total; ++i)
        if (!std::isfinite(w[i])) return fail(W4_ERR_NONFINITE, "non-finite weight at index %lld", (long long)i);
    float gscale = 0.f;
    if (nv) {  // UE4M3 block scales saturate; only the global scale is computed here
        float amax = 0.f;
        for (int64_t i = 0; i < total; ++i) amax = std::fmax(amax, std::fabs(w[i]));
        gscale = amax / 2688.0f;  // 6 x 448
        *global_scale = gscale;
    } else if (format != W4_FMT_MXFP4_E8M0S32) {  // E8M0 covers every finite fp32 block
        for (int64_t b = 0; b < total / g; ++b) {
            float a = 0.f;
            for (int i = 0; i < g; ++i) a = std::fmax(a, std::fabs(w[b * g + i]));
            if (!std::isfinite(f16_bits_to_f32(f32_to_f16_bits(a / qmax))))
                return fail(W4_ERR_RANGE, "block %lld: scale %g overflows fp16", (long long)b, (double)(a / qmax));
        }
    }
    // rows are independent: split them over a few host threads for big matrices
    unsigned nt = std::thread::hardware_concurrency();
    nt = nt ? (nt > 16 ? 16 : nt) : 1;
    if (total < (int64_t(1) << 22) || n < (int64_t)nt) nt = 1;
    if (nt == 1) {
        quantize_rows(format, w, 0, n, k, codes, scales, gscale);
    } else {
        std::vector<std::thread> th;
        const int64_t per = (n + nt - 1) / nt;
        for (unsigned t = 0; t < nt; ++t) {
            const int64_t r0 = t * per, r1 = r0 + per < n ? r0 + per : n;
            if (r0 >= r1) break;
            th.emplace_back(quantize_rows, format, w, r0, r1, k, codes, scales, gscale);
        }
        for (auto &t : th) t.join();
    }
    return W4_OK;
}

int w4_pack_nibbles(const uint8_t *nibbles, int64_t n, int64_t k, uint8_t *packed) {
    clear_error();
    if (!nibbles || !packed) return fail(W4_ERR_INVALID_ARG, "null pointer");
    if (n < 1 || k < 2 || (k & 1)) return fail(W4_ERR_INVALID_ARG, "need n >= 1 and even k >= 2");
    const int64_t total = n * k;
    for (int64_t i = 0; i < total; ++i)
        if (nibbles[i] > 15) return fail(W4_ERR_INVALID_ARG, "nibble value %d > 15 at %lld", nibbles[i], (long long)i);
    for (int64_t i = 0; i < total / 2; ++i) packed[i] = (uint8_t)(nibbles[2 * i] | (nibbles[2 * i + 1] << 4));
    return W4_OK;
}

int w4_unpack_nibbles(const uint8_t *packed, int64_t n, int64_t k, uint8_t *nibbles) {
    clear_error();
    if (!nibbles || !packed) return fail(W4_ERR_INVALID_ARG, "null pointer");
    if (n < 1 || k < 2 || (k & 1)) return fail(W4_ERR_INVALID_ARG, "need n >= 1 and even k >= 2");
    const int64_t total = n * k;
    for (int64_t i = 0; i < total / 2; ++i) {
        nibbles[2 * i] = packed[i] & 0xF;
        nibbles[2 * i + 1] = packed[i] >> 4;
    }
    return W4_OK;
}

// Canonical <-> device layouts.  GFX950_V1 stores each row as one record: the
// row's codes (canonical nibble order) followed by its block scales, padded
// with zero bytes to a multiple of 16.  GFX950_KT16 stores each 16-wide K tile
// of a matrix as one record: every row's 8 code bytes of the tile, then every
// row's scale of the tile, padded to 16.  Both directions move bytes only, so
// they are exact inverses for any input (padding excepted).
static int pack_args(int32_t format, int64_t groups, int64_t n, int64_t k, int32_t layout, const void *a,
                     const void *b, const void *c) {
    int st = check_shape(format, layout, groups, n, k);
    if (st) return st;
    if (!a || !c) return fail(W4_ERR_INVALID_ARG, "null codes pointer");
    if (!b && format != W4_FMT_BF16) return fail(W4_ERR_INVALID_ARG, "null scales pointer");
    return W4_OK;
}

int w4_pack(int32_t format, int64_t groups, int64_t n, int64_t k, const uint8_t *codes, const void *scales,
            int32_t dst_layout, uint8_t *codes_out, void *scales_out) {
    clear_error();
    int st = pack_args(format, groups, n, k, dst_layout, codes, scales, codes_out);
    if (st) return st;
    const size_t rows = (size_t)groups * (size_t)n;
    const size_t cb = code_bytes_per_row(format, k), sb = scale_bytes_per_row(format, k);
    if (dst_layout == W4_LAYOUT_CANONICAL) {
        if (sb && !scales_out) return fail(W4_ERR_INVALID_ARG, "null scales_out");
        std::memmove(codes_out, codes, rows * cb);
        if (sb) std::memmove(scales_out, scales, rows * sb);
        return W4_OK;
    }
    const uint8_t *sc = static_cast<const uint8_t *>(scales);
    if (dst_layout == W4_LAYOUT_GFX950_KT16) {
        const size_t ts = kt16_tile_bytes(format, n), ssz = sb / (size_t)(k / 16), nt = (size_t)(k / 16);
        for (size_t g = 0; g < (size_t)groups; ++g)
            for (size_t t = 0; t < nt; ++t) {
                uint8_t *dst = codes_out + (g * nt + t) * ts;
                for (size_t r = 0; r < (size_t)n; ++r) {
                    const size_t row = g * (size_t)n + r;
                    std::memcpy(dst + r * 8, codes + row * cb + t * 8, 8);
                    std::memcpy(dst + (size_t)n * 8 + r * ssz, sc + row * sb + t * ssz, ssz);
                }
                std::memset(dst + (size_t)n * (8 + ssz), 0, ts - (size_t)n * (8 + ssz));
            }
        return W4_OK;
    }
    const size_t rs = v1_row_bytes(format, k);
    for (size_t r = 0; r < rows; ++r) {
        uint8_t *dst = codes_out + r * rs;
        std::memcpy(dst, codes + r * cb, cb);
        if (sb) std::memcpy(dst + cb, sc + r * sb, sb);
        std::memset(dst + cb + sb, 0, rs - cb - sb);
    }
    return W4_OK;
}

int w4_unpack(int32_t format, int64_t groups, int64_t n, int64_t k, int32_t src_layout, const uint8_t *codes_in,
              const void *scales_in, uint8_t *codes, void *scales) {
    clear_error();
    int st = check_shape(format, src_layout, groups, n, k);
    if (st) return st;
    if (!codes_in || !codes) return fail(W4_ERR_INVALID_ARG, "null codes pointer");
    const size_t rows = (size_t)groups * (size_t)n;
    const size_t cb = code_bytes_per_row(format, k), sb = scale_bytes_per_row(format, k);
    if (sb && !scales) return fail(W4_ERR_INVALID_ARG, "null scales output");
    if (src_layout == W4_LAYOUT_CANONICAL) {
        if (sb && !scales_in) return fail(W4_ERR_INVALID_ARG, "null scales_in");
        std::memmove(codes, codes_in, rows * cb);
        if (sb) std::memmove(scales, scales_in, rows * sb);
        return W4_OK;
    }
    uint8_t *sc = static_cast<uint8_t *>(scales);
    if (src_layout == W4_LAYOUT_GFX950_KT16) {
        const size_t ts = kt16_tile_bytes(format, n), ssz = sb / (size_t)(k / 16), nt = (size_t)(k / 16);
        for (size_t g = 0; g < (size_t)groups; ++g)
            for (size_t t = 0; t < nt; ++t) {
                const uint8_t *src = codes_in + (g * nt + t) * ts;
                for (size_t r = 0; r < (size_t)n; ++r) {
                    const size_t row = g * (size_t)n + r;
                    std::memcpy(codes + row * cb + t * 8, src + r * 8, 8);
                    std::memcpy(sc + row * sb + t * ssz, src + (size_t)n * 8 + r * ssz, ssz);
                }
            }
        return W4_OK;
    }
    const size_t rs = v1_row_bytes(format, k);
    for (size_t r = 0; r < rows; ++r) {
        const uint8_t *src = codes_in + r * rs;
        std::memcpy(codes + r * cb, src, cb);
        if (sb) std::memcpy(sc + r * sb, src + cb, sb);
    }
    return W4_OK;
}

}  // extern "C"
