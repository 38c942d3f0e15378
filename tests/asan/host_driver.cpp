// Host-only driver of the w4moe host code (quantisers, layouts, sizes and
// every validation path), built with AddressSanitizer by test_host_asan.py.
// Exits non-zero on a wrong status or a failed round trip; ASan aborts on any
// out-of-bounds access, use after free or leak.
#include "w4moe.h"

#include <cmath>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

static int failures = 0;
#define EXPECT(cond)                                                          \
    do {                                                                      \
        if (!(cond)) {                                                        \
            std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

static const int32_t FMTS[] = {W4_FMT_E2M1_F16S16, W4_FMT_INT4_F16S128, W4_FMT_NVFP4_E4M3S16, W4_FMT_MXFP4_E8M0S32};

static size_t scale_elem(int32_t f) { return (f == W4_FMT_NVFP4_E4M3S16 || f == W4_FMT_MXFP4_E8M0S32) ? 1 : 2; }
static int64_t group(int32_t f) { return f == W4_FMT_INT4_F16S128 ? 128 : f == W4_FMT_MXFP4_E8M0S32 ? 32 : 16; }

// quantise (exact-size buffers, so any overrun is caught), then pack and unpack
// in every device layout the format has
static void quantise_and_layouts(int32_t fmt, int64_t n, int64_t k, std::mt19937 &rng) {
    std::normal_distribution<float> nd(0.f, 0.02f);
    std::vector<float> w((size_t)(n * k));
    for (auto &v : w) v = nd(rng);
    const size_t cb = w4_codes_bytes(fmt, W4_LAYOUT_CANONICAL, 1, n, k);
    const size_t sb = w4_scales_bytes(fmt, W4_LAYOUT_CANONICAL, 1, n, k);
    EXPECT(cb == (size_t)(n * k / 2));
    EXPECT(sb == (size_t)(n * (k / group(fmt))) * scale_elem(fmt));
    std::vector<uint8_t> codes(cb), scales(sb);
    float g = 0.f;
    EXPECT(w4_quantize(fmt, w.data(), n, k, codes.data(), scales.data(), &g) == W4_OK);
    const int32_t layouts[] = {W4_LAYOUT_CANONICAL, W4_LAYOUT_GFX950_V1, W4_LAYOUT_GFX950_KT16};
    for (int32_t lay : layouts) {
        const size_t rb = w4_codes_bytes(fmt, lay, 1, n, k);
        if (rb == 0) {  // a layout this format does not have
            EXPECT(lay == W4_LAYOUT_GFX950_KT16 && fmt != W4_FMT_E2M1_F16S16 && fmt != W4_FMT_NVFP4_E4M3S16);
            continue;
        }
        const size_t rs = w4_scales_bytes(fmt, lay, 1, n, k);
        std::vector<uint8_t> rec(rb), rsc(rs ? rs : 1);
        EXPECT(w4_pack(fmt, 1, n, k, codes.data(), scales.data(), lay, rec.data(), rs ? rsc.data() : nullptr) == W4_OK);
        std::vector<uint8_t> c2(cb), s2(sb);
        EXPECT(w4_unpack(fmt, 1, n, k, lay, rec.data(), rs ? rsc.data() : nullptr, c2.data(), s2.data()) == W4_OK);
        EXPECT(c2 == codes && s2 == scales);
    }
}

int main() {
    std::mt19937 rng(7);
    // small shapes and one large enough for the threaded quantiser (>= 2^22 elements)
    for (int32_t f : FMTS) {
        quantise_and_layouts(f, 3, 256, rng);
        quantise_and_layouts(f, 37, 384 + (f == W4_FMT_INT4_F16S128 ? 0 : 32), rng);
    }
    quantise_and_layouts(W4_FMT_E2M1_F16S16, 2048, 2048, rng);
    quantise_and_layouts(W4_FMT_INT4_F16S128, 2048, 2048, rng);
    quantise_and_layouts(W4_FMT_NVFP4_E4M3S16, 2048, 2048, rng);
    {  // bf16 rows: no scales; both row layouts coincide
        std::vector<float> w(64 * 64, 0.5f);
        std::vector<uint16_t> bits(64 * 64);
        EXPECT(w4_quantize(W4_FMT_BF16, w.data(), 64, 64, reinterpret_cast<uint8_t *>(bits.data()), nullptr, nullptr) == W4_OK);
        EXPECT(w4_codes_bytes(W4_FMT_BF16, W4_LAYOUT_GFX950_V1, 1, 64, 64) == 64 * 64 * 2);
    }
    // validation paths: nothing may be written, no access out of bounds
    std::vector<float> w(16 * 32, 1.f);
    std::vector<uint8_t> c(16 * 16), s(16 * 2 * 2);
    float g = 0.f;
    EXPECT(w4_quantize(99, w.data(), 16, 32, c.data(), s.data(), &g) == W4_ERR_LAYOUT);
    EXPECT(w4_quantize(W4_FMT_E2M1_F16S16, w.data(), 16, 30, c.data(), s.data(), &g) == W4_ERR_INVALID_ARG);
    EXPECT(w4_quantize(W4_FMT_E2M1_F16S16, nullptr, 16, 32, c.data(), s.data(), &g) == W4_ERR_INVALID_ARG);
    EXPECT(w4_quantize(W4_FMT_NVFP4_E4M3S16, w.data(), 16, 32, c.data(), s.data(), nullptr) == W4_ERR_INVALID_ARG);
    w[5] = NAN;
    EXPECT(w4_quantize(W4_FMT_E2M1_F16S16, w.data(), 16, 32, c.data(), s.data(), &g) == W4_ERR_NONFINITE);
    w[5] = 1e9f;
    EXPECT(w4_quantize(W4_FMT_E2M1_F16S16, w.data(), 16, 32, c.data(), s.data(), &g) == W4_ERR_RANGE);
    EXPECT(w4_pack(W4_FMT_E2M1_F16S16, 1, 16, 32, c.data(), s.data(), 7, c.data(), nullptr) == W4_ERR_LAYOUT);
    EXPECT(w4_pack(W4_FMT_INT4_F16S128, 1, 16, 128, c.data(), s.data(), W4_LAYOUT_GFX950_KT16, c.data(), nullptr) ==
           W4_ERR_UNSUPPORTED);
    EXPECT(w4_unpack(W4_FMT_E2M1_F16S16, 1, 16, 32, W4_LAYOUT_GFX950_V1, nullptr, nullptr, c.data(), s.data()) ==
           W4_ERR_INVALID_ARG);
    std::vector<uint8_t> nib(4 * 8, 16);
    std::vector<uint8_t> packed(4 * 4);
    EXPECT(w4_pack_nibbles(nib.data(), 4, 8, packed.data()) == W4_ERR_INVALID_ARG);
    EXPECT(w4_unpack_nibbles(packed.data(), 4, 7, nib.data()) == W4_ERR_INVALID_ARG);
    EXPECT(std::strlen(w4_last_error()) > 0);
    EXPECT(std::strcmp(w4_status_string(W4_ERR_RANGE), "W4_ERR_RANGE") == 0);
    if (failures) return 1;
    std::printf("host code under ASan: ok\n");
    return 0;
}
