// Decode kernels of an MoE layer whose down projections are K-tiled
// (W4_LAYOUT_GFX950_KT16).  After the router launch, two launches finish the
// layer:
//   k_moe_dec          one block per (token, slot, 16-value slice of the
//                      expert's intermediate): the block ranks the experts
//                      (routed slots), streams its 16 gate and 16 up rows of
//                      W13 and, in the same breath, the K tile of W2 those 16
//                      values multiply (one contiguous record), forms
//                      h = silu(gate) * up in fp32 and writes the tile's fp32
//                      contribution to every output row;
//   k_moe_dec_combine  y = sum over routed slots of w_j * (sum of the slot's
//                      tile contributions) + sigma * (the shared expert's),
//                      tiles and slots summed in a fixed order, one rounding
//                      to bf16.  No float atomics.
// Splitting the down projection over its K dimension (the intermediate) lets a
// block start its W2 loads as soon as it knows its expert instead of after a
// kernel boundary, so the layer's second weight stream overlaps the first.
// Sources: lynn-engine README status notes P28/P29 (gate_up_silu and
// down_weighted_sum contracts), P46/P48 (no float atomics, fixed-order sums),
// P55 (gate and up rows together); tutorials index note 06 (router order).
#include "w4moe_decode.h"
#include "w4moe_device.h"

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <type_traits>

namespace w4k {

template <int FMT, int L, int PL>
__global__ __launch_bounds__(64 * DEC_WAVES) void k_moe_dec(DecArgs a) {
    constexpr int RG = 64 / L;                 // rows of one load group
    constexpr int NLG = RG >= 4 ? 1 : 4 / RG;  // load groups holding the wave's 4 rows
    constexpr int MAXKS = DEC_MAX_H / (32 * L) < 1 ? 1 : (DEC_MAX_H / (32 * L) > 2 ? 2 : DEC_MAX_H / (32 * L));
    constexpr int PAIRS = DEC_MAX_H / 2 / (64 * DEC_WAVES);  // W2 row pairs per thread at most
    __shared__ int s_ids[16];
    __shared__ float s_gu[2 * DEC_TILE];
    __shared__ float4 s_h[DEC_TILE / 4];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    // blocks of a token: the shared expert's tiles first (they need no ranking
    // and start streaming at once), then the routed slots in order
    const int per_tok = a.S * a.tiles;
    const int t = blockIdx.x / per_tok;
    const int rem = blockIdx.x - t * per_tok;
    const int js = rem / a.tiles;
    const int j = a.S > a.K ? (js == 0 ? a.K : js - 1) : js;
    const int tile = rem - js * a.tiles;
    const int H = a.H, I = a.I;
    const int lk = lane % L, rsub = lane / L;
    const int ks = (H + 32 * L - 1) / (32 * L);
    const bool shared = j == a.K;  // uniform per block
    const RowLayout rl = shared ? a.s_rl13 : a.rl13;
    const uint32_t mat13 = (uint32_t)(2 * I) * rl.cs, mats13 = (uint32_t)(2 * I) * rl.ss;
    const uint32_t mat2 = (uint32_t)a.tiles * a.tile_bytes;

    // activations first: they do not depend on the routing
    const Buf xb = make_buf(a.x + (size_t)t * H, (uint32_t)H * 2u);
    XSlice<FMT> xs[MAXKS];
#pragma unroll
    for (int s = 0; s < MAXKS; ++s) {
        const int k0 = 32 * (L * s + lk);
        load_xslice<FMT>(xs[s], xb, (s < ks && k0 < H) ? (uint32_t)k0 * 2u : OOB);
    }

    // which expert: shared slot, ranked once per block, or supplied
    const uint8_t *c13, *s13, *c2;
    const float *g13 = nullptr, *g2 = nullptr;
    bool valid = true;
    if (shared) {
        c13 = a.s_codes13, s13 = static_cast<const uint8_t *>(a.s_scales13), c2 = a.s_codes2;
        g13 = a.s_gs13, g2 = a.s_gs2;
    } else {
        int e;
        if (a.route) {
            if (wv == 0) {
                const bool writer = (j == 0 && tile == 0);
                int my_id;
                float my_val;
                wave_topk<PL>(a.logits + (size_t)t * a.lstride, a.bias, a.E, writer ? a.K : j + 1, j, my_id, my_val);
                if (lane <= j) s_ids[lane] = my_id;
                if (writer) {
                    // weights = softmax over the k selected logits (lane 0 holds the
                    // largest); the sum runs in a fixed lane order
                    const float vmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_val), 0));
                    const float ex = lane < a.K ? expf(my_val - vmax) : 0.f;
                    const float sum = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(group_sum<64>(ex)), 63));
                    if (lane < a.K) {
                        const float w = ex / sum;
                        a.ids_ws[t * a.K + lane] = my_id;
                        a.w_ws[t * a.K + lane] = w;
                        if (a.ids_user) a.ids_user[t * a.K + lane] = my_id;
                        if (a.w_user) a.w_user[t * a.K + lane] = w;
                    }
                }
            }
            __syncthreads();
            e = __builtin_amdgcn_readfirstlane(s_ids[j]);
        } else {
            e = ld_uniform(a.ids_in, t * a.K + j);
        }
        valid = e >= 0 && e < a.E;  // an id out of range reads nothing and poisons the slot
        const int eo = valid ? e : 0;
        c13 = a.codes13 + (size_t)eo * mat13;
        s13 = static_cast<const uint8_t *>(a.scales13) + (size_t)eo * mats13;
        c2 = a.codes2 + (size_t)eo * mat2;
        if (a.gs13) g13 = a.gs13 + eo;
        if (a.gs2) g2 = a.gs2 + eo;
    }

    // the slice's W2 tile: row pairs (2p, 2p+1) of the record, codes then scales
    const Buf cb2 = make_buf(c2 + (size_t)tile * a.tile_bytes, valid ? a.tile_bytes : 0u);
    const int npairs = H >> 1;
    uint4 w2c[PAIRS];
    uint32_t w2s[PAIRS];
#pragma unroll
    for (int q = 0; q < PAIRS; ++q) {
        const int p = tid + 64 * DEC_WAVES * q;
        const bool v = p < npairs;
        w2c[q] = ld128(cb2, v ? 16u * (uint32_t)p : OOB);
        if constexpr (FMT == FMT_NVFP4)
            w2s[q] = ld16(cb2, v ? (uint32_t)H * 8u + 2u * (uint32_t)p : OOB);
        else
            w2s[q] = ld32(cb2, v ? (uint32_t)H * 8u + 4u * (uint32_t)p : OOB);
    }

    // the wave's gate rows i0 + 2 wv + {0, 1} and the matching up rows
    const Buf cb = make_buf(c13, valid ? mat13 : 0u);
    const Buf sb = make_buf(s13, valid ? mats13 : 0u);
    const int i0 = tile * DEC_TILE + 2 * wv;
    float acc[NLG];
#pragma unroll
    for (int l = 0; l < NLG; ++l) acc[l] = 0.f;
#pragma unroll
    for (int s = 0; s < MAXKS; ++s) {
        if (s >= ks) break;
        const int k0 = 32 * (L * s + lk);
        const bool kv = k0 < H;
        uint4 cw[NLG];
        uint32_t sw[NLG];
#pragma unroll
        for (int l = 0; l < NLG; ++l) {
            const int q = l * RG + rsub;
            const uint32_t row = (uint32_t)(q < 2 ? i0 + q : I + i0 + q - 2);
            const bool v = kv && q < 4;
            cw[l] = ld128(cb, v ? row * rl.cs + (uint32_t)(k0 >> 1) : OOB);
            sw[l] = ld_scales<FMT>(sb, v ? row * rl.ss + scale_col<FMT>(k0) : OOB);
        }
        prep_xslice<FMT>(xs[s]);
#pragma unroll
        for (int l = 0; l < NLG; ++l) acc[l] = chunk_dot_bf16<FMT>(cw[l], sw[l], xs[s], acc[l]);
    }
    float g1 = 1.f;
    if constexpr (FMT == FMT_NVFP4) g1 = ld_uniform(g13, 0);
#pragma unroll
    for (int l = 0; l < NLG; ++l) {
        const float v = group_sum<L>(acc[l]) * g1;
        const int q = l * RG + rsub;
        if (group_leader<L>(lane) && q < 4) s_gu[(q < 2 ? 0 : DEC_TILE) + 2 * wv + (q & 1)] = v;
    }
    __syncthreads();
    if (tid < DEC_TILE) {
        const float g = s_gu[tid], u = s_gu[DEC_TILE + tid];
        reinterpret_cast<float *>(s_h)[tid] = valid ? (g / (1.f + expf(-g))) * u : __builtin_nanf("");
    }
    __syncthreads();
    float4 hq[DEC_TILE / 4];
#pragma unroll
    for (int i = 0; i < DEC_TILE / 4; ++i) hq[i] = s_h[i];
    const float *h = reinterpret_cast<const float *>(hq);

    // the tile's contribution to every output row: 16 codes x h, times the row's
    // scale of the tile (NVFP4: times the matrix's global scale)
    float g2s = 1.f;
    if constexpr (FMT == FMT_NVFP4) g2s = ld_uniform(g2, 0);
    float *out = a.part + (((size_t)t * a.S + j) * a.tiles + tile) * H;
#pragma unroll
    for (int q = 0; q < PAIRS; ++q) {
        const int p = tid + 64 * DEC_WAVES * q;
        if (p >= npairs) break;
        const uint32_t cw4[4] = {w2c[q].x, w2c[q].y, w2c[q].z, w2c[q].w};
        float d[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            float v = 0.f;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const uint32_t c = cw4[2 * r + m];
                f32x2 wv2;
                wv2 = e2m1x2_f32<0>(c); v = fmaf(wv2.x, h[8 * m + 0], v); v = fmaf(wv2.y, h[8 * m + 1], v);
                wv2 = e2m1x2_f32<1>(c); v = fmaf(wv2.x, h[8 * m + 2], v); v = fmaf(wv2.y, h[8 * m + 3], v);
                wv2 = e2m1x2_f32<2>(c); v = fmaf(wv2.x, h[8 * m + 4], v); v = fmaf(wv2.y, h[8 * m + 5], v);
                wv2 = e2m1x2_f32<3>(c); v = fmaf(wv2.x, h[8 * m + 6], v); v = fmaf(wv2.y, h[8 * m + 7], v);
            }
            d[r] = v;
        }
        const f32x2 sc = block_scales2<FMT>(w2s[q]);
        *reinterpret_cast<float2 *>(out + 2 * p) = make_float2(d[0] * sc.x * g2s, d[1] * sc.y * g2s);
    }
}

// y[t][r] = sum_j w[t][j] (sum_tile part[t][j][tile][r]) + sigma_t (sum_tile
// part[t][K][tile][r]).  Thread (column of 4 rows c, slot j, tile group q)
// sums tiles 8q .. 8q+7 of its slot in order (its coefficient is loaded with
// them); the groups of a slot are then added in order and scaled, and the
// slots added in order, through LDS; one rounding to bf16.
__global__ __launch_bounds__(1024) void k_moe_dec_combine(DecCombineArgs a) {
    extern __shared__ float4 red[];  // [S][G8][cols], then [S][cols]
    const int G8 = (a.tiles + 7) >> 3;
    const int cols = blockDim.x / (a.S * G8);
    const int tid = threadIdx.x;
    const int c = tid % cols, rest = tid / cols;
    const int q = rest % G8, j = rest / G8;
    const int ncol4 = a.H >> 2;
    const int t = blockIdx.y;
    const int col = blockIdx.x * cols + c;
    float coef = 0.f;
    if (q == 0)
        coef = j < a.K ? a.w[t * a.K + j] : 1.f / (1.f + expf(-a.logits[(size_t)t * a.lstride + a.E]));
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (col < ncol4) {
        const float4 *base = reinterpret_cast<const float4 *>(a.part + ((size_t)t * a.S + j) * a.tiles * a.H) + col;
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int tt = 8 * q + u;
            v[u] = tt < a.tiles ? base[(size_t)tt * ncol4] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) s.x += v[u].x, s.y += v[u].y, s.z += v[u].z, s.w += v[u].w;
    }
    red[(j * G8 + q) * cols + c] = s;
    __syncthreads();
    float4 *slot = red + a.S * G8 * cols;
    if (q == 0) {
        float4 sj = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int qq = 0; qq < G8; ++qq) {
            const float4 r = red[(j * G8 + qq) * cols + c];
            sj.x += r.x, sj.y += r.y, sj.z += r.z, sj.w += r.w;
        }
        slot[j * cols + c] = make_float4(coef * sj.x, coef * sj.y, coef * sj.z, coef * sj.w);
    }
    __syncthreads();
    if (rest != 0 || col >= ncol4) return;
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int jj = 0; jj < a.S; ++jj) {
        const float4 r = slot[jj * cols + c];
        y.x += r.x, y.y += r.y, y.z += r.z, y.w += r.w;
    }
    uint16_t *o = a.y + (size_t)t * a.H + 4 * col;
    const uint32_t lo = f32_to_bf16_rne(y.x) | ((uint32_t)f32_to_bf16_rne(y.y) << 16);
    const uint32_t hi = f32_to_bf16_rne(y.z) | ((uint32_t)f32_to_bf16_rne(y.w) << 16);
    *reinterpret_cast<uint2 *>(o) = make_uint2(lo, hi);
}

// ---------------------------------------------------------------- launchers

namespace {
template <typename F, typename... Args>
void go_ev(hipStream_t st, hipEvent_t e0, hipEvent_t e1, F kernel, dim3 g, dim3 b, uint32_t shm, Args... args) {
    if (e0)
        hipExtLaunchKernelGGL(kernel, g, b, shm, st, e0, e1, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, g, b, shm, st, args...);
}

int lanes_of(int k) {
    int need = (k + 31) / 32, L = 1;
    while (L < need && L < 64) L <<= 1;
    return L;
}
}  // namespace

void launch_dec(DecArgs &a, int fmt, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    const dim3 g((unsigned)(a.T * a.S * a.tiles)), b(64 * DEC_WAVES);
    const int pl = (a.E + 63) / 64;
    auto with = [&](auto F, auto Lc) {
        constexpr int FM = decltype(F)::value, L = decltype(Lc)::value;
        if (pl <= 1) go_ev(st, e0, e1, k_moe_dec<FM, L, 1>, g, b, 0, a);
        else if (pl <= 2) go_ev(st, e0, e1, k_moe_dec<FM, L, 2>, g, b, 0, a);
        else if (pl <= 4) go_ev(st, e0, e1, k_moe_dec<FM, L, 4>, g, b, 0, a);
        else if (pl <= 8) go_ev(st, e0, e1, k_moe_dec<FM, L, 8>, g, b, 0, a);
        else go_ev(st, e0, e1, k_moe_dec<FM, L, 16>, g, b, 0, a);
    };
    auto with_fmt = [&](auto F) {
        switch (lanes_of(a.H)) {
        case 1: case 2: case 4: case 8: with(F, std::integral_constant<int, 8>()); break;
        case 16: with(F, std::integral_constant<int, 16>()); break;
        case 32: with(F, std::integral_constant<int, 32>()); break;
        default: with(F, std::integral_constant<int, 64>()); break;
        }
    };
    if (fmt == FMT_NVFP4) with_fmt(std::integral_constant<int, FMT_NVFP4>());
    else with_fmt(std::integral_constant<int, FMT_E2M1>());
}

void launch_dec_combine(DecCombineArgs &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    const int G8 = (a.tiles + 7) / 8;
    int cols = 1;  // columns of 4 output rows per block: up to 4, so that the grid spreads over the chip
    while (cols * 2 <= 4 && cols * 2 * a.S * G8 <= 1024) cols *= 2;
    const int ncol4 = a.H / 4;
    const dim3 g((unsigned)((ncol4 + cols - 1) / cols), (unsigned)a.T), b((unsigned)(cols * a.S * G8));
    go_ev(st, e0, e1, k_moe_dec_combine, g, b, (uint32_t)(cols * a.S * (G8 + 1) * sizeof(float4)), a);
}

}  // namespace w4k
