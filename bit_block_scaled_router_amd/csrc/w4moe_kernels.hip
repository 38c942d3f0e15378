// gfx950 kernels and device entry points of the w4moe C ABI (include/w4moe.h).
//
// The MoE decode layer runs as three launches on the caller's stream, with no
// host synchronisation:
//   k_router   router GEMV logits = Wr x (bf16 weights, fp32 accumulate) plus the
//              shared-expert gate dot, one wave per row;
//   k_moe_w13  one launch over every (token, slot, row tile): slot j < k is the
//              j-th routed expert, slot k the shared expert.  Each wave finds its
//              expert by ranking the logits itself (softmax over all experts ->
//              top-k -> renormalise, evaluated as softmax over the k selected
//              logits), streams gate row i and up row i of that expert's packed
//              W13 together, and writes h = silu(gate) * up in fp32;
//   k_moe_down one launch; a block owns a tile of output rows of one token, its
//              waves take the slots, each dot is scaled by its routing weight (or
//              the shared gate sigma) and the block sums the slots in slot order
//              through LDS before one rounding to bf16.  No float atomics.
// Sources: lynn-engine tutorials index note 06 (router order, sigmoid-gated
// shared expert); lynn-engine README status notes P28 (gate/up + SiLU over a
// grouped packed tensor with top-k ids), P29 (down weighted sum), P45 (one-call
// shape), P46/P48 (atomics drift; row-owning down kernel), P55 (gate and up rows
// processed together); "Lynn Engine" article stage P1 (packed matvec).
#include "w4moe_decode.h"
#include "w4moe_device.h"
#include "w4moe_grouped.h"
#include "w4moe_internal.h"

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

namespace w4k {

// ================================================================= dense GEMV

// y[t][n] = sum_k W[n][k] x[t][k].  A wave owns RT load-groups of 64/L rows and
// issues all of its weight loads before the first use.
// NVFP4: the row sums are multiplied by the matrix's global scale *gsc.
template <int FMT, int L, int RT>
__global__ __launch_bounds__(256) void k_gemv(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                              const float *__restrict__ gsc, const uint16_t *__restrict__ x,
                                              uint16_t *__restrict__ y, int n, int k, int m, uint32_t cs,
                                              uint32_t ss) {
    constexpr int RG = 64 / L;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int lk = lane % L, rsub = lane / L;
    const int row0 = wave * RT * RG;
    if (row0 >= n) return;  // uniform per wave
    const int ks = (k + 32 * L - 1) / (32 * L);
    const Buf cb = make_buf(codes, (uint32_t)n * cs);
    const Buf sb = make_buf(scales, (uint32_t)n * ss);
    const Buf xb = make_buf(x, (uint32_t)m * (uint32_t)k * 2u);
    float g = 1.f;
    if constexpr (FMT == FMT_NVFP4) g = ld_uniform(gsc, 0);
    for (int t = 0; t < m; ++t) {
        float acc[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r] = 0.f;
        for (int s = 0; s < ks; ++s) {
            const int k0 = 32 * (L * s + lk);
            const bool kv = k0 < k;
            XSlice<FMT> xs;  // activations first: they return from cache before the weights
            load_xslice<FMT>(xs, xb, kv ? (uint32_t)(t * k + k0) * 2u : OOB);
            uint4 cw[RT];
            uint32_t sw[RT];
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const int row = row0 + r * RG + rsub;
                const bool v = kv && row < n;
                cw[r] = ld128(cb, v ? (uint32_t)row * cs + (uint32_t)(k0 >> 1) : OOB);
                sw[r] = ld_scales<FMT>(sb, v ? (uint32_t)row * ss + scale_col<FMT>(k0) : OOB);
            }
            prep_xslice<FMT>(xs);
#pragma unroll
            for (int r = 0; r < RT; ++r) acc[r] = chunk_dot_bf16<FMT>(cw[r], sw[r], xs, acc[r]);
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            float v = group_sum<L>(acc[r]);
            if constexpr (FMT == FMT_NVFP4) v *= g;
            const int row = row0 + r * RG + rsub;
            if (group_leader<L>(lane) && row < n) y[(size_t)t * n + row] = f32_to_bf16_rne(v);
        }
    }
}

// ================================================================= dequant hook

// out[row][k] = value(code) * fp32(scale), with the bf16 decode the GEMV uses
// (NVFP4: times the global scale of the row's matrix, gsc[row / n]).
template <int FMT, int L>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                                 const float *__restrict__ gsc, float *__restrict__ out, int64_t rows,
                                                 int64_t n, int k, uint32_t cs, uint32_t ss) {
    constexpr int RG = 64 / L;
    const int lane = threadIdx.x & 63;
    const int64_t wave = wave_id();
    const int lk = lane % L;
    const int64_t row0 = wave * RG;  // wave-uniform
    if (row0 >= rows) return;
    const int64_t row = row0 + lane / L;
    const bool rv = row < rows;
    const int64_t nrows = rows - row0 < RG ? rows - row0 : RG;
    const Buf cb = make_buf(codes + row0 * cs, (uint32_t)(nrows * cs));
    const Buf sb = make_buf(scales + row0 * ss, (uint32_t)(nrows * ss));
    const uint32_t rl = (uint32_t)(lane / L);
    float g = 1.f;
    if constexpr (FMT == FMT_NVFP4) g = rv ? gsc[row / n] : 0.f;
    for (int k0 = 32 * lk; k0 < k; k0 += 32 * L) {
        const uint4 c = ld128(cb, rv ? rl * cs + (uint32_t)(k0 >> 1) : OOB);
        const uint32_t sc = ld_scales<FMT>(sb, rv ? rl * ss + scale_col<FMT>(k0) : OOB);
        const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
        float v[32];
        if constexpr (FMT != FMT_INT4) {
            const f32x2 s2 = block_scales2<FMT>(sc);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const float s = d < 2 ? s2.x : s2.y;
                bf16x2 p;
                p = e2m1x2_bf16<0>(cw[d]); v[8 * d + 0] = (float)p.x * s; v[8 * d + 1] = (float)p.y * s;
                p = e2m1x2_bf16<1>(cw[d]); v[8 * d + 2] = (float)p.x * s; v[8 * d + 3] = (float)p.y * s;
                p = e2m1x2_bf16<2>(cw[d]); v[8 * d + 4] = (float)p.x * s; v[8 * d + 5] = (float)p.y * s;
                p = e2m1x2_bf16<3>(cw[d]); v[8 * d + 6] = (float)p.x * s; v[8 * d + 7] = (float)p.y * s;
            }
        } else {
            const float s = f16_bits_to_f32(sc);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t lo, hi;
                int4_split(cw[d], lo, hi);
                bf16x2 p;
                p = u4x2_bf16<false>(lo); v[8 * d + 0] = ((float)p.x - 8.f) * s; v[8 * d + 2] = ((float)p.y - 8.f) * s;
                p = u4x2_bf16<true>(lo);  v[8 * d + 4] = ((float)p.x - 8.f) * s; v[8 * d + 6] = ((float)p.y - 8.f) * s;
                p = u4x2_bf16<false>(hi); v[8 * d + 1] = ((float)p.x - 8.f) * s; v[8 * d + 3] = ((float)p.y - 8.f) * s;
                p = u4x2_bf16<true>(hi);  v[8 * d + 5] = ((float)p.x - 8.f) * s; v[8 * d + 7] = ((float)p.y - 8.f) * s;
            }
        }
        if constexpr (FMT == FMT_NVFP4) {
#pragma unroll
            for (int i = 0; i < 32; ++i) v[i] *= g;  // code * scale is exact: one rounding
        }
        if (rv) {
            float4 *o = reinterpret_cast<float4 *>(out + row * k + k0);
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
        }
    }
}

// ================================================================= streaming-read probe

// Reads bytes [0, n16 * 16) of src with 128-bit loads, UNROLL per thread in
// flight, grid-stride; the block's XOR of everything read is stored to *sink
// only if it equals an improbable constant, so the loads cannot be dropped and
// nothing else is written.  A measurement aid: the box's practical ceiling for
// a plain read of a given size, beside which the kernels' bandwidths are read.
template <int UNROLL>
__global__ __launch_bounds__(256) void k_stream_read(const uint4 *__restrict__ src, size_t n16,
                                                     uint32_t *__restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
        uint4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u) *sink = acc;
}

// ================================================================= router

// logits[t][r] for rows r in [r_begin, r_begin + gridDim.x) of the stacked
// [E routed rows; 1 shared-gate row]: one block per row; its waves take the
// tokens in chunks of TB (wave w: chunks w, w + nw, ...), so the row's weights
// are fetched from HBM once per block and served to the other waves by the
// cache.  Lane l covers elements 8l + 512s; NS = number of 512-element steps
// (H <= 512 * NS).  The activations of a chunk are loaded before its first dot.
template <int NS, int TB>
__global__ __launch_bounds__(512) void k_router(const uint16_t *__restrict__ wr, const uint16_t *__restrict__ wsg,
                                                const uint16_t *__restrict__ x, float *__restrict__ logits, int E,
                                                int H, int T, int r_begin, int lstride, int32_t *arrive) {
    const int lane = threadIdx.x & 63;
    if (arrive && blockIdx.x == 0 && threadIdx.x == 0) *arrive = 0;  // the grouping launch's arrival counter
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nw = blockDim.x >> 6;
    const int r = r_begin + blockIdx.x;
    const Buf wb = make_buf(r < E ? wr + (size_t)r * H : wsg, (uint32_t)H * 2u);
    const Buf xb = make_buf(x, (uint32_t)T * (uint32_t)H * 2u);
    uint4 w[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int e0 = 8 * lane + 512 * s;
        w[s] = ld128(wb, e0 < H ? (uint32_t)e0 * 2u : OOB);
    }
    for (int t0 = wv * TB; t0 < T; t0 += nw * TB) {
        uint4 xv[TB][NS];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int e0 = 8 * lane + 512 * s;
                xv[tb][s] = ld128(xb, (e0 < H && t0 + tb < T) ? (uint32_t)((t0 + tb) * H + e0) * 2u : OOB);
            }
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            float acc = 0.f;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                acc = dot2(as_bf16x2(w[s].x), xv[tb][s].x, acc);
                acc = dot2(as_bf16x2(w[s].y), xv[tb][s].y, acc);
                acc = dot2(as_bf16x2(w[s].z), xv[tb][s].z, acc);
                acc = dot2(as_bf16x2(w[s].w), xv[tb][s].w, acc);
            }
            acc = group_sum<64>(acc);
            if (group_leader<64>(lane) && t0 + tb < T) logits[(size_t)(t0 + tb) * lstride + r] = acc;
        }
    }
}

// Large batches: the router as a bf16 GEMM on MFMA, logits[t][r] = Wr[r] . x[t]
// for rows r_begin <= r < r_end (row E = the shared-gate weight).  A block
// covers 16 rows x 64 tokens (four 16-token MFMA column tiles); its 4 waves
// split K into quarters (16x16x32 MFMAs, the next 128-wide chunk loaded while
// the current one is multiplied) and the partial sums are added in wave order
// through LDS.  Every x tile is read by ceil(rows / 16) blocks and every router
// row by ceil(T / 64), instead of all T tokens per row as in k_router.
template <int NT>
__global__ __launch_bounds__(256) void k_router_mfma(const uint16_t *__restrict__ wr,
                                                     const uint16_t *__restrict__ wsg,
                                                     const uint16_t *__restrict__ x, float *__restrict__ logits,
                                                     int E, int H, int T, int r_begin, int r_end, int lstride,
                                                     int32_t *arrive) {
    __shared__ float red[3][16][64];
    // the arrival counter of the grouping launch that follows
    if (arrive && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *arrive = 0;
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, q = lane >> 4;
    const int row0 = r_begin + (int)blockIdx.y * 16;
    const int row = row0 + r;  // this lane's A row
    const int tok0 = (int)blockIdx.x * (16 * NT);
    const Buf wb = make_buf(wr, (uint32_t)E * (uint32_t)H * 2u);
    const Buf gb = make_buf(wsg, wsg ? (uint32_t)H * 2u : 0u);
    const Buf xb = make_buf(x, (uint32_t)T * (uint32_t)H * 2u);
    const bool in_wr = row < E && row < r_end, in_g = row == E && row < r_end;
    const uint32_t aoff = (uint32_t)row * (uint32_t)H * 2u;
    uint32_t xoff[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int t = tok0 + 16 * nt + r;
        xoff[nt] = t < T ? (uint32_t)t * (uint32_t)H * 2u : OOB;
    }
    // this wave's K range: chunks of 128 dealt round-robin
    auto load = [&](int k0, uint4 (&av)[4], uint4 (&bv)[4][NT]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t kb = (uint32_t)(k0 + 32 * s + 8 * q) * 2u;
            const bool kv = k0 >= 0 && k0 + 32 * s < H;
            const uint4 u = ld128(wb, (in_wr && kv) ? aoff + kb : OOB);
            const uint4 v = ld128(gb, (in_g && kv) ? kb : OOB);
            av[s] = make_uint4(u.x | v.x, u.y | v.y, u.z | v.z, u.w | v.w);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bv[s][nt] = ld128(xb, (kv && xoff[nt] != OOB) ? xoff[nt] + kb : OOB);
        }
    };
    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint4 av[4], bv[4][NT];
    int k0 = 128 * wv;
    load(k0 < H ? k0 : -1, av, bv);
    for (; k0 < H; k0 += 512) {
        uint4 ac[4], bc[4][NT];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            ac[s] = av[s];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bc[s][nt] = bv[s][nt];
        }
        if (k0 + 512 < H) load(k0 + 512, av, bv);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[nt] = mfma16x16x32(__builtin_bit_cast(bf16x8, ac[s]), __builtin_bit_cast(bf16x8, bc[s][nt]), acc[nt]);
    }
    if (wv > 0) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int j = 0; j < 4; ++j) red[wv - 1][nt * 4 + j][lane] = acc[nt][j];
    }
    __syncthreads();
    if (wv == 0) {
        // lane holds rows 4q + j, token column r of each tile
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int t = tok0 + 16 * nt + r;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float v = acc[nt][j];
#pragma unroll
                for (int w = 0; w < 3; ++w) v += red[w][nt * 4 + j][lane];
                const int rr = row0 + 4 * q + j;
                if (t < T && rr < r_end) logits[(size_t)t * lstride + rr] = v;
            }
        }
    }
}

// ================================================================= MoE W13 + SiLU

struct W13Args {
    const uint8_t *codes;         // routed W13 [E][2I][H/2]
    const uint8_t *scales;        // routed W13 scales (bytes)
    const uint8_t *s_codes;       // shared W13 [2I][H/2] (or null)
    const uint8_t *s_scales;
    const uint16_t *x;            // [T][H]
    const float *logits;          // [T][lstride] (routed mode)
    const float *bias;            // [E] or null
    const int32_t *ids_in;        // [T][k] (supplied mode)
    int32_t *ids_ws;              // [T][k] routing outputs for k_moe_down
    float *w_ws;                  // [T][k]
    int32_t *ids_user;            // optional copies for the caller
    float *w_user;
    float *h;                     // [T][S][hstride] fp32, order of the down kernel's lanes
    int H, I, E, K, S, T, tiles, lstride, hstride, route;
    int L2;                       // lanes per row of the down kernel (h order)
    // (fields of the format variants last: the fields above keep the argument
    // offsets the prologue's first loads were tuned for, ~0.25 us per step)
    int s_bf16;                   // shared expert in bf16 (s_codes = bf16 [2I][H])
    const float *gs, *s_gs;       // NVFP4 global scales: routed [E], shared [1]
    RowLayout rl, s_rl;           // row strides of the routed and shared matrices
};

// h index of intermediate element i in the down kernel's lane order: lane lk of
// step s reads 8 consecutive float4 q = 0..7, so element 32(L2 s + lk) + 4q + c
// sits at s*32*L2 + (q*L2 + lk)*4 + c.
__device__ __forceinline__ int h_index(int i, int L2) {
    const int span = 32 * L2;
    const int s = i / span, rem = i - s * span;
    const int lk = rem >> 5, q = (rem & 31) >> 2, c = rem & 3;
    return s * span + (q * L2 + lk) * 4 + c;
}

// Blocks are laid out so that all WPB waves of a block work on one (token,
// slot): block b covers tiles [tb*WPB, tb*WPB + WPB) of slot j of token t.  For
// a routed slot, wave 0 of the block ranks the experts once and publishes the
// ids through LDS; the block's writer (token t, slot 0, first tile block) also
// stores the routing weights for the down kernel and the caller.  SBF: the
// layer's shared expert is bf16 (its slot streams bf16 rows; a separate
// instantiation so that 4-bit-only layers keep the smaller register budget).
template <int FMT, int L, int RT, int PL, bool SBF>
__global__ __launch_bounds__(1024) void k_moe_w13(W13Args a) {
    constexpr int RG = 64 / L;
    __shared__ int s_ids[16];
    const int lane = threadIdx.x & 63;
    const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave in block
    const int wpb = blockDim.x >> 6;
    const int tblocks = (a.tiles + wpb - 1) / wpb;  // tile blocks per slot
    const int b = blockIdx.x;
    const int t = b / (a.S * tblocks);
    const int rem = b - t * (a.S * tblocks);
    const int j = rem / tblocks;
    const int tb = rem - j * tblocks;
    const int tile = tb * wpb + wib;
    const bool tile_ok = tile < a.tiles;
    const int lk = lane % L, rsub = lane / L;
    const int H = a.H, I = a.I;
    const int ks = (H + 32 * L - 1) / (32 * L);
    // row strides of this slot's matrix (the shared expert may use another layout)
    const uint32_t cs = j == a.K ? a.s_rl.cs : a.rl.cs, ss = j == a.K ? a.s_rl.ss : a.rl.ss;
    const uint32_t mat_codes = (uint32_t)(2 * I) * cs;
    const uint32_t mat_scales = (uint32_t)(2 * I) * ss;
    const Buf xb = make_buf(a.x + (size_t)t * H, (uint32_t)H * 2u);
    XSlice<FMT> xs0;  // step-0 activations, in flight while the experts are ranked
    load_xslice<FMT>(xs0, xb, 32 * lk < H ? (uint32_t)(32 * lk) * 2u : OOB);

    // which expert: shared slot, ranked once per block, or supplied
    const uint8_t *cbase;
    const uint8_t *sbase;
    const float *gp = nullptr;  // NVFP4 global scale of the expert's matrix
    bool valid = true;
    if (j == a.K) {
        cbase = a.s_codes;
        sbase = a.s_scales;
        gp = a.s_gs;
    } else {
        int e;
        if (a.route) {
            if (wib == 0) {
                const bool writer = (j == 0 && tb == 0);
                int my_id;
                float my_val;
                wave_topk<PL>(a.logits + (size_t)t * a.lstride, a.bias, a.E, writer ? a.K : j + 1, j, my_id, my_val);
                if (lane <= j) s_ids[lane] = my_id;
                if (writer) {
                    // weights = softmax over the k selected logits; lane q holds the
                    // q-th, lane 0 the largest; the sum runs in a fixed lane order
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
        valid = e >= 0 && e < a.E;  // an id out of range reads nothing and poisons h
        const int eo = valid ? e : 0;
        cbase = a.codes + (size_t)eo * mat_codes;
        sbase = a.scales + (size_t)eo * mat_scales;
        gp = a.gs ? a.gs + eo : nullptr;
    }
    if (!tile_ok) return;  // after the block's barrier; uniform per wave
    const Buf cb = make_buf(cbase, valid ? mat_codes : 0u);
    const Buf sb = make_buf(sbase, valid ? mat_scales : 0u);

    const int i0 = tile * RT * RG;  // first gate row of this tile
    float ag[RT], au[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) ag[r] = au[r] = 0.f;
    const bool sbf = SBF && j == a.K;  // bf16 shared expert slot (uniform per block)
    if (sbf) {
        const uint32_t rowb = cs;
        const Buf wb = make_buf(cbase, (uint32_t)(2 * I) * rowb);
        for (int s = 0; s < ks; ++s) {
            const int k0 = 32 * (L * s + lk);
            const bool kv = k0 < H;
            XSlice<FMT> xs;
            if (s == 0) xs = xs0;
            else load_xslice<FMT>(xs, xb, kv ? (uint32_t)k0 * 2u : OOB);
            uint4 wg[RT][4], wu[RT][4];
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const int i = i0 + r * RG + rsub;
                const bool v = kv && i < I;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    wg[r][q] = ld128(wb, v ? (uint32_t)i * rowb + (uint32_t)k0 * 2u + 16u * q : OOB);
                    wu[r][q] = ld128(wb, v ? (uint32_t)(I + i) * rowb + (uint32_t)k0 * 2u + 16u * q : OOB);
                }
            }
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                ag[r] = bf16w_dot_bf16<FMT>(wg[r], xs, ag[r]);
                au[r] = bf16w_dot_bf16<FMT>(wu[r], xs, au[r]);
            }
        }
    }
    for (int s = 0; s < (sbf ? 0 : ks); ++s) {
        const int k0 = 32 * (L * s + lk);
        const bool kv = k0 < H;
        XSlice<FMT> xs;
        if (s == 0) xs = xs0;
        else load_xslice<FMT>(xs, xb, kv ? (uint32_t)k0 * 2u : OOB);
        uint4 cg[RT], cu[RT];
        uint32_t sg[RT], su[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const int i = i0 + r * RG + rsub;
            const bool v = kv && i < I;
            const uint32_t rg = (uint32_t)i, ru = (uint32_t)(I + i);
            cg[r] = ld128(cb, v ? rg * cs + (uint32_t)(k0 >> 1) : OOB);
            cu[r] = ld128(cb, v ? ru * cs + (uint32_t)(k0 >> 1) : OOB);
            sg[r] = ld_scales<FMT>(sb, v ? rg * ss + scale_col<FMT>(k0) : OOB);
            su[r] = ld_scales<FMT>(sb, v ? ru * ss + scale_col<FMT>(k0) : OOB);
        }
        prep_xslice<FMT>(xs);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            ag[r] = chunk_dot_bf16<FMT>(cg[r], sg[r], xs, ag[r]);
            au[r] = chunk_dot_bf16<FMT>(cu[r], su[r], xs, au[r]);
        }
    }
    float gsc = 1.f;
    if constexpr (FMT == FMT_NVFP4) gsc = sbf ? 1.f : ld_uniform(gp, 0);
    float *hrow = a.h + ((size_t)t * a.S + j) * a.hstride;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        float g = group_sum<L>(ag[r]);
        float u = group_sum<L>(au[r]);
        if constexpr (FMT == FMT_NVFP4) g *= gsc, u *= gsc;
        const int i = i0 + r * RG + rsub;
        if (group_leader<L>(lane) && i < I) {
            const float hv = valid ? (g / (1.f + expf(-g))) * u : __builtin_nanf("");
            hrow[h_index(i, a.L2)] = hv;
        }
    }
}

// ================================================================= MoE down + combine

struct DownArgs {
    const uint8_t *codes;         // routed W2 [E][H][I/2]
    const uint8_t *scales;        // (bytes)
    const uint8_t *s_codes;       // shared W2 [H][I/2]
    const uint8_t *s_scales;
    const int32_t *ids;           // [T][k]
    const float *w;               // [T][k]
    const float *logits;          // [T][lstride]; column E = shared-gate logit
    const float *h;               // [T][S][hstride]
    uint16_t *y;                  // [T][H] bf16
    int H, I, E, K, S, T, lstride, hstride, blocks_per_tok;
    int s_bf16;                   // shared expert in bf16 (s_codes = bf16 [H][I])
    const float *gs, *s_gs;       // NVFP4 global scales: routed [E], shared [1]
    RowLayout rl, s_rl;           // row strides of the routed and shared matrices
};

// Block = W waves; tile of RT*64/L output rows of one token.  LDS holds one
// fp32 partial per (slot, row); the final sum runs over slots in order.
template <int FMT, int L, int RT, bool SBF>
__global__ __launch_bounds__(1024) void k_moe_down(DownArgs a) {
    constexpr int RG = 64 / L;
    constexpr int ROWS = RT * RG;
    extern __shared__ float part[];  // [S][ROWS]
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int nw = blockDim.x >> 6;
    const int t = blockIdx.x / a.blocks_per_tok;
    const int row0 = (blockIdx.x - t * a.blocks_per_tok) * ROWS;
    const int lk = lane % L, rsub = lane / L;
    const int I = a.I, H = a.H;
    const int ks = (I + 32 * L - 1) / (32 * L);

    for (int j = wv; j < a.S; j += nw) {
        // step-0 activations first: they do not depend on the routing
        const Buf hb = make_buf(a.h + ((size_t)t * a.S + j) * a.hstride, (uint32_t)a.hstride * 4u);
        float4 hv0[8];
        {
            const uint32_t h0 = (uint32_t)lk * 16u;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                hv0[q] = __builtin_bit_cast(float4, ld128(hb, 32 * lk < I ? h0 + (uint32_t)q * L * 16u : OOB));
        }
        const uint8_t *cbase;
        const uint8_t *sbase;
        const float *gp;
        float coef;
        bool valid = true;
        // row strides of this slot's matrix (the shared expert may use another layout)
        const uint32_t cs = j == a.K ? a.s_rl.cs : a.rl.cs, ss = j == a.K ? a.s_rl.ss : a.rl.ss;
        const uint32_t mat_codes = (uint32_t)H * cs, mat_scales = (uint32_t)H * ss;
        if (j == a.K) {
            cbase = a.s_codes;
            sbase = a.s_scales;
            gp = a.s_gs;
            coef = 1.f / (1.f + expf(-ld_uniform(a.logits, t * a.lstride + a.E)));
        } else {
            const int e = ld_uniform(a.ids, t * a.K + j);
            valid = e >= 0 && e < a.E;
            const int eo = valid ? e : 0;
            cbase = a.codes + (size_t)eo * mat_codes;
            sbase = a.scales + (size_t)eo * mat_scales;
            gp = a.gs ? a.gs + eo : nullptr;
            coef = ld_uniform(a.w, t * a.K + j);
        }
        const bool sbf = SBF && j == a.K;  // bf16 shared expert slot (uniform per wave)
        if constexpr (FMT == FMT_NVFP4) {
            if (!sbf) coef *= ld_uniform(gp, 0);  // (w x g) x row sum
        }
        const Buf cb = make_buf(cbase, valid ? mat_codes : 0u);
        const Buf sb = make_buf(sbase, valid ? mat_scales : 0u);
        float acc[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r] = 0.f;
        if (sbf) {
            for (int s = 0; s < ks; ++s) {
                const int k0 = 32 * (L * s + lk);
                const bool kv = k0 < I;
                float4 hv[8];
                if (s == 0) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) hv[q] = hv0[q];
                } else {
                    const uint32_t h0 = ((uint32_t)s * 32u * L + (uint32_t)lk * 4u) * 4u;
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        hv[q] = __builtin_bit_cast(float4, ld128(hb, kv ? h0 + (uint32_t)q * L * 16u : OOB));
                }
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    const int row = row0 + r * RG + rsub;
                    const bool v = kv && row < H;
                    uint4 w[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        w[q] = ld128(cb, v ? (uint32_t)row * cs + (uint32_t)k0 * 2u + 16u * q : OOB);
                    acc[r] = bf16w_dot_f32(w, hv, acc[r]);
                }
            }
        }
        for (int s = 0; s < (sbf ? 0 : ks); ++s) {
            const int k0 = 32 * (L * s + lk);
            const bool kv = k0 < I;
            float4 hv[8];  // activations first
            if (s == 0) {
#pragma unroll
                for (int q = 0; q < 8; ++q) hv[q] = hv0[q];
            } else {
                const uint32_t h0 = ((uint32_t)s * 32u * L + (uint32_t)lk * 4u) * 4u;
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    hv[q] = __builtin_bit_cast(float4, ld128(hb, kv ? h0 + (uint32_t)q * L * 16u : OOB));
            }
            uint4 cw[RT];
            uint32_t sw[RT];
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const int row = row0 + r * RG + rsub;
                const bool v = kv && row < H;
                cw[r] = ld128(cb, v ? (uint32_t)row * cs + (uint32_t)(k0 >> 1) : OOB);
                sw[r] = ld_scales<FMT>(sb, v ? (uint32_t)row * ss + scale_col<FMT>(k0) : OOB);
            }
            float hs = 0.f;
            int hx = 0;
            if constexpr (FMT == FMT_INT4) {
#pragma unroll
                for (int q = 0; q < 8; ++q) hs += (hv[q].x + hv[q].y) + (hv[q].z + hv[q].w);
            }
            if constexpr (FMT == FMT_MXFP4) hx = mx8_block_f32(hv);  // the lane's 32 h values: one MXFP8 block
#pragma unroll
            for (int r = 0; r < RT; ++r) acc[r] = chunk_dot_f32<FMT>(cw[r], sw[r], hv, hs, acc[r], hx);
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const float v = group_sum<L>(acc[r]);
            if (group_leader<L>(lane)) part[j * ROWS + r * RG + rsub] = valid ? v * coef : __builtin_nanf("");
        }
    }
    __syncthreads();
    for (int rr = threadIdx.x; rr < ROWS; rr += blockDim.x) {
        const int row = row0 + rr;
        if (row >= H) continue;
        float v = 0.f;
        for (int j = 0; j < a.S; ++j) v += part[j * ROWS + rr];
        a.y[(size_t)t * H + row] = f32_to_bf16_rne(v);
    }
}

}  // namespace w4k

// ================================================================= scratch of the no-allocation entry point

// The workspace of moe_w4a16_forward_noalloc: one array per GPU, in the code
// object's device memory (each device that loads the library holds its own copy
// until the process ends).  Host code must use the address hipGetSymbolAddress
// returns for it on each device, never this name.
static __device__ __align__(256) unsigned char scratch[W4_NOALLOC_SCRATCH_BYTES];

// ================================================================= host side

using namespace w4k;
using w4::fail;

namespace {

// A launch target: the stream and, for the measurement entry point, the pair of
// events the runtime records at the kernel's start and end.
struct Launch {
    hipStream_t st;
    hipEvent_t start = nullptr, stop = nullptr;
};

template <typename F, typename... Args>
void go(const Launch &l, F kernel, dim3 grid, dim3 block, uint32_t shmem, Args... args) {
    if (l.start)
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, l.st, l.start, l.stop, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, shmem, l.st, args...);
}

int lanes_for(int64_t k) {
    int64_t need = (k + 31) / 32;
    int L = 1;
    while (L < need && L < 64) L <<= 1;
    return L;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// kt16: the caller reads K-tiled matrices (the decode down projection); every
// other use of a matrix dots whole rows and needs a row layout.
int check_matrix(const w4_matrix *W, const char *what, bool kt16 = false) {
    if (!W) return fail(W4_ERR_INVALID_ARG, "%s: null matrix", what);
    int st = w4::check_shape(W->format, W->layout, W->groups, W->n, W->k);
    if (st) return st;
    if (W->layout == W4_LAYOUT_GFX950_KT16 && !kt16)
        return fail(W4_ERR_UNSUPPORTED, "%s: the K-tiled layout serves only an MoE layer's down projection", what);
    if (!W->codes || (!W->scales && W->format != W4_FMT_BF16 && W->layout == W4_LAYOUT_CANONICAL))
        return fail(W4_ERR_INVALID_ARG, "%s: null codes/scales", what);
    if (!aligned(W->codes, 16)) return fail(W4_ERR_ALIGNMENT, "%s: codes not 16-byte aligned", what);
    if (!aligned(W->scales, 4)) return fail(W4_ERR_ALIGNMENT, "%s: scales not 4-byte aligned", what);
    if (W->format == W4_FMT_NVFP4_E4M3S16) {
        if (!W->global_scales) return fail(W4_ERR_INVALID_ARG, "%s: NVFP4 needs global_scales", what);
        if (!aligned(W->global_scales, 4)) return fail(W4_ERR_ALIGNMENT, "%s: global_scales not 4-byte aligned", what);
    }
    if (W->n > (1 << 30) || W->k > (1 << 20)) return fail(W4_ERR_UNSUPPORTED, "%s: dimension too large", what);
    // one matrix of the stack is addressed through 32-bit buffer offsets
    if ((uint64_t)W->n * (uint64_t)w4::v1_row_bytes(W->format, W->k) >= (1ull << 31))
        return fail(W4_ERR_UNSUPPORTED, "%s: one matrix must hold fewer than 2^31 bytes", what);
    return W4_OK;
}

// Row strides of a matrix in its layout, and the base of its block scales (the
// device layout keeps them inside each row record, after the codes).
RowLayout row_layout(const w4_matrix *W) {
    if (W->layout == W4_LAYOUT_GFX950_V1) {
        const uint32_t r = (uint32_t)w4::v1_row_bytes(W->format, W->k);
        return RowLayout{r, r};
    }
    return RowLayout{(uint32_t)w4::code_bytes_per_row(W->format, W->k), (uint32_t)w4::scale_bytes_per_row(W->format, W->k)};
}

const uint8_t *scale_base(const w4_matrix *W) {
    if (W->layout == W4_LAYOUT_GFX950_V1) return W->codes + w4::code_bytes_per_row(W->format, W->k);
    return static_cast<const uint8_t *>(W->scales);
}

int hip_status(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(W4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return W4_OK;
}

// ---------------------------------------------------------------- GEMV launch

#ifndef W4_GEMV_ROWS
#define W4_GEMV_ROWS 2  // rows per wave of the dense GEMV (at least one load group)
#endif
#ifndef W4_GEMV_WPB
#define W4_GEMV_WPB 4  // waves per block of the dense GEMV
#endif
static_assert(W4_GEMV_WPB >= 1 && W4_GEMV_WPB * 64 <= 256, "k_gemv is compiled for blocks of at most 256 threads");

template <int FMT, int L>
void launch_gemv_L(const w4_matrix *W, const uint16_t *x, int m, uint16_t *y, hipStream_t st) {
    constexpr int RG = 64 / L;
    constexpr int RT = RG >= W4_GEMV_ROWS ? 1 : W4_GEMV_ROWS / RG;
    const int n = (int)W->n, k = (int)W->k;
    const int waves = (n + RT * RG - 1) / (RT * RG);
    const int wpb = W4_GEMV_WPB;
    const int blocks = (waves + wpb - 1) / wpb;
    const RowLayout rl = row_layout(W);
    hipLaunchKernelGGL((k_gemv<FMT, L, RT>), dim3(blocks), dim3(64 * wpb), 0, st, W->codes, scale_base(W),
                       W->global_scales, x, y, n, k, m, rl.cs, rl.ss);
}

template <int FMT>
void launch_gemv(const w4_matrix *W, const uint16_t *x, int m, uint16_t *y, hipStream_t st) {
    switch (lanes_for(W->k)) {
    case 1: launch_gemv_L<FMT, 1>(W, x, m, y, st); break;
    case 2: launch_gemv_L<FMT, 2>(W, x, m, y, st); break;
    case 4: launch_gemv_L<FMT, 4>(W, x, m, y, st); break;
    case 8: launch_gemv_L<FMT, 8>(W, x, m, y, st); break;
    case 16: launch_gemv_L<FMT, 16>(W, x, m, y, st); break;
    case 32: launch_gemv_L<FMT, 32>(W, x, m, y, st); break;
    default: launch_gemv_L<FMT, 64>(W, x, m, y, st); break;
    }
}

template <int FMT, int L>
void launch_dequant_L(const w4_matrix *W, float *out, hipStream_t st) {
    constexpr int RG = 64 / L;
    const int64_t rows = W->groups * W->n;
    const int64_t waves = (rows + RG - 1) / RG;
    const int wpb = 4;
    const int64_t blocks = (waves + wpb - 1) / wpb;
    const RowLayout rl = row_layout(W);
    hipLaunchKernelGGL((k_dequant<FMT, L>), dim3((unsigned)blocks), dim3(64 * wpb), 0, st, W->codes, scale_base(W),
                       W->global_scales, out, rows, W->n, (int)W->k, rl.cs, rl.ss);
}

template <int FMT>
void launch_dequant(const w4_matrix *W, float *out, hipStream_t st) {
    switch (lanes_for(W->k)) {
    case 1: launch_dequant_L<FMT, 1>(W, out, st); break;
    case 2: launch_dequant_L<FMT, 2>(W, out, st); break;
    case 4: launch_dequant_L<FMT, 4>(W, out, st); break;
    case 8: launch_dequant_L<FMT, 8>(W, out, st); break;
    case 16: launch_dequant_L<FMT, 16>(W, out, st); break;
    case 32: launch_dequant_L<FMT, 32>(W, out, st); break;
    default: launch_dequant_L<FMT, 64>(W, out, st); break;
    }
}

// ---------------------------------------------------------------- MoE plan

constexpr int MAX_TOPK = 16;
constexpr int MAX_EXPERTS = 1024;  // 64 lanes x 16 logits per lane
constexpr int MAX_TOKENS = 16384;

#ifndef W4_GROUPED_MIN_T
#define W4_GROUPED_MIN_T 4  // batches of at least this many tokens group their pairs by expert
#endif
#ifndef W4_MULTI_ROUTE_MIN_T
#define W4_MULTI_ROUTE_MIN_T (1 << 30)  // smaller batches than this (and <= 4096 pairs) group in one block
#endif
#ifndef W4_RMFMA_NT
#define W4_RMFMA_NT 2  // 16-token column tiles per block of the MFMA router
#endif
#ifndef W4_PF_MIN_PAIRS
#define W4_PF_MIN_PAIRS 1024  // batches of more pairs run W13 / W2 as LDS-staged grouped GEMMs (<= 4096: one-block grouping's limit)
#endif
#ifndef W4_ROUTER_MFMA_MIN_T
// batches of at least this many tokens run the router on MFMA (measured at the
// 35B-A3B shape: the MFMA router ~12.3 us from T = 64 to 512, the per-row VALU
// router 6.2 us at T = 64, 10.4 at 128, 18.6 at 256)
#define W4_ROUTER_MFMA_MIN_T 160
#endif
#ifndef W4_MFMA_MIN
#define W4_MFMA_MIN 2  // expert groups of at least this many rows run on MFMA (single rows on VALU)
#endif
constexpr int MAX_GROUPED_PAIRS = 65536;  // (token, slot) pairs of one grouped call
constexpr int MAX_ONE_BLOCK_PAIRS = 4096;  // up to this many, one block groups them (LDS counting sort)

struct MoEPlan {
    int H, I, E, K, S, T;
    int L13, L2, hstride, lstride;
    bool grouped, mx;
    bool multi;  // grouping over three launches (large batches, or T >= W4_MULTI_ROUTE_MIN_T)
    bool pf;     // W13 / W2 as large-batch grouped GEMMs (more than W4_PF_MIN_PAIRS pairs)
    bool dec;    // K-tiled down projections: the decode kernels (k_moe_dec + k_moe_dec_combine)
    int P, Gmax, nblk, tpb, tiles16;
    size_t off_part;
    size_t off_logits, off_ids, off_w, off_h, total;
    size_t off_grp, off_pairs, off_hp, off_out, off_xq, off_route;
    size_t off_arrive;  // arrival counter of the multi-block ranking (int32)
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int check_layer(const moe_w4a16_layer *Lr, int64_t T, MoEPlan &p) {
    if (!Lr) return fail(W4_ERR_INVALID_ARG, "null layer");
    if (T < 1 || T > MAX_TOKENS) return fail(W4_ERR_INVALID_ARG, "T=%lld out of range [1, %d]", (long long)T, MAX_TOKENS);
    const int64_t H = Lr->hidden, I = Lr->inter, E = Lr->num_experts, K = Lr->top_k;
    if (H < 64 || H % 64) return fail(W4_ERR_UNSUPPORTED, "hidden=%lld must be a positive multiple of 64", (long long)H);
    if (H > (1 << 16) || I < 1 || I > (1 << 16)) return fail(W4_ERR_UNSUPPORTED, "hidden/inter too large");
    if (E < 1 || E > MAX_EXPERTS) return fail(W4_ERR_UNSUPPORTED, "num_experts=%lld out of [1, %d]", (long long)E, MAX_EXPERTS);
    if (K < 1 || K > E || K > MAX_TOPK) return fail(W4_ERR_INVALID_ARG, "top_k=%lld out of [1, min(E, %d)]", (long long)K, MAX_TOPK);
    if (!Lr->router_w) return fail(W4_ERR_INVALID_ARG, "null router_w");
    if (!aligned(Lr->router_w, 16)) return fail(W4_ERR_ALIGNMENT, "router_w not 16-byte aligned");
    int st;
    if ((st = check_matrix(&Lr->w13, "w13"))) return st;
    if ((st = check_matrix(&Lr->w2, "w2", true))) return st;
    const int32_t fmt = Lr->w13.format;
    if (fmt == W4_FMT_BF16) return fail(W4_ERR_UNSUPPORTED, "routed experts must be 4-bit (bf16 is for the shared expert)");
    if (Lr->w2.format != fmt) return fail(W4_ERR_LAYOUT, "w13 and w2 formats differ");
    if (Lr->w13.groups != E || Lr->w13.n != 2 * I || Lr->w13.k != H)
        return fail(W4_ERR_INVALID_ARG, "w13 must be [E][2I][H]");
    if (Lr->w2.groups != E || Lr->w2.n != H || Lr->w2.k != I) return fail(W4_ERR_INVALID_ARG, "w2 must be [E][H][I]");
    if (Lr->has_shared != 0 && Lr->has_shared != 1) return fail(W4_ERR_INVALID_ARG, "has_shared must be 0 or 1");
    if (Lr->has_shared) {
        if (Lr->shared_inter != I)
            return fail(W4_ERR_UNSUPPORTED, "shared_inter=%lld must equal inter=%lld", (long long)Lr->shared_inter, (long long)I);
        if ((st = check_matrix(&Lr->shared_w13, "shared_w13"))) return st;
        if ((st = check_matrix(&Lr->shared_w2, "shared_w2", true))) return st;
        const int32_t sf = Lr->shared_w13.format;
        if ((sf != fmt && sf != W4_FMT_BF16) || Lr->shared_w2.format != sf)
            return fail(W4_ERR_LAYOUT, "shared expert must use the routed experts' format or bf16 for both matrices");
        if (fmt == W4_FMT_MXFP4_E8M0S32 && sf == W4_FMT_BF16)
            return fail(W4_ERR_UNSUPPORTED, "the MXFP4 path takes an MXFP4 shared expert");
        if (Lr->shared_w13.groups != 1 || Lr->shared_w13.n != 2 * I || Lr->shared_w13.k != H)
            return fail(W4_ERR_INVALID_ARG, "shared_w13 must be [1][2I][H]");
        if (Lr->shared_w2.groups != 1 || Lr->shared_w2.n != H || Lr->shared_w2.k != I)
            return fail(W4_ERR_INVALID_ARG, "shared_w2 must be [1][H][I]");
        if (!Lr->shared_gate_w) return fail(W4_ERR_INVALID_ARG, "null shared_gate_w");
        if (!aligned(Lr->shared_gate_w, 16)) return fail(W4_ERR_ALIGNMENT, "shared_gate_w not 16-byte aligned");
    }
    if (Lr->router_bias && !aligned(Lr->router_bias, 4)) return fail(W4_ERR_ALIGNMENT, "router_bias not aligned");
    p.H = (int)H, p.I = (int)I, p.E = (int)E, p.K = (int)K, p.T = (int)T;
    p.S = (int)K + (Lr->has_shared ? 1 : 0);
    p.L13 = lanes_for(H);
    p.L2 = lanes_for(I);
    const int ks2 = (int)((I + 32 * p.L2 - 1) / (32 * p.L2));
    p.hstride = ks2 * 32 * p.L2;
    p.lstride = (int)align_up((size_t)E + 1, 64);
    // batches: group the (token, slot) pairs by expert (E2M1 or NVFP4 weights,
    // and int4 up to MAX_ONE_BLOCK_PAIRS pairs; 128-wide K chunks for the MFMA
    // tiles; the shared expert 4-bit or bf16)
    p.P = (int)(T * K);
    p.Gmax = (int)(E < p.P ? E : p.P);
    // (the VALU small-group path keeps at most 2 k-steps of 32 x 64 elements)
    p.mx = fmt == W4_FMT_MXFP4_E8M0S32;
    p.grouped = T >= W4_GROUPED_MIN_T && H % 128 == 0 && I % 128 == 0 && H <= 4096 && I <= 4096 &&
                ((fmt == W4_FMT_E2M1_F16S16 || fmt == W4_FMT_NVFP4_E4M3S16) ? p.P <= MAX_GROUPED_PAIRS
                                                                          : fmt == W4_FMT_INT4_F16S128 &&
                                                                                p.P <= MAX_ONE_BLOCK_PAIRS);
    if (p.mx) {  // batches run grouped on the scaled FP4 MFMA; single tokens on the VALU kernels
        if (H % 128 || I % 128)
            return fail(W4_ERR_UNSUPPORTED, "MXFP4 layers need hidden and inter multiples of 128");
        if (p.P > MAX_GROUPED_PAIRS)
            return fail(W4_ERR_UNSUPPORTED, "MXFP4 layers take at most %d (token, slot) pairs per call",
                        MAX_GROUPED_PAIRS);
        p.grouped = T >= W4_GROUPED_MIN_T;
    }
    // K-tiled down projections: the decode kernels, for every T (batches re-read
    // each selected expert per token there, so they suit decode, not prefill)
    p.dec = Lr->w2.layout == W4_LAYOUT_GFX950_KT16;
    if (Lr->has_shared && (Lr->shared_w2.layout == W4_LAYOUT_GFX950_KT16) != p.dec)
        return fail(W4_ERR_UNSUPPORTED, "w2 and shared_w2 must both be K-tiled or both not");
    if (p.dec) {
        if (fmt != W4_FMT_E2M1_F16S16 && fmt != W4_FMT_NVFP4_E4M3S16)
            return fail(W4_ERR_UNSUPPORTED, "K-tiled down projections need E2M1 or NVFP4 experts");
        if (Lr->has_shared && Lr->shared_w13.format != fmt)
            return fail(W4_ERR_UNSUPPORTED, "with K-tiled down projections the shared expert uses the routed format");
        if (H > DEC_MAX_H) return fail(W4_ERR_UNSUPPORTED, "K-tiled down projections need hidden <= %d", DEC_MAX_H);
        if (I % DEC_TILE) return fail(W4_ERR_UNSUPPORTED, "K-tiled down projections need inter a multiple of 16");
        if (T > 1024) return fail(W4_ERR_UNSUPPORTED, "a layer with K-tiled down projections serves up to 1024 tokens");
        p.grouped = false;
        p.mx = false;
    }
    p.tiles16 = (int)(I / DEC_TILE);
    p.pf = p.grouped && p.P > W4_PF_MIN_PAIRS && fmt != W4_FMT_INT4_F16S128;
    p.multi = p.pf || (p.grouped && T >= W4_MULTI_ROUTE_MIN_T);
    p.tpb = T <= 256 ? 4 : ROUTE_MAX_TPB;  // one token per wave while that keeps the scan short
    p.nblk = (int)((T + p.tpb - 1) / p.tpb);
    size_t off = 0;
    p.off_logits = off; off = align_up(off + (size_t)T * p.lstride * 4, 256);
    p.off_ids = off;    off = align_up(off + (size_t)T * K * 4, 256);
    p.off_w = off;      off = align_up(off + (size_t)T * K * 4, 256);
    if (p.dec) {  // fp32 contribution of every (token, slot, 16-value tile) to every output row
        p.off_part = off; off = align_up(off + (size_t)T * p.S * p.tiles16 * H * 4, 256);
    } else if (!p.grouped) {
        p.off_h = off;  off = align_up(off + (size_t)T * p.S * p.hstride * 4, 256);
    } else {
        const size_t rows = (size_t)p.P + (size_t)T;
        p.off_grp = off;   off = align_up(off + (size_t)(2 + 3 * p.Gmax) * 4, 256);
        p.off_arrive = off; off = align_up(off + 4, 256);
        p.off_pairs = off; off = align_up(off + rows * 4, 256);
        p.off_hp = off;    off = align_up(off + rows * (size_t)I * 4, 256);  // h_hi then h_lo, bf16 (MX: codes, scales)
        p.off_out = off;   off = align_up(off + rows * (size_t)H * 4, 256);
        if (p.mx) {  // x as MXFP8: codes [T][H], then scales [T][H/32]
            p.off_xq = off; off = align_up(off + (size_t)T * H + (size_t)T * (H / 32), 256);
        }
        if (p.multi) {  // e_of [P], off_e [E], cntb [nblk][E], column tiles [2][Gmax + P/64 + 1], cbase [nblk][E]
            p.off_route = off;
            off = align_up(off + ((size_t)p.P + (size_t)E + 2 * (size_t)p.nblk * (size_t)E +
                                  2 * ((size_t)p.Gmax + (size_t)p.P / 64 + 1)) * 4, 256);
        }
    }
    p.total = off;
    return W4_OK;
}

int launch_router(const moe_w4a16_layer *Lr, const MoEPlan &p, const uint16_t *x, float *logits, int r_begin,
                  int r_end, const Launch &st, int32_t *arrive = nullptr) {
    const int nrows = r_end - r_begin;
    if (nrows <= 0) return W4_OK;
    if (p.T >= W4_ROUTER_MFMA_MIN_T) {
        go(st, k_router_mfma<W4_RMFMA_NT>, dim3((unsigned)((p.T + 16 * W4_RMFMA_NT - 1) / (16 * W4_RMFMA_NT)),
                                             (unsigned)((nrows + 15) / 16)), dim3(256), 0,
           Lr->router_w, Lr->shared_gate_w, x, logits, p.E, p.H, p.T, r_begin, r_end, p.lstride, arrive);
        return W4_OK;
    }
    const int ns = (p.H + 511) / 512;
    // tokens per chunk: 1 for single-token decode, else 4 (activation loads in flight together)
    auto with_ns = [&](auto NSc) {
        constexpr int NS = decltype(NSc)::value;
        if (p.T == 1) {
            go(st, k_router<NS, 1>, dim3(nrows), dim3(64), 0, Lr->router_w, Lr->shared_gate_w, x, logits, p.E, p.H,
               p.T, r_begin, p.lstride, arrive);
        } else {  // chunks of 4 tokens (2 for the widest rows), up to 8 waves per row
            constexpr int TB = NS >= 16 ? 2 : 4;
            const int waves = (p.T + TB - 1) / TB < 8 ? (p.T + TB - 1) / TB : 8;
            go(st, k_router<NS, TB>, dim3(nrows), dim3(64 * waves), 0, Lr->router_w, Lr->shared_gate_w, x, logits,
               p.E, p.H, p.T, r_begin, p.lstride, arrive);
        }
    };
    if (ns <= 1) with_ns(std::integral_constant<int, 1>());
    else if (ns <= 2) with_ns(std::integral_constant<int, 2>());
    else if (ns <= 4) with_ns(std::integral_constant<int, 4>());
    else if (ns <= 8) with_ns(std::integral_constant<int, 8>());
    else if (ns <= 16) with_ns(std::integral_constant<int, 16>());
    else return fail(W4_ERR_UNSUPPORTED, "hidden=%d too large for the router kernel", p.H);
    return W4_OK;
}

#ifndef W4_W13_ROWS
#define W4_W13_ROWS 2  // gate rows (and as many up rows) per wave of the W13 kernel
#endif
#ifndef W4_W13_WPB
#define W4_W13_WPB 2  // waves per block of the W13 kernel
#endif
static_assert(W4_W13_WPB >= 1 && W4_W13_WPB <= 16, "k_moe_w13 is compiled for blocks of at most 1024 threads");

template <int FMT, int L>
void launch_w13_L(const MoEPlan &p, W13Args &a, const Launch &st) {
    constexpr int RG = 64 / L;
    constexpr int RT = RG >= W4_W13_ROWS ? 1 : W4_W13_ROWS / RG;
    a.tiles = (p.I + RT * RG - 1) / (RT * RG);
    const int wpb = a.tiles < W4_W13_WPB ? a.tiles : W4_W13_WPB;
    const int tblocks = (a.tiles + wpb - 1) / wpb;
    const int blocks = p.T * p.S * tblocks;
    const int pl = (p.E + 63) / 64;
    const dim3 g(blocks), bl(64 * wpb);
    auto with_pl = [&](auto SBFc) {
        constexpr bool SB = decltype(SBFc)::value;
        if (pl <= 1) go(st, k_moe_w13<FMT, L, RT, 1, SB>, g, bl, 0, a);
        else if (pl <= 2) go(st, k_moe_w13<FMT, L, RT, 2, SB>, g, bl, 0, a);
        else if (pl <= 4) go(st, k_moe_w13<FMT, L, RT, 4, SB>, g, bl, 0, a);
        else if (pl <= 8) go(st, k_moe_w13<FMT, L, RT, 8, SB>, g, bl, 0, a);
        else go(st, k_moe_w13<FMT, L, RT, 16, SB>, g, bl, 0, a);
    };
    if (a.s_bf16) with_pl(std::true_type());
    else with_pl(std::false_type());
}

template <int FMT>
void launch_w13(const MoEPlan &p, W13Args &a, const Launch &st) {
    switch (p.L13) {
    case 1: launch_w13_L<FMT, 1>(p, a, st); break;
    case 2: launch_w13_L<FMT, 2>(p, a, st); break;
    case 4: launch_w13_L<FMT, 4>(p, a, st); break;
    case 8: launch_w13_L<FMT, 8>(p, a, st); break;
    case 16: launch_w13_L<FMT, 16>(p, a, st); break;
    case 32: launch_w13_L<FMT, 32>(p, a, st); break;
    default: launch_w13_L<FMT, 64>(p, a, st); break;
    }
}

#ifndef W4_DOWN_ROWS
#define W4_DOWN_ROWS 8  // output rows per block of the down kernel (at least one load group)
#endif
#ifndef W4_DOWN_WAVES
#define W4_DOWN_WAVES 16  // at most this many waves per block; the slots are spread over them
#endif
static_assert(W4_DOWN_WAVES >= 1 && W4_DOWN_WAVES <= 16, "k_moe_down is compiled for blocks of at most 1024 threads");

template <int FMT, int L>
void launch_down_L(const MoEPlan &p, DownArgs &a, const Launch &st) {
    constexpr int RG = 64 / L;
    constexpr int RT = RG >= W4_DOWN_ROWS ? 1 : W4_DOWN_ROWS / RG;
    constexpr int ROWS = RT * RG;
    a.blocks_per_tok = (p.H + ROWS - 1) / ROWS;
    int nw = p.S < W4_DOWN_WAVES ? p.S : W4_DOWN_WAVES;
    nw = (p.S + ((p.S + nw - 1) / nw) - 1) / ((p.S + nw - 1) / nw);  // equal slots per wave
    const size_t lds = (size_t)p.S * ROWS * sizeof(float);
    if (a.s_bf16) go(st, k_moe_down<FMT, L, RT, true>, dim3(p.T * a.blocks_per_tok), dim3(64 * nw), (uint32_t)lds, a);
    else go(st, k_moe_down<FMT, L, RT, false>, dim3(p.T * a.blocks_per_tok), dim3(64 * nw), (uint32_t)lds, a);
}

template <int FMT>
void launch_down(const MoEPlan &p, DownArgs &a, const Launch &st) {
    switch (p.L2) {
    case 1: launch_down_L<FMT, 1>(p, a, st); break;
    case 2: launch_down_L<FMT, 2>(p, a, st); break;
    case 4: launch_down_L<FMT, 4>(p, a, st); break;
    case 8: launch_down_L<FMT, 8>(p, a, st); break;
    case 16: launch_down_L<FMT, 16>(p, a, st); break;
    case 32: launch_down_L<FMT, 32>(p, a, st); break;
    default: launch_down_L<FMT, 64>(p, a, st); break;
    }
}

int run_grouped(const moe_w4a16_layer *Lr, const MoEPlan &p, const uint16_t *x, const int32_t *ids_in,
                const float *w_in, uint16_t *y, int32_t *topk_ids, float *topk_w, char *wsb, hipStream_t sm,
                void *const *events);

int run_decode(const moe_w4a16_layer *Lr, const MoEPlan &p, const uint16_t *x, const int32_t *ids_in,
               const float *w_in, uint16_t *y, int32_t *topk_ids, float *topk_w, char *wsb, hipStream_t sm,
               void *const *events);

int stage_count(const MoEPlan &p) {
    if (!p.grouped) return 3;
    return 5 + (p.mx ? 1 : 0) + (p.multi ? 2 : 0);
}

int run_moe(const moe_w4a16_layer *Lr, const uint16_t *x, int64_t T, const int32_t *ids_in, const float *w_in,
            uint16_t *y, int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, void *stream,
            void *const *events = nullptr, int n_events = 0) {
    MoEPlan p{};
    int st = check_layer(Lr, T, p);
    if (st) return st;
    if (!x || !y) return fail(W4_ERR_INVALID_ARG, "null x or y");
    if (!aligned(x, 16)) return fail(W4_ERR_ALIGNMENT, "x not 16-byte aligned");
    if (!aligned(y, 2)) return fail(W4_ERR_ALIGNMENT, "y not 2-byte aligned");
    if (!ws) return fail(W4_ERR_WORKSPACE, "null workspace");
    if (!aligned(ws, 256)) return fail(W4_ERR_ALIGNMENT, "workspace not 256-byte aligned");
    if (ws_bytes < p.total) return fail(W4_ERR_WORKSPACE, "workspace %zu < required %zu bytes", ws_bytes, p.total);
    const bool route = ids_in == nullptr;
    if (!route && !w_in) return fail(W4_ERR_INVALID_ARG, "null routing weights");
    if ((topk_ids && !aligned(topk_ids, 4)) || (topk_w && !aligned(topk_w, 4)) || (ids_in && !aligned(ids_in, 4)) ||
        (w_in && !aligned(w_in, 4)))
        return fail(W4_ERR_ALIGNMENT, "routing arrays not 4-byte aligned");
    hipStream_t sm = (hipStream_t)stream;
    char *wsb = (char *)ws;
    float *logits = (float *)(wsb + p.off_logits);
    int32_t *ids_ws = (int32_t *)(wsb + p.off_ids);
    float *w_ws = (float *)(wsb + p.off_w);
    float *h = (float *)(wsb + p.off_h);

    if (events) {
        const int need = 2 * stage_count(p);
        if (n_events < need)
            return fail(W4_ERR_INVALID_ARG, "%s path needs %d events, got %d", p.grouped ? "grouped" : "single-token",
                        need, n_events);
        for (int i = 0; i < need; ++i)
            if (!events[i]) return fail(W4_ERR_INVALID_ARG, "null stage event %d", i);
    }
    if (p.dec) return run_decode(Lr, p, x, ids_in, w_in, y, topk_ids, topk_w, wsb, sm, events);
    if (p.grouped) return run_grouped(Lr, p, x, ids_in, w_in, y, topk_ids, topk_w, wsb, sm, events);
    Launch l_router{sm}, l_w13{sm}, l_down{sm};
    if (events) {
        l_router.start = (hipEvent_t)events[0], l_router.stop = (hipEvent_t)events[1];
        l_w13.start = (hipEvent_t)events[2], l_w13.stop = (hipEvent_t)events[3];
        l_down.start = (hipEvent_t)events[4], l_down.stop = (hipEvent_t)events[5];
    }
    (void)hipGetLastError();  // clear a stale error so the checks below see only ours
    // 1) router logits (all experts + shared gate) or just the shared gate
    if (route) st = launch_router(Lr, p, x, logits, 0, p.E + (Lr->has_shared ? 1 : 0), l_router);
    else if (Lr->has_shared) st = launch_router(Lr, p, x, logits, p.E, p.E + 1, l_router);
    if (st) return st;
    if ((st = hip_status("router launch"))) return st;

    // 2) W13 + SiLU over all (token, slot, tile)
    W13Args a{};
    a.codes = Lr->w13.codes;
    a.scales = scale_base(&Lr->w13);
    a.rl = row_layout(&Lr->w13);
    a.gs = Lr->w13.global_scales;
    a.s_codes = Lr->has_shared ? Lr->shared_w13.codes : nullptr;
    a.s_scales = Lr->has_shared ? scale_base(&Lr->shared_w13) : nullptr;
    a.s_gs = Lr->has_shared ? Lr->shared_w13.global_scales : nullptr;
    if (Lr->has_shared) a.s_rl = row_layout(&Lr->shared_w13);
    a.s_bf16 = Lr->has_shared && Lr->shared_w13.format == W4_FMT_BF16;
    a.x = x;
    a.logits = logits;
    a.bias = Lr->router_bias;
    a.ids_in = ids_in;
    a.ids_ws = ids_ws;
    a.w_ws = w_ws;
    a.ids_user = route ? topk_ids : nullptr;
    a.w_user = route ? topk_w : nullptr;
    a.h = h;
    a.H = p.H, a.I = p.I, a.E = p.E, a.K = p.K, a.S = p.S, a.T = p.T;
    a.lstride = p.lstride, a.hstride = p.hstride, a.route = route ? 1 : 0, a.L2 = p.L2;
    if (Lr->w13.format == W4_FMT_E2M1_F16S16) launch_w13<FMT_E2M1>(p, a, l_w13);
    else if (Lr->w13.format == W4_FMT_NVFP4_E4M3S16) launch_w13<FMT_NVFP4>(p, a, l_w13);
    else if (Lr->w13.format == W4_FMT_MXFP4_E8M0S32) launch_w13<FMT_MXFP4>(p, a, l_w13);
    else launch_w13<FMT_INT4>(p, a, l_w13);
    if ((st = hip_status("w13 launch"))) return st;

    // 3) down projection + weighted combine
    DownArgs d{};
    d.codes = Lr->w2.codes;
    d.scales = scale_base(&Lr->w2);
    d.rl = row_layout(&Lr->w2);
    d.gs = Lr->w2.global_scales;
    d.s_codes = Lr->has_shared ? Lr->shared_w2.codes : nullptr;
    d.s_scales = Lr->has_shared ? scale_base(&Lr->shared_w2) : nullptr;
    d.s_gs = Lr->has_shared ? Lr->shared_w2.global_scales : nullptr;
    if (Lr->has_shared) d.s_rl = row_layout(&Lr->shared_w2);
    d.s_bf16 = Lr->has_shared && Lr->shared_w2.format == W4_FMT_BF16;
    d.ids = route ? ids_ws : ids_in;
    d.w = route ? w_ws : w_in;
    d.logits = logits;
    d.h = h;
    d.y = y;
    d.H = p.H, d.I = p.I, d.E = p.E, d.K = p.K, d.S = p.S, d.T = p.T;
    d.lstride = p.lstride, d.hstride = p.hstride;
    if (Lr->w2.format == W4_FMT_E2M1_F16S16) launch_down<FMT_E2M1>(p, d, l_down);
    else if (Lr->w2.format == W4_FMT_NVFP4_E4M3S16) launch_down<FMT_NVFP4>(p, d, l_down);
    else if (Lr->w2.format == W4_FMT_MXFP4_E8M0S32) launch_down<FMT_MXFP4>(p, d, l_down);
    else launch_down<FMT_INT4>(p, d, l_down);
    return hip_status("down launch");
}

int run_decode(const moe_w4a16_layer *Lr, const MoEPlan &p, const uint16_t *x, const int32_t *ids_in,
               const float *w_in, uint16_t *y, int32_t *topk_ids, float *topk_w, char *wsb, hipStream_t sm,
               void *const *events) {
    const bool route = ids_in == nullptr;
    float *logits = (float *)(wsb + p.off_logits);
    int32_t *ids_ws = (int32_t *)(wsb + p.off_ids);
    float *w_ws = (float *)(wsb + p.off_w);
    float *part = (float *)(wsb + p.off_part);
    auto ev = [&](int i) { return events ? (hipEvent_t)events[i] : (hipEvent_t) nullptr; };
    int st;
    (void)hipGetLastError();
    // 1) router logits (and the shared-gate logit)
    Launch l_router{sm, ev(0), ev(1)};
    if (route) st = launch_router(Lr, p, x, logits, 0, p.E + (Lr->has_shared ? 1 : 0), l_router);
    else if (Lr->has_shared) st = launch_router(Lr, p, x, logits, p.E, p.E + 1, l_router);
    else st = W4_OK;
    if (st) return st;
    if ((st = hip_status("router launch"))) return st;
    // 2) per (token, slot, 16-value tile): W13 rows, SiLU * up, the tile of W2
    DecArgs a{};
    a.codes13 = Lr->w13.codes, a.scales13 = scale_base(&Lr->w13), a.rl13 = row_layout(&Lr->w13);
    a.codes2 = Lr->w2.codes;
    a.tile_bytes = (uint32_t)w4::kt16_tile_bytes(Lr->w2.format, Lr->w2.n);
    a.gs13 = Lr->w13.global_scales, a.gs2 = Lr->w2.global_scales;
    if (Lr->has_shared) {
        a.s_codes13 = Lr->shared_w13.codes, a.s_scales13 = scale_base(&Lr->shared_w13);
        a.s_rl13 = row_layout(&Lr->shared_w13);
        a.s_codes2 = Lr->shared_w2.codes;
        a.s_gs13 = Lr->shared_w13.global_scales, a.s_gs2 = Lr->shared_w2.global_scales;
    }
    a.x = x, a.logits = logits, a.bias = Lr->router_bias, a.ids_in = ids_in;
    a.ids_ws = ids_ws, a.w_ws = w_ws;
    a.ids_user = route ? topk_ids : nullptr, a.w_user = route ? topk_w : nullptr;
    a.part = part;
    a.H = p.H, a.I = p.I, a.E = p.E, a.K = p.K, a.S = p.S, a.T = p.T, a.tiles = p.tiles16;
    a.lstride = p.lstride, a.route = route ? 1 : 0;
    launch_dec(a, Lr->w13.format == W4_FMT_NVFP4_E4M3S16 ? FMT_NVFP4 : FMT_E2M1, sm, ev(2), ev(3));
    if ((st = hip_status("decode expert launch"))) return st;
    // 3) ordered combine of the tile contributions
    DecCombineArgs c{};
    c.w = route ? w_ws : w_in;
    c.logits = logits, c.part = part, c.y = y;
    c.H = p.H, c.E = p.E, c.K = p.K, c.S = p.S, c.T = p.T, c.tiles = p.tiles16, c.lstride = p.lstride;
    c.has_shared = Lr->has_shared;
    launch_dec_combine(c, sm, ev(4), ev(5));
    return hip_status("decode combine launch");
}

int run_grouped(const moe_w4a16_layer *Lr, const MoEPlan &p, const uint16_t *x, const int32_t *ids_in,
                const float *w_in, uint16_t *y, int32_t *topk_ids, float *topk_w, char *wsb, hipStream_t sm,
                void *const *events) {
    const bool route = ids_in == nullptr;
    float *logits = (float *)(wsb + p.off_logits);
    int32_t *ids_ws = (int32_t *)(wsb + p.off_ids);
    float *w_ws = (float *)(wsb + p.off_w);
    int32_t *grp = (int32_t *)(wsb + p.off_grp);
    int32_t *pairs = (int32_t *)(wsb + p.off_pairs);
    uint16_t *h_hi = (uint16_t *)(wsb + p.off_hp);
    uint16_t *h_lo = h_hi + ((size_t)p.P + p.T) * p.I;
    float *outp = (float *)(wsb + p.off_out);
    auto ev = [&](int i) { return events ? (hipEvent_t)events[i] : (hipEvent_t) nullptr; };
    // stage events after the router (and the MX quantiser): the grouping takes
    // 1 launch, or 3 for large batches
    int next_ev = p.mx ? 4 : 2;
    int32_t *arrive = (int32_t *)(wsb + p.off_arrive);
    auto group = [&](GroupArgs &ga) {
        if (!p.multi) {
            // routed: ranking over many blocks (the router launch zeroes the
            // arrival counter); caller routing: one block reads the ids
            if (route) launch_rank_group(ga, arrive, sm, ev(next_ev), ev(next_ev + 1));
            else launch_route_group(ga, sm, ev(next_ev), ev(next_ev + 1));
            next_ev += 2;
            return;
        }
        RouteArgs r{};
        r.g = ga;
        int32_t *rb = (int32_t *)(wsb + p.off_route);
        r.e_of = rb, r.off_e = rb + p.P, r.cntb = rb + p.P + p.E, r.nblk = p.nblk, r.tpb = p.tpb;
        r.ctg = r.cntb + (size_t)p.nblk * p.E;
        r.cbase = r.ctg + 2 * ((size_t)p.Gmax + (size_t)p.P / 64 + 1);
        hipEvent_t e6[6];
        for (int i = 0; i < 6; ++i) e6[i] = ev(next_ev + i);
        launch_route_multi(r, sm, events ? e6 : nullptr);
        next_ev += 6;
    };
    int st;
    (void)hipGetLastError();
    // 1) router logits (and the shared-gate logit)
    Launch l_router{sm, ev(0), ev(1)};
    if (route)
        st = launch_router(Lr, p, x, logits, 0, p.E + (Lr->has_shared ? 1 : 0), l_router, p.multi ? nullptr : arrive);
    else if (Lr->has_shared) st = launch_router(Lr, p, x, logits, p.E, p.E + 1, l_router);
    else st = W4_OK;
    if (st) return st;
    if ((st = hip_status("router launch"))) return st;
    // 2) top-k + grouping
    GroupArgs ga{};
    ga.logits = logits, ga.bias = Lr->router_bias, ga.ids_in = ids_in;
    ga.ids_ws = ids_ws, ga.w_ws = w_ws;
    ga.ids_user = route ? topk_ids : nullptr, ga.w_user = route ? topk_w : nullptr;
    ga.grp = grp, ga.pairs = pairs;
    ga.E = p.E, ga.K = p.K, ga.T = p.T, ga.P = p.P, ga.Gmax = p.Gmax, ga.lstride = p.lstride, ga.route = route ? 1 : 0;
    ga.mfma_min = W4_MFMA_MIN;
    if (p.mx) {
        // x -> MXFP8 (its own stage, recorded between router and grouping)
        uint8_t *xq = (uint8_t *)(wsb + p.off_xq);
        MXQuantArgs q{};
        q.x = x, q.q = xq, q.s = xq + (size_t)p.T * p.H, q.rows = p.T, q.n = p.H;
        launch_mx_quant(q, sm, ev(2), ev(3));
        if ((st = hip_status("mx quantise launch"))) return st;
        group(ga);
        if ((st = hip_status("route/group launch"))) return st;
        const size_t rows = (size_t)p.P + p.T;
        uint8_t *hq = (uint8_t *)(wsb + p.off_hp), *hs = hq + rows * p.I;
        MX13Args a{};
        a.codes = Lr->w13.codes, a.scales = scale_base(&Lr->w13), a.rl = row_layout(&Lr->w13);
        a.s_codes = Lr->has_shared ? Lr->shared_w13.codes : nullptr;
        a.s_scales = Lr->has_shared ? scale_base(&Lr->shared_w13) : nullptr;
        if (Lr->has_shared) a.s_rl = row_layout(&Lr->shared_w13);
        a.xq = q.q, a.xs = q.s, a.grp = grp, a.pairs = pairs, a.hq = hq, a.hs = hs;
        a.H = p.H, a.I = p.I, a.K = p.K, a.T = p.T, a.P = p.P, a.Gmax = p.Gmax;
        int32_t *ctg = p.multi ? (int32_t *)(wsb + p.off_route) + p.P + p.E + (size_t)p.nblk * p.E : nullptr;
        a.ctg = ctg;
        if (p.pf) launch_pfmx13(a, sm, ev(next_ev), ev(next_ev + 1));
        else launch_mx13(a, sm, ev(next_ev), ev(next_ev + 1));
        if ((st = hip_status("mx w13 launch"))) return st;
        MX2Args d{};
        d.codes = Lr->w2.codes, d.scales = scale_base(&Lr->w2), d.rl = row_layout(&Lr->w2);
        d.s_codes = Lr->has_shared ? Lr->shared_w2.codes : nullptr;
        d.s_scales = Lr->has_shared ? scale_base(&Lr->shared_w2) : nullptr;
        if (Lr->has_shared) d.s_rl = row_layout(&Lr->shared_w2);
        d.grp = grp, d.pairs = pairs, d.hq = hq, d.hs = hs, d.out = outp;
        d.H = p.H, d.I = p.I, d.K = p.K, d.T = p.T, d.P = p.P, d.Gmax = p.Gmax;
        d.ctg = ctg;
        if (p.pf) launch_pfmx2(d, sm, ev(next_ev + 2), ev(next_ev + 3));
        else launch_mx2(d, sm, ev(next_ev + 2), ev(next_ev + 3));
        if ((st = hip_status("mx w2 launch"))) return st;
        next_ev += 4;
    } else {
    group(ga);
    if ((st = hip_status("route/group launch"))) return st;
    // 3) grouped W13 + SiLU
    GW13Args a{};
    a.codes = Lr->w13.codes, a.scales = scale_base(&Lr->w13), a.rl = row_layout(&Lr->w13);
    a.s_codes = Lr->has_shared ? Lr->shared_w13.codes : nullptr;
    a.s_scales = Lr->has_shared ? scale_base(&Lr->shared_w13) : nullptr;
    if (Lr->has_shared) a.s_rl = row_layout(&Lr->shared_w13);
    a.x = x, a.grp = grp, a.pairs = pairs, a.h_hi = h_hi, a.h_lo = h_lo;
    a.H = p.H, a.I = p.I, a.K = p.K, a.T = p.T, a.P = p.P, a.Gmax = p.Gmax, a.mfma_min = W4_MFMA_MIN;
    a.fmt = Lr->w13.format == W4_FMT_NVFP4_E4M3S16 ? FMT_NVFP4
            : Lr->w13.format == W4_FMT_INT4_F16S128 ? FMT_INT4
                                                    : FMT_E2M1;
    a.gs = Lr->w13.global_scales, a.s_gs = Lr->has_shared ? Lr->shared_w13.global_scales : nullptr;
    a.s_bf16 = Lr->has_shared && Lr->shared_w13.format == W4_FMT_BF16;
    int32_t *ctg = p.multi ? (int32_t *)(wsb + p.off_route) + p.P + p.E + (size_t)p.nblk * p.E : nullptr;
    a.ctg = ctg;
    if (p.pf) launch_pf13(a, sm, ev(next_ev), ev(next_ev + 1));
    else launch_gw13(a, sm, ev(next_ev), ev(next_ev + 1));
    if ((st = hip_status("grouped w13 launch"))) return st;
    // 4) grouped W2
    GW2Args d{};
    d.codes = Lr->w2.codes, d.scales = scale_base(&Lr->w2), d.rl = row_layout(&Lr->w2);
    d.s_codes = Lr->has_shared ? Lr->shared_w2.codes : nullptr;
    d.s_scales = Lr->has_shared ? scale_base(&Lr->shared_w2) : nullptr;
    if (Lr->has_shared) d.s_rl = row_layout(&Lr->shared_w2);
    d.grp = grp, d.pairs = pairs, d.h_hi = h_hi, d.h_lo = h_lo, d.out = outp;
    d.H = p.H, d.I = p.I, d.K = p.K, d.T = p.T, d.P = p.P, d.Gmax = p.Gmax, d.mfma_min = W4_MFMA_MIN;
    d.fmt = a.fmt;
    d.gs = Lr->w2.global_scales, d.s_gs = Lr->has_shared ? Lr->shared_w2.global_scales : nullptr;
    d.s_bf16 = a.s_bf16;
    d.ctg = ctg;
    if (p.pf) launch_pf2(d, sm, ev(next_ev + 2), ev(next_ev + 3));
    else launch_gw2(d, sm, ev(next_ev + 2), ev(next_ev + 3));
    next_ev += 4;
    if ((st = hip_status("grouped w2 launch"))) return st;
    }
    // 5) ordered combine
    GCombineArgs c{};
    c.ids = route ? ids_ws : ids_in;
    c.w = route ? w_ws : w_in;
    c.logits = logits, c.out = outp, c.y = y;
    c.H = p.H, c.E = p.E, c.K = p.K, c.T = p.T, c.P = p.P, c.lstride = p.lstride, c.has_shared = Lr->has_shared;
    launch_gcombine(c, sm, ev(next_ev), ev(next_ev + 1));
    return hip_status("combine launch");
}

}  // namespace

extern "C" {

int w4a16_gemv(const w4_matrix *W, const uint16_t *x, int64_t m, uint16_t *y, void *stream) {
    w4::clear_error();
    int st = check_matrix(W, "W");
    if (st) return st;
    if (W->groups != 1) return fail(W4_ERR_INVALID_ARG, "gemv needs groups == 1");
    if (W->format == W4_FMT_BF16) return fail(W4_ERR_UNSUPPORTED, "bf16 matrices serve only as the shared expert");
    if (W->format == W4_FMT_MXFP4_E8M0S32)
        return fail(W4_ERR_UNSUPPORTED, "MXFP4 matrices serve the MoE layer (MXFP8 activations), not the GEMV");
    if (m < 1 || m > 64) return fail(W4_ERR_UNSUPPORTED, "m=%lld out of [1, 64]", (long long)m);
    if (!x || !y) return fail(W4_ERR_INVALID_ARG, "null x or y");
    if (!aligned(x, 16)) return fail(W4_ERR_ALIGNMENT, "x not 16-byte aligned");
    if (!aligned(y, 2)) return fail(W4_ERR_ALIGNMENT, "y not 2-byte aligned");
    (void)hipGetLastError();
    hipStream_t sm = (hipStream_t)stream;
    if (W->format == W4_FMT_E2M1_F16S16) launch_gemv<FMT_E2M1>(W, x, (int)m, y, sm);
    else if (W->format == W4_FMT_NVFP4_E4M3S16) launch_gemv<FMT_NVFP4>(W, x, (int)m, y, sm);
    else launch_gemv<FMT_INT4>(W, x, (int)m, y, sm);
    return hip_status("gemv launch");
}

int w4_dequant_device(const w4_matrix *W, float *out, void *stream) {
    w4::clear_error();
    int st = check_matrix(W, "W");
    if (st) return st;
    if (W->format == W4_FMT_BF16) return fail(W4_ERR_UNSUPPORTED, "bf16 matrices need no dequantisation");
    if (!out) return fail(W4_ERR_INVALID_ARG, "null out");
    if (!aligned(out, 16)) return fail(W4_ERR_ALIGNMENT, "out not 16-byte aligned");
    (void)hipGetLastError();
    hipStream_t sm = (hipStream_t)stream;
    if (W->format == W4_FMT_E2M1_F16S16) launch_dequant<FMT_E2M1>(W, out, sm);
    else if (W->format == W4_FMT_NVFP4_E4M3S16) launch_dequant<FMT_NVFP4>(W, out, sm);
    else if (W->format == W4_FMT_MXFP4_E8M0S32) launch_dequant<FMT_MXFP4>(W, out, sm);
    else launch_dequant<FMT_INT4>(W, out, sm);
    return hip_status("dequant launch");
}

int w4_mx_dot_device(const w4_matrix *A, const uint8_t *b_codes, const uint8_t *b_scales, int64_t m, float *out,
                     void *stream) {
    w4::clear_error();
    int st = check_matrix(A, "A");
    if (st) return st;
    if (A->format != W4_FMT_MXFP4_E8M0S32) return fail(W4_ERR_LAYOUT, "A must be MXFP4");
    if (A->groups != 1) return fail(W4_ERR_INVALID_ARG, "A must have groups == 1");
    if (A->n % 16 || A->k % 128 || m < 16 || m % 16 || m > (1 << 20))
        return fail(W4_ERR_UNSUPPORTED, "needs n and m multiples of 16 and k a multiple of 128");
    if ((uint64_t)m * (uint64_t)A->k >= (1ull << 31)) return fail(W4_ERR_UNSUPPORTED, "B too large");
    if (!b_codes || !b_scales || !out) return fail(W4_ERR_INVALID_ARG, "null B or out");
    if (!aligned(b_codes, 16) || !aligned(out, 4)) return fail(W4_ERR_ALIGNMENT, "B codes / out misaligned");
    (void)hipGetLastError();
    launch_mx_dot(A->codes, scale_base(A), row_layout(A), b_codes, b_scales, out, (int)A->n, (int)m, (int)A->k,
                  (hipStream_t)stream);
    return hip_status("mx dot launch");
}

#ifndef W4_SR_UNROLL
#define W4_SR_UNROLL 1
#endif
#ifndef W4_SR_BLOCKS
#define W4_SR_BLOCKS ((size_t)1 << 30)
#endif
int w4_bench_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
    w4::clear_error();
    if (!src || !sink) return fail(W4_ERR_INVALID_ARG, "null src or sink");
    if (bytes == 0 || bytes % 16) return fail(W4_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
    if (!aligned(src, 16) || !aligned(sink, 4)) return fail(W4_ERR_ALIGNMENT, "src not 16-byte aligned");
    const size_t n16 = bytes / 16;
    // W4_SR_UNROLL loads per thread, at most W4_SR_BLOCKS blocks of 256 threads: one
    // 16-byte load per thread in as many one-shot blocks as the buffer needs
    // streams fastest (measured against 2-16 loads per thread and grid-stride
    // grids of 1-8 K blocks: 6.6 against 5.4-6.4 TB/s at 4 GiB, 3.3 against
    // 2.0-3.1 TB/s at 11.8 MB)
    size_t blocks = (n16 + W4_SR_UNROLL * 256 - 1) / (W4_SR_UNROLL * 256);
    if (blocks > W4_SR_BLOCKS) blocks = W4_SR_BLOCKS;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_stream_read<W4_SR_UNROLL>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint4 *)src, n16, sink);
    return hip_status("stream read launch");
}

size_t moe_w4a16_workspace_bytes(const moe_w4a16_layer *L, int64_t T) {
    MoEPlan p{};
    if (check_layer(L, T, p) != W4_OK) return 0;
    return p.total;
}

int moe_w4a16_forward(const moe_w4a16_layer *L, const uint16_t *x, int64_t T, uint16_t *y, int32_t *topk_ids,
                      float *topk_w, void *ws, size_t ws_bytes, void *stream) {
    w4::clear_error();
    return run_moe(L, x, T, nullptr, nullptr, y, topk_ids, topk_w, ws, ws_bytes, stream);
}

int moe_w4a16_forward_timed(const moe_w4a16_layer *L, const uint16_t *x, int64_t T, uint16_t *y, int32_t *topk_ids,
                            float *topk_w, void *ws, size_t ws_bytes, void *stream, void *const *events,
                            int32_t n_events) {
    w4::clear_error();
    if (!events) return fail(W4_ERR_INVALID_ARG, "null events");
    return run_moe(L, x, T, nullptr, nullptr, y, topk_ids, topk_w, ws, ws_bytes, stream, events, n_events);
}

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch[MAX_DEVICES] = {};

// Device address of the current device's scratch array, looked up once per
// device (with that device current) and kept.
int scratch_of_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(W4_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= MAX_DEVICES) return fail(W4_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(W4_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return W4_OK;
}
}  // namespace

int moe_w4a16_forward_noalloc(const moe_w4a16_layer *L, const uint16_t *x, int64_t T, uint16_t *y,
                              int32_t *topk_ids, float *topk_w, void *stream) {
    w4::clear_error();
    MoEPlan p{};
    int st = check_layer(L, T, p);
    if (st) return st;
    if (p.total > W4_NOALLOC_SCRATCH_BYTES)
        return fail(W4_ERR_WORKSPACE, "T=%lld needs %zu bytes of workspace, more than the %zu-byte scratch of the "
                                      "no-allocation entry point (use moe_w4a16_forward with a workspace)",
                    (long long)T, p.total, (size_t)W4_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if ((st = scratch_of_current_device(&ws))) return st;
    return run_moe(L, x, T, nullptr, nullptr, y, topk_ids, topk_w, ws, W4_NOALLOC_SCRATCH_BYTES, stream);
}

int moe_w4a16_stage_count(const moe_w4a16_layer *L, int64_t T) {
    MoEPlan p{};
    if (check_layer(L, T, p) != W4_OK) return 0;
    return stage_count(p);
}

int moe_w4a16_experts(const moe_w4a16_layer *L, const uint16_t *x, int64_t T, const int32_t *ids, const float *w,
                      uint16_t *y, void *ws, size_t ws_bytes, void *stream) {
    w4::clear_error();
    if (!ids) return fail(W4_ERR_INVALID_ARG, "null ids");
    return run_moe(L, x, T, ids, w, y, nullptr, nullptr, ws, ws_bytes, stream);
}

}  // extern "C"
