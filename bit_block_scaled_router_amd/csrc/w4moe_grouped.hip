// Batched-decode path of the MoE layer (T tokens at once): the (token, slot)
// pairs are grouped by expert so that each active expert's weights are read
// once per step, and groups of at least W4_MFMA_MIN tokens run on MFMA.
//
//   k_moe_route_group  one block: top-k + routing weights per token (as in the
//                      single-token path), then a counting sort of the pairs by
//                      expert; writes the group table and the pair lists.
//   k_moe_gw13         per (group, 16-row tile): gate/up rows of the group's
//                      expert against the group's token activations, SiLU*up
//                      -> h[pair], stored as two bf16 arrays h_hi + h_lo (the
//                      fp32 value truncated, then its rounded residual).  MFMA
//                      for big groups (K split over the block's waves,
//                      fixed-order LDS sum), VALU otherwise.
//   k_moe_gw2          per (group, 64-row tile): down projection of the group's
//                      h rows -> out[pair][row] (fp32, unscaled).
//   k_moe_gcombine     y[t] = sum_j w[t][j] out[t*k+j] + sigma_t out[shared t],
//                      slots in order, one rounding to bf16.
//
// MFMA operands: the per-16 FP16 scale cannot be folded into a coarser
// hardware block scale without losing accuracy (lynn-engine README, status
// notes P18/P52), so each dequantised weight code*s is split exactly into two
// bf16 terms (split_scale) and both are multiplied by the bf16 activations;
// the down projection multiplies both weight terms by both h terms.
// Placement of pairs inside a group does not affect any result: every MFMA
// column and every VALU token is computed independently, and the combine reads
// pairs by (token, slot).
// Sources: lynn-engine README, R5 notes (tokens_per_expert grouping, inverse
// scatter to [T, top_k, N]); status notes P85-P92 (per-16 scale applied
// exactly, split-16); "Lynn Engine" article, "2. MoE 优化" (grouped kernel).
#include "w4moe_device.h"
#include "w4moe_grouped.h"

#include <hip/hip_ext.h>
#include <type_traits>
#include <hip/hip_runtime.h>

namespace w4k {

// k-steps (32 elements per lane each) the VALU small-group paths keep in registers
constexpr int KS_VALU = 2;
// waves per block of the multi-block ranking (two tokens per wave)
constexpr int RG_WAVES = 2;
constexpr int RG_TOKENS = 2 * RG_WAVES;
// 128-wide K chunks per wave whose weights the batched W13 launch requests at once
#ifndef W4_GW_CPW
#define W4_GW_CPW 4
#endif
constexpr int GW_CPW = W4_GW_CPW;
#ifndef W4_GW_MINBLK
#define W4_GW_MINBLK 3  // blocks per CU the batched W13 / W2 kernels are compiled to fit
#endif                  // (W2 with I > 512, int4 layers, and layers with a bf16 shared expert
                        // fit 2 or 1: fitting 3 would spill)

// ================================================================= route + group

// Exclusive scans over the experts' pair counts cnt[E] by one wave: off[e] =
// where expert e's pair list starts; the group table lists the experts with
// pairs (grp[0] = their number).  Lane l owns experts l*PL .. l*PL+PL-1; the
// counts (sums < 2^17) and the has-pairs flags (sums < 2^11) share one 32-bit
// scan.  ORDER = false: groups in expert order.  ORDER = true: by size class,
// groups of at least 16 pairs, then of at least `mid`, then the rest (expert
// order within a class), so that the expert launches, which walk their units in
// table order, start the longest units first.
template <int PL, bool ORDER>
__device__ __forceinline__ void scan_groups(const int *cnt, int *off, int32_t *grp, int E, int Gmax, int lane,
                                            int mid = 0) {
    constexpr int GSH = 17, CSH = 11, BIG = 16;
    auto cls = [&](int c) { return ORDER ? (c >= BIG ? 1 : 0) + (c >= mid && c < BIG ? (1 << CSH) : 0) : 0; };
    int c[PL], loc = 0, cl = 0;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int e = lane * PL + i;
        c[i] = e < E ? cnt[e] : 0;
        loc += c[i] + (c[i] > 0 ? (1 << GSH) : 0);
        cl += cls(c[i]);
    }
    const int inc = wave_incl_scan(loc);
    int run = inc - loc;
    int crun = 0, n0 = 0, n1 = 0;
    if constexpr (ORDER) {  // class ranks: large groups in the low field, middle ones above
        const int cinc = wave_incl_scan(cl);
        crun = cinc - cl;
        const int tot = __builtin_amdgcn_readlane(cinc, 63);
        n0 = tot & ((1 << CSH) - 1);
        n1 = tot >> CSH;
    }
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int e = lane * PL + i;
        const int ex = run & ((1 << GSH) - 1), gex = run >> GSH;
        if (e < E) off[e] = ex;
        if (c[i] > 0) {
            int g = gex;
            if constexpr (ORDER) {
                const int r0 = crun & ((1 << CSH) - 1), r1 = crun >> CSH;
                g = c[i] >= BIG ? r0 : c[i] >= mid ? n0 + r1 : n0 + n1 + (gex - r0 - r1);
            }
            grp[1 + g] = e;
            grp[1 + Gmax + g] = ex;
            grp[1 + 2 * Gmax + g] = c[i];
        }
        run += c[i] + (c[i] > 0 ? (1 << GSH) : 0);
        crun += cls(c[i]);
    }
    if (lane == 63) grp[0] = inc >> GSH;
}

// Top-k and routing weights of tokens t and t2 (t2 < 0: none) by one wave,
// their rankings interleaved; lanes j < K write the j-th id and weight of each
// and get them back in e[0], e[1] (-1 for lanes >= K, invalid supplied ids and
// the missing token).
template <int PL>
__device__ __forceinline__ void route_tokens2(const GroupArgs &a, int t, int t2, int lane, int (&e)[2]) {
    const int K = a.K;
    const int tt[2] = {t, t2};
    if (a.route) {
        const float *lg[2] = {a.logits + (size_t)t * a.lstride, a.logits + (size_t)(t2 >= 0 ? t2 : t) * a.lstride};
        int my_id[2];
        float my_val[2];
        wave_topk_n<PL, 2>(lg, a.bias, a.E, t2 >= 0 ? 2 : 1, K, 0, my_id, my_val);
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            e[n] = -1;
            if (tt[n] < 0) continue;
            const float vmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_val[n]), 0));
            const float ex = lane < K ? expf(my_val[n] - vmax) : 0.f;
            const float sum = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(group_sum<64>(ex)), 63));
            if (lane < K) {
                const float w = ex / sum;
                const int o = tt[n] * K + lane;
                a.ids_ws[o] = my_id[n];
                a.w_ws[o] = w;
                if (a.ids_user) a.ids_user[o] = my_id[n];
                if (a.w_user) a.w_user[o] = w;
                e[n] = my_id[n];
            }
        }
        return;
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        e[n] = -1;
        if (tt[n] < 0 || lane >= K) continue;
        const int v = a.ids_in[tt[n] * K + lane];
        e[n] = (v >= 0 && v < a.E) ? v : -1;  // invalid ids join no group
    }
}

// Counting sort of the pairs by expert, by the whole block, from the expert of
// every pair in LDS e_of [P] (-1: the pair joins no group); cnt [E], off [E] and
// pos [P] are LDS scratch.  Writes the group table and the pair lists.
template <int PL>
__device__ __forceinline__ void group_pairs(const GroupArgs &a, int *cnt, int *off, const int *e_of, int *pos) {
    const int E = a.E, T = a.T, P = a.P;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int i = tid; i < E; i += blockDim.x) cnt[i] = 0;
    __syncthreads();
    // position of each pair inside its expert's group (LDS atomics: the order
    // inside a group is free, see the file header)
    for (int p = tid; p < P; p += blockDim.x) {
        const int e = e_of[p];
        pos[p] = e >= 0 ? atomicAdd(&cnt[e], 1) : -1;
    }
    __syncthreads();
    // exclusive scans over the experts: where each expert's pair list starts,
    // and the group index of each active expert (groups by size class, largest first)
    if (wv == 0) scan_groups<PL, true>(cnt, off, a.grp, E, a.Gmax, lane, a.mfma_min);
    __syncthreads();
    for (int p = tid; p < P; p += blockDim.x) {
        const int e = e_of[p];
        if (e >= 0) a.pairs[off[e] + pos[p]] = p;
    }
    for (int t = tid; t < T; t += blockDim.x) a.pairs[P + t] = P + t;
}

template <int PL>
__global__ __launch_bounds__(1024) void k_moe_route_group(GroupArgs a) {
    extern __shared__ int g_lds[];
    const int E = a.E, K = a.K, T = a.T, P = a.P;
    int *cnt = g_lds;        // [E]
    int *off = cnt + E;      // [E]
    int *e_of = off + E;     // [P]
    int *pos = e_of + P;     // [P]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), nw = blockDim.x >> 6;

    for (int t = wv; t < T; t += 2 * nw) {  // tokens t and t + nw, ranked together
        const int t2 = t + nw < T ? t + nw : -1;
        int e[2];
        route_tokens2<PL>(a, t, t2, lane, e);
        if (lane < K) {
            e_of[t * K + lane] = e[0];
            if (t2 >= 0) e_of[t2 * K + lane] = e[1];
        }
    }
    group_pairs<PL>(a, cnt, off, e_of, pos);
}

// Routed batches: the top-k ranking is spread over ceil(T / RG_TOKENS) blocks
// (two tokens per wave, so that no CU ranks more than RG_TOKENS tokens), and
// the last block to finish groups the pairs.  Each block publishes its
// tokens' ids (release fence, then one device-scope atomic increment of the
// arrival counter `arrive`, which the router launch before this one set to
// zero); the block that reads gridDim.x - 1 from the counter knows that every
// id is written, acquires them, sets the counter back to zero and runs the
// counting sort.  No block waits for another, so the grid drains whatever the
// schedule.
template <int PL>
__global__ __launch_bounds__(64 * RG_WAVES) void k_moe_rank_group(GroupArgs a, int32_t *arrive) {
    extern __shared__ int g_lds[];
    __shared__ int s_last;
    const int E = a.E, T = a.T, P = a.P;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = ((int)blockIdx.x * RG_WAVES + wv) * 2;  // this wave's tokens t, t + 1
    if (t < T) {
        int e[2];
        route_tokens2<PL>(a, t, t + 1 < T ? t + 1 : -1, lane, e);
    }
    __syncthreads();
    if (tid == 0) {
        __threadfence();  // release: this block's ids and weights before its arrival
        s_last = atomicAdd(arrive, 1) == (int)gridDim.x - 1;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();  // acquire: every block's ids
    int *cnt = g_lds;     // [E]
    int *off = cnt + E;   // [E]
    int *e_of = off + E;  // [P]
    int *pos = e_of + P;  // [P]
    for (int p = tid; p < P; p += blockDim.x) e_of[p] = a.ids_ws[p];
    if (tid == 0) *arrive = 0;  // every block has arrived: ready for a launch without the router before it
    __syncthreads();
    group_pairs<PL>(a, cnt, off, e_of, pos);
}

// Multi-launch grouping: r.tpb tokens per block (4 waves), top-k and
// weights per token, the expert of each pair, and the block's expert histogram
// (LDS counts; only the totals are used, so the order of the increments is free).
template <int PL>
__global__ __launch_bounds__(256) void k_route_topk(RouteArgs r) {
    __shared__ int hist[1024];
    const GroupArgs &a = r.g;
    const int E = a.E, K = a.K;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int i = tid; i < E; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    const int t0 = blockIdx.x * r.tpb;
    const int t1 = min(t0 + r.tpb, a.T);
    for (int t = t0 + wv; t < t1; t += 8) {  // tokens t and t + 4, ranked together
        const int t2 = t + 4 < t1 ? t + 4 : -1;
        int e[2];
        route_tokens2<PL>(a, t, t2, lane, e);
        if (lane < K) {
            r.e_of[t * K + lane] = e[0];
            if (e[0] >= 0) atomicAdd(&hist[e[0]], 1);
            if (t2 >= 0) {
                r.e_of[t2 * K + lane] = e[1];
                if (e[1] >= 0) atomicAdd(&hist[e[1]], 1);
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < E; i += blockDim.x) r.cntb[(size_t)blockIdx.x * E + i] = hist[i];
}

// One block: per expert, the exclusive scan of the block histograms (cntb ->
// cbase: each block's base inside the expert's list) and the expert's total;
// then the group table and each expert's list start.
__global__ __launch_bounds__(1024) void k_route_scan(RouteArgs r) {
    __shared__ int tot[1024], off[1024], part[1024];
    const int E = r.g.E, Gmax = r.g.Gmax;
    const int tid = threadIdx.x;
    // F threads per expert, each owning a contiguous range of the blocks: the
    // range sums first (16 loads in flight), then each thread rewrites its range
    // as running sums from the sums of the ranges before it
    int F = 1;
    while (2 * F * E <= (int)blockDim.x && F < 16) F *= 2;
    const int e = tid % E, f = tid / E;
    const int per = (r.nblk + F - 1) / F, b_lo = f * per, b_hi = min(r.nblk, b_lo + per);
    const bool act = f < F;
    int sum = 0;
    if (act) {
        for (int b0 = b_lo; b0 < b_hi; b0 += 16) {
            int c[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) c[i] = b0 + i < b_hi ? r.cntb[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) sum += c[i];
        }
        part[f * E + e] = sum;
    }
    __syncthreads();
    if (act) {
        int run = 0;
        for (int g = 0; g < f; ++g) run += part[g * E + e];
        for (int b0 = b_lo; b0 < b_hi; b0 += 16) {
            int c[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) c[i] = b0 + i < b_hi ? r.cntb[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (b0 + i < b_hi) {
                    r.cbase[(size_t)(b0 + i) * E + e] = run;
                    run += c[i];
                }
        }
        if (f == F - 1) tot[e] = run;
    }
    __syncthreads();
    if (tid < 64) {
        scan_groups<16, false>(tot, off, r.g.grp, E, Gmax, tid);  // (any E up to 1024; column tiles need expert order)
        // the routed groups' 64-column tiles in group order (groups = experts with pairs)
        int crun = 0, grun = 0;
        for (int base = 0; base < E; base += 64) {
            const int e = base + tid;
            const int c = e < E ? tot[e] : 0;
            const int nct = (c + 63) / 64, nz = c > 0 ? 1 : 0;
            int inc = nct, ginc = nz;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int u = __shfl_up(inc, d), gu = __shfl_up(ginc, d);
                if (tid >= d) inc += u, ginc += gu;
            }
            const int c0 = crun + inc - nct, g = grun + ginc - nz;
            for (int j = 0; j < nct; ++j) {
                r.ctg[2 * (c0 + j)] = g;
                r.ctg[2 * (c0 + j) + 1] = 64 * j;
            }
            crun += __shfl(inc, 63);
            grun += __shfl(ginc, 63);
        }
        if (tid == 0) r.g.grp[1 + 3 * Gmax] = crun;
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) r.off_e[e] = off[e];
}

// Same blocks as k_route_topk: each pair goes to off_e[e] + the block's base
// for e + its rank among the block's earlier pairs of expert e.
__global__ __launch_bounds__(256) void k_route_scatter(RouteArgs r) {
    __shared__ int es[ROUTE_MAX_TPB * 16];
    const GroupArgs &a = r.g;
    const int E = a.E, K = a.K;
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * r.tpb;
    const int t1 = min(t0 + r.tpb, a.T);
    const int p0 = t0 * K, np = (t1 - t0) * K;
    for (int i = tid; i < np; i += blockDim.x) es[i] = r.e_of[p0 + i];
    __syncthreads();
    for (int i = tid; i < np; i += blockDim.x) {
        const int e = es[i];
        if (e < 0) continue;
        int rank = 0;
        for (int q = 0; q < i; ++q) rank += es[q] == e ? 1 : 0;
        a.pairs[r.off_e[e] + r.cbase[(size_t)blockIdx.x * E + e] + rank] = p0 + i;
    }
    for (int t = t0 + tid; t < t1; t += blockDim.x) a.pairs[a.P + t] = a.P + t;
}

// Which expert and which pairs a work unit covers.  Group slot 0 is the shared
// expert (pairs P .. P+T-1, one per token) when there is one; the routed groups
// follow in the order of the group table.
template <typename S>
struct GroupView {
    const uint8_t *codes;
    const S *scales;
    int off, m;       // first entry in the pair list, number of pairs
    int e;            // expert id (-1: the shared expert)
    uint32_t cs, ss;  // row strides (bytes) of the group's codes and scales
    size_t mat_codes, mat_scales;  // bytes of one matrix: n * cs, n * ss
};

// n: rows per matrix; rl / srl: row strides of the routed / shared matrices
template <typename S>
__device__ __forceinline__ GroupView<S> group_view(const int32_t *grp, int gs, int Gmax, int P, int T, int n,
                                                   const uint8_t *codes, const void *scales, RowLayout rl,
                                                   const uint8_t *s_codes, const void *s_scales, RowLayout srl) {
    GroupView<S> v{};
    if (s_codes != nullptr) {
        if (gs == 0) {
            v.codes = s_codes, v.scales = reinterpret_cast<const S *>(s_scales), v.off = P, v.m = T, v.e = -1;
            v.cs = srl.cs, v.ss = srl.ss;
            v.mat_codes = (size_t)n * srl.cs, v.mat_scales = (size_t)n * srl.ss;
            return v;
        }
        --gs;
    }
    const int e = ld_uniform(grp, 1 + gs);
    v.e = e;
    v.off = ld_uniform(grp, 1 + Gmax + gs);
    v.m = ld_uniform(grp, 1 + 2 * Gmax + gs);
    v.cs = rl.cs, v.ss = rl.ss;
    v.mat_codes = (size_t)n * rl.cs, v.mat_scales = (size_t)n * rl.ss;
    v.codes = codes + (size_t)e * v.mat_codes;
    v.scales = reinterpret_cast<const S *>(static_cast<const uint8_t *>(scales) + (size_t)e * v.mat_scales);
    return v;
}

// number of work units: (routed groups + shared) x row tiles
__device__ __forceinline__ int unit_count(const int32_t *grp, bool shared, int tiles) {
    return (ld_uniform(grp, 0) + (shared ? 1 : 0)) * tiles;
}

__device__ __forceinline__ int token_of(int p, int P, int K) { return p < P ? p / K : p - P; }

// ================================================================= grouped W13 + SiLU

// One work unit of the W13 launch: group slot gs, gate rows 16*tile .. +16 (and
// the matching up rows).  FMT: E2M1 (FP16 scale per 16: every weight is two
// exact bf16 terms) or NVFP4 (UE4M3 scale per 16: code x scale has at most 6
// significant bits, one exact bf16 term; the matrix's global scale multiplies
// the gate and up sums).  SB: the layer's shared expert is bf16 (its rows are
// the MFMA operands; a separate instantiation keeps the 4-bit-only kernels'
// register budget).
template <int FMT, int L, bool SB>
__device__ __forceinline__ void gw13_unit(const GW13Args &a, int gs, int tile, float (*red)[16][64]) {
    using SC = typename std::conditional<FMT == FMT_NVFP4, uint8_t, uint16_t>::type;
    constexpr int RG = 64 / L;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int H = a.H, I = a.I;
    const GroupView<SC> gv = group_view<SC>(a.grp, gs, a.Gmax, a.P, a.T, 2 * I, a.codes, a.scales, a.rl, a.s_codes,
                                            a.s_scales, a.s_rl);
    const uint32_t cs = gv.cs, ss = gv.ss;  // row strides (bytes)
    // a bf16 shared expert: its rows are the MFMA operands themselves (the
    // MFMA branch takes every size of that group)
    const bool sbf = SB && gv.e < 0;
    const Buf cb = make_buf(gv.codes, (uint32_t)gv.mat_codes);
    const Buf sb = make_buf(gv.scales, sbf ? 0u : (uint32_t)gv.mat_scales);
    float gsc = 1.f;  // NVFP4 global scale of the matrix
    if constexpr (FMT == FMT_NVFP4) gsc = sbf ? 1.f : gv.e < 0 ? ld_uniform(a.s_gs, 0) : ld_uniform(a.gs, gv.e);
    const int i0 = tile * 16;  // first gate row of the tile
    const int *plist = a.pairs + gv.off;

    if (gv.m >= a.mfma_min || sbf) {
        auto mfma = [&](auto SBFc) {
            constexpr bool SBF = decltype(SBFc)::value;
            // ---- MFMA: 16 gate + 16 up rows x 16-token column tiles; the 128-wide K
            // chunks are dealt round-robin to the 4 waves and summed in wave order.
            // The weights are the A operand (lane (r, q) = (lane % 16, lane / 16)
            // ends with rows 4q .. 4q + 3 of its column token r), except for int4
            // codes: there the activations are A and the codes B, so the lane ends
            // with tokens 4q .. 4q + 3 of the one row r and needs one group scale
            // instead of four.
            constexpr bool TR = FMT == FMT_INT4 && !SBF;
            const int r = lane & 15, q = lane >> 4;
            const bool rg_ok = i0 + r < I;
            const uint32_t rowg = (uint32_t)(i0 + r), rowu = (uint32_t)(I + i0 + r);
            const int nchunks = H >> 7;
            const Buf xall = make_buf(a.x, (uint32_t)a.T * (uint32_t)H * 2u);
            for (int n0 = 0; n0 < gv.m; n0 += 32) {
                // two 16-column tiles: pairs n0 + lane%16 and n0 + 16 + lane%16
                int pr[2], tk[2];
                bool pv[2];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int idx = n0 + nt * 16 + r;
                    pv[nt] = idx < gv.m;
                    pr[nt] = pv[nt] ? plist[idx] : 0;
                    tk[nt] = token_of(pr[nt], a.P, a.K);
                }
                const bool two = n0 + 16 < gv.m;  // second column tile in use (uniform)
                f32x4 ag[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
                f32x4 au[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
                for (int cb0 = wv; cb0 < nchunks; cb0 += 4 * GW_CPW) {
                    // the codes and scales of up to GW_CPW of this wave's chunks are
                    // requested before the first of them is multiplied
                    uint4 cgv[GW_CPW], cuv[GW_CPW];
                    uint32_t sgv[GW_CPW], suv[GW_CPW];
                    if constexpr (!SBF) {
#pragma unroll
                        for (int i = 0; i < GW_CPW; ++i) {
                            const int c = cb0 + 4 * i;
                            const bool cv = rg_ok && c < nchunks;
                            const int k0 = c * 128 + 32 * q;
                            cgv[i] = ld128(cb, cv ? rowg * cs + (uint32_t)(k0 >> 1) : OOB);
                            cuv[i] = ld128(cb, cv ? rowu * cs + (uint32_t)(k0 >> 1) : OOB);
                            if constexpr (FMT != FMT_INT4) {
                                sgv[i] = ld_scales<FMT>(sb, cv ? rowg * ss + scale_col<FMT>(k0) : OOB);
                                suv[i] = ld_scales<FMT>(sb, cv ? rowu * ss + scale_col<FMT>(k0) : OOB);
                            }
                        }
                    }
#pragma unroll
                    for (int ci = 0; ci < GW_CPW; ++ci) {
                        const int c = cb0 + 4 * ci;
                        if (c >= nchunks) break;
                        const int k0 = c * 128 + 32 * q;  // this lane's 32 elements
                        // B: 32 activations of each column token
                        uint4 xb[2][4];
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) {
                            const uint32_t xo = (uint32_t)(tk[nt] * H + k0) * 2u;
#pragma unroll
                            for (int s = 0; s < 4; ++s)
                                xb[nt][s] = (nt == 0 || two) ? ld128(xall, pv[nt] ? xo + 16u * s : OOB)
                                                             : make_uint4(0, 0, 0, 0);
                        }
                        if constexpr (SBF) {  // bf16 rows, 8 weights per MFMA step
                            const uint32_t rb = cs;
#pragma unroll
                            for (int s = 0; s < 4; ++s) {
                                const uint32_t ko = (uint32_t)(k0 + 8 * s) * 2u;
                                const bf16x8 wg = __builtin_bit_cast(bf16x8, ld128(cb, rg_ok ? rowg * rb + ko : OOB));
                                const bf16x8 wu = __builtin_bit_cast(bf16x8, ld128(cb, rg_ok ? rowu * rb + ko : OOB));
#pragma unroll
                                for (int nt = 0; nt < 2; ++nt) {
                                    if (nt == 1 && !two) break;
                                    const bf16x8 b = __builtin_bit_cast(bf16x8, xb[nt][s]);
                                    ag[nt] = mfma16x16x32(wg, b, ag[nt]);
                                    au[nt] = mfma16x16x32(wu, b, au[nt]);
                                }
                            }
                            continue;
                        }
                        const uint4 cg = cgv[ci], cu = cuv[ci];
                        if constexpr (FMT == FMT_INT4) {
                            // the chunk is one scale group: MFMAs on the raw offset codes
                            // u = q + 8 (exact bf16) and on 8 (the offset), then the
                            // difference times the scale of the lane's row
                            const float so_g = f16_bits_to_f32(ld16(sb, rg_ok ? rowg * ss + (uint32_t)c * 2u : OOB));
                            const float so_u = f16_bits_to_f32(ld16(sb, rg_ok ? rowu * ss + (uint32_t)c * 2u : OOB));
                            const uint32_t cgw[4] = {cg.x, cg.y, cg.z, cg.w}, cuw[4] = {cu.x, cu.y, cu.z, cu.w};
                            f32x4 tg[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, tu[2] = {tg[0], tg[0]},
                                  tc[2] = {tg[0], tg[0]};
#pragma unroll
                            for (int s = 0; s < 4; ++s) {
                                const bf16x8 ug = u4x8_bf16(cgw[s]), uu = u4x8_bf16(cuw[s]);
                                // both column tiles unconditionally (a missing second tile has
                                // zero activations): the chunk's sums are read right after
                                // these MFMAs, and straight-line code keeps the compiler's
                                // MFMA-result wait states in place (behind a branch they were
                                // not, and the first read saw a stale accumulator)
#pragma unroll
                                for (int nt = 0; nt < 2; ++nt) {
                                    const bf16x8 b = __builtin_bit_cast(bf16x8, xb[nt][s]);
                                    tg[nt] = mfma16x16x32(b, ug, tg[nt]);
                                    tu[nt] = mfma16x16x32(b, uu, tu[nt]);
                                    tc[nt] = mfma16x16x32(b, bf16x8_splat8(), tc[nt]);
                                }
                            }
#pragma unroll
                            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    ag[nt][j] = fmaf(so_g, tg[nt][j] - tc[nt][j], ag[nt][j]);
                                    au[nt][j] = fmaf(so_u, tu[nt][j] - tc[nt][j], au[nt][j]);
                                }
                            continue;
                        }
                        const uint32_t sg = sgv[ci], su = suv[ci];
                        const uint32_t cgw[4] = {cg.x, cg.y, cg.z, cg.w}, cuw[4] = {cu.x, cu.y, cu.z, cu.w};
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            if constexpr (FMT == FMT_NVFP4) {
                                const f32x2 sgv = block_scales2<FMT>(sg), suv = block_scales2<FMT>(su);
                                const bf16x8 ag1 = e2m1x8_scaled(cgw[s], s < 2 ? sgv.x : sgv.y);
                                const bf16x8 au1 = e2m1x8_scaled(cuw[s], s < 2 ? suv.x : suv.y);
#pragma unroll
                                for (int nt = 0; nt < 2; ++nt) {
                                    if (nt == 1 && !two) break;
                                    const bf16x8 b = __builtin_bit_cast(bf16x8, xb[nt][s]);
                                    ag[nt] = mfma16x16x32(ag1, b, ag[nt]);
                                    au[nt] = mfma16x16x32(au1, b, au[nt]);
                                }
                            } else {
                                float gh, gl, uh, ul;
                                split_scale(f16_bits_to_f32(s < 2 ? sg : (sg >> 16)), gh, gl);
                                split_scale(f16_bits_to_f32(s < 2 ? su : (su >> 16)), uh, ul);
                                bf16x8 agh, agl, auh, aul;
                                e2m1x8_split(cgw[s], gh, gl, agh, agl);
                                e2m1x8_split(cuw[s], uh, ul, auh, aul);
#pragma unroll
                                for (int nt = 0; nt < 2; ++nt) {
                                    if (nt == 1 && !two) break;
                                    const bf16x8 b = __builtin_bit_cast(bf16x8, xb[nt][s]);
                                    ag[nt] = mfma16x16x32(agh, b, ag[nt]);
                                    ag[nt] = mfma16x16x32(agl, b, ag[nt]);
                                    au[nt] = mfma16x16x32(auh, b, au[nt]);
                                    au[nt] = mfma16x16x32(aul, b, au[nt]);
                                }
                            }
                        }
                    }
                }
                // fixed-order sum of the four K partials
                if (wv > 0) {
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            red[wv - 1][nt * 8 + j][lane] = ag[nt][j];
                            red[wv - 1][nt * 8 + 4 + j][lane] = au[nt][j];
                        }
                }
                __syncthreads();
                if (wv == 0) {
#pragma unroll
                    for (int w = 0; w < 3; ++w)
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                ag[nt][j] += red[w][nt * 8 + j][lane];
                                au[nt][j] += red[w][nt * 8 + 4 + j][lane];
                            }
                    if constexpr (TR) {
                        // lane holds tokens 4q + j of each column tile for row i0 + r;
                        // the pair of column c was read by lane c
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const int p = __shfl(pr[nt], 4 * q + j, 64);
                                if (rg_ok && n0 + nt * 16 + 4 * q + j < gv.m) {
                                    const float gg = ag[nt][j], uu = au[nt][j];
                                    uint16_t bh, bl;
                                    split_bf16((gg / (1.f + expf(-gg))) * uu, bh, bl);
                                    const size_t o = (size_t)p * I + rowg;
                                    a.h_hi[o] = bh;
                                    a.h_lo[o] = bl;
                                }
                            }
                    } else {
                        // lane holds rows i0 + 4q + j of column r
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) {
                            const int idx = n0 + nt * 16 + r;
                            if (idx < gv.m) {
                                const int p = plist[idx];
                                float hv[4];
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    float gg = ag[nt][j], uu = au[nt][j];
                                    if constexpr (FMT == FMT_NVFP4) gg *= gsc, uu *= gsc;
                                    hv[j] = (gg / (1.f + expf(-gg))) * uu;
                                }
                                // I is a multiple of 128 (host check): rows i0 + 4q .. +3 all exist
                                uint16_t bh[4], bl[4];
#pragma unroll
                                for (int j = 0; j < 4; ++j) split_bf16(hv[j], bh[j], bl[j]);
                                const size_t o = (size_t)p * I + i0 + 4 * q;
                                *reinterpret_cast<uint2 *>(a.h_hi + o) =
                                    make_uint2(bh[0] | ((uint32_t)bh[1] << 16), bh[2] | ((uint32_t)bh[3] << 16));
                                *reinterpret_cast<uint2 *>(a.h_lo + o) =
                                    make_uint2(bl[0] | ((uint32_t)bl[1] << 16), bl[2] | ((uint32_t)bl[3] << 16));
                            }
                        }
                    }
                }
                __syncthreads();
            }
        };
        if constexpr (SB) {
            if (sbf) {
                mfma(std::true_type());
                return;
            }
        }
        mfma(std::false_type());
        return;
    }

    // ---- VALU (small groups): wave wv owns gate rows i0 + 4wv .. +4 and the
    // matching up rows; their codes are loaded once, then each token in turn.
    constexpr int NLG = RG >= 4 ? 1 : 4 / RG;  // load groups per wave
    const int lk = lane % L, rsub = lane / L;
    const int ks = (H + 32 * L - 1) / (32 * L);  // at most KS_VALU (checked by the host)
    uint4 cg[KS_VALU][NLG], cu[KS_VALU][NLG];
    uint32_t sg[KS_VALU][NLG], su[KS_VALU][NLG];
#pragma unroll
    for (int s = 0; s < KS_VALU; ++s)
#pragma unroll
        for (int l = 0; l < NLG; ++l) {
            const int k0 = 32 * (L * s + lk);
            const int i = i0 + 4 * wv + l * RG + rsub;
            const bool v = s < ks && k0 < H && i < I && (l * RG + rsub) < 4;
            const uint32_t rg = (uint32_t)i, ru = (uint32_t)(I + i);
            cg[s][l] = ld128(cb, v ? rg * cs + (uint32_t)(k0 >> 1) : OOB);
            cu[s][l] = ld128(cb, v ? ru * cs + (uint32_t)(k0 >> 1) : OOB);
            sg[s][l] = ld_scales<FMT>(sb, v ? rg * ss + scale_col<FMT>(k0) : OOB);
            su[s][l] = ld_scales<FMT>(sb, v ? ru * ss + scale_col<FMT>(k0) : OOB);
        }
    for (int idx = 0; idx < gv.m; ++idx) {
        if constexpr (FMT == FMT_INT4) {
            // keep the int4 decode inside the token loop: hoisted, every row's
            // decoded pairs stay live (about 300 registers, one block per CU)
#pragma unroll
            for (int s = 0; s < KS_VALU; ++s)
#pragma unroll
                for (int l = 0; l < NLG; ++l) {
                    asm volatile("" : "+v"(cg[s][l].x), "+v"(cg[s][l].y), "+v"(cg[s][l].z), "+v"(cg[s][l].w));
                    asm volatile("" : "+v"(cu[s][l].x), "+v"(cu[s][l].y), "+v"(cu[s][l].z), "+v"(cu[s][l].w));
                }
        }
        const int p = ld_uniform(plist, idx);
        const int t = token_of(p, a.P, a.K);
        const Buf xb = make_buf(a.x + (size_t)t * H, (uint32_t)H * 2u);
        float accg[NLG], accu[NLG];
#pragma unroll
        for (int l = 0; l < NLG; ++l) accg[l] = accu[l] = 0.f;
#pragma unroll
        for (int s = 0; s < KS_VALU; ++s) {
            if (s >= ks) break;
            const int k0 = 32 * (L * s + lk);
            XSlice<FMT> xs;
            load_xslice<FMT>(xs, xb, k0 < H ? (uint32_t)k0 * 2u : OOB);
            prep_xslice<FMT>(xs);
#pragma unroll
            for (int l = 0; l < NLG; ++l) {
                accg[l] = chunk_dot_bf16<FMT>(cg[s][l], sg[s][l], xs, accg[l]);
                accu[l] = chunk_dot_bf16<FMT>(cu[s][l], su[s][l], xs, accu[l]);
            }
        }
#pragma unroll
        for (int l = 0; l < NLG; ++l) {
            const float gg = group_sum<L>(accg[l]) * gsc;
            const float uu = group_sum<L>(accu[l]) * gsc;
            const int i = i0 + 4 * wv + l * RG + rsub;
            if (group_leader<L>(lane) && i < I && (l * RG + rsub) < 4) {
                uint16_t bh, bl;
                split_bf16((gg / (1.f + expf(-gg))) * uu, bh, bl);
                a.h_hi[(size_t)p * I + i] = bh;
                a.h_lo[(size_t)p * I + i] = bl;
            }
        }
    }
}

// Blocks walk the work units (group slot x row tile) with a grid stride, so the
// grid needs no bound on the number of active experts.
template <int FMT, int L, bool SB>
__global__ __launch_bounds__(256, FMT == FMT_INT4 ? 1 : SB ? 2 : W4_GW_MINBLK) void k_moe_gw13(GW13Args a) {
    __shared__ float red[3][16][64];  // MFMA K-split partials of waves 1..3
    const int nu = unit_count(a.grp, a.s_codes != nullptr, a.tiles);
    for (int u = blockIdx.x; u < nu; u += gridDim.x) {
        const int gs = u / a.tiles;
        gw13_unit<FMT, L, SB>(a, gs, u - gs * a.tiles, red);
    }
}

// ================================================================= grouped W2

// One work unit of the down launch: group slot gs, output rows 64*tile .. +64.
// FMT, SB as in gw13_unit (NVFP4: one bf16 weight term, sums times the global scale).
template <int FMT, int L, bool SB>
__device__ __forceinline__ void gw2_unit(const GW2Args &a, int gs, int tile, float (*red)[4][8][64]) {
    using SC = typename std::conditional<FMT == FMT_NVFP4, uint8_t, uint16_t>::type;
    constexpr int RG = 64 / L;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int H = a.H, I = a.I;
    const GroupView<SC> gv = group_view<SC>(a.grp, gs, a.Gmax, a.P, a.T, H, a.codes, a.scales, a.rl, a.s_codes,
                                            a.s_scales, a.s_rl);
    const uint32_t cs = gv.cs, ss = gv.ss;  // row strides (bytes)
    const bool sbf = SB && gv.e < 0;  // bf16 shared expert (MFMA branch at every size)
    const Buf cb = make_buf(gv.codes, (uint32_t)gv.mat_codes);
    const Buf sb = make_buf(gv.scales, sbf ? 0u : (uint32_t)gv.mat_scales);
    float gsc = 1.f;  // NVFP4 global scale of the matrix
    if constexpr (FMT == FMT_NVFP4) gsc = sbf ? 1.f : gv.e < 0 ? ld_uniform(a.s_gs, 0) : ld_uniform(a.gs, gv.e);
    const int *plist = a.pairs + gv.off;
    const uint32_t hbytes = (uint32_t)(a.P + a.T) * (uint32_t)I * 2u;
    const Buf hhi = make_buf(a.h_hi, hbytes), hlo = make_buf(a.h_lo, hbytes);

    if (gv.m >= a.mfma_min || sbf) {
        auto mfma = [&](auto SBFc) {
            constexpr bool SBF = decltype(SBFc)::value;
            // ---- MFMA: the 64 rows of the unit x up to 32 columns per pass.  The
            // 128-wide K chunks are dealt round-robin to the 4 waves, so each h
            // element is read once per unit; each wave multiplies its chunk into all
            // four 16-row tiles, and the partials are summed in wave order via LDS.
            // int4 codes are the B operand (h is A), so a lane's four sums share
            // one row and its group scale, as in gw13_unit.
            constexpr bool TR = FMT == FMT_INT4 && !SBF;
            const int r = lane & 15, q = lane >> 4;
            const int nchunks = I >> 7;
            const int u0 = tile * 64;  // first row of the unit
            for (int n0 = 0; n0 < gv.m; n0 += 32) {
                int pr[2];
                bool pv[2];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int idx = n0 + nt * 16 + r;
                    pv[nt] = idx < gv.m;
                    pr[nt] = pv[nt] ? plist[idx] : 0;
                }
                const bool two = n0 + 16 < gv.m;  // second column tile in use (uniform)
                f32x4 acc[4][2];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) acc[rt][0] = acc[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
                for (int c = wv; c < nchunks; c += 4) {
                    const int k0 = c * 128 + 32 * q;
                    uint4 cw[4];
                    uint32_t sc[4];
                    if constexpr (!SBF) {
#pragma unroll
                        for (int rt = 0; rt < 4; ++rt) {
                            const int rr = u0 + 16 * rt + r;
                            const bool rv = rr < H;
                            cw[rt] = ld128(cb, rv ? (uint32_t)rr * cs + (uint32_t)(k0 >> 1) : OOB);
                            sc[rt] = ld_scales<FMT>(sb, rv ? (uint32_t)rr * ss + scale_col<FMT>(k0) : OOB);
                        }
                    }
                    uint4 bh[2][4], bl[2][4];
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const uint32_t ho = (uint32_t)(pr[nt] * I + k0) * 2u;
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            const bool on = nt == 0 || two;
                            bh[nt][s] = on ? ld128(hhi, pv[nt] ? ho + 16u * s : OOB) : make_uint4(0, 0, 0, 0);
                            bl[nt][s] = on ? ld128(hlo, pv[nt] ? ho + 16u * s : OOB) : make_uint4(0, 0, 0, 0);
                        }
                    }
                    if constexpr (SBF) {  // bf16 rows: the weights are the operands; h as hi + lo
#pragma unroll
                        for (int rt = 0; rt < 4; ++rt) {
                            const int rr = u0 + 16 * rt + r;
                            const bool rv = rr < H;
#pragma unroll
                            for (int s = 0; s < 4; ++s) {
                                const uint32_t o = (uint32_t)rr * cs + (uint32_t)(k0 + 8 * s) * 2u;
                                const bf16x8 w = __builtin_bit_cast(bf16x8, ld128(cb, rv ? o : OOB));
#pragma unroll
                                for (int nt = 0; nt < 2; ++nt) {
                                    if (nt == 1 && !two) break;
                                    acc[rt][nt] = mfma16x16x32(w, __builtin_bit_cast(bf16x8, bh[nt][s]), acc[rt][nt]);
                                    acc[rt][nt] = mfma16x16x32(w, __builtin_bit_cast(bf16x8, bl[nt][s]), acc[rt][nt]);
                                }
                            }
                        }
                        continue;
                    }
                    if constexpr (FMT == FMT_INT4) {
                        // as in gw13: raw offset codes and the offset 8 on the MFMA,
                        // the difference times the output rows' scales of the chunk
                        f32x4 tcor[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                        for (int s = 0; s < 4; ++s)
#pragma unroll
                            for (int nt = 0; nt < 2; ++nt) {  // both tiles: no branch before the reads below
                                tcor[nt] = mfma16x16x32(__builtin_bit_cast(bf16x8, bh[nt][s]), bf16x8_splat8(), tcor[nt]);
                                tcor[nt] = mfma16x16x32(__builtin_bit_cast(bf16x8, bl[nt][s]), bf16x8_splat8(), tcor[nt]);
                            }
#pragma unroll
                        for (int rt = 0; rt < 4; ++rt) {
                            const uint32_t o = (uint32_t)(u0 + 16 * rt + r);  // the lane's row
                            const float so = f16_bits_to_f32(ld16(sb, o < (uint32_t)H ? o * ss + (uint32_t)c * 2u : OOB));
                            const uint32_t cws[4] = {cw[rt].x, cw[rt].y, cw[rt].z, cw[rt].w};
                            f32x4 t[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                            for (int s = 0; s < 4; ++s) {
                                const bf16x8 u = u4x8_bf16(cws[s]);
#pragma unroll
                                for (int nt = 0; nt < 2; ++nt) {
                                    t[nt] = mfma16x16x32(__builtin_bit_cast(bf16x8, bh[nt][s]), u, t[nt]);
                                    t[nt] = mfma16x16x32(__builtin_bit_cast(bf16x8, bl[nt][s]), u, t[nt]);
                                }
                            }
#pragma unroll
                            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                                for (int j = 0; j < 4; ++j)
                                    acc[rt][nt][j] = fmaf(so, t[nt][j] - tcor[nt][j], acc[rt][nt][j]);
                        }
                        continue;
                    }
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) {
                        const uint32_t cws[4] = {cw[rt].x, cw[rt].y, cw[rt].z, cw[rt].w};
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            if constexpr (FMT == FMT_NVFP4) {
                                const f32x2 sv = block_scales2<FMT>(sc[rt]);
                                const bf16x8 a1 = e2m1x8_scaled(cws[s], s < 2 ? sv.x : sv.y);
#pragma unroll
                                for (int nt = 0; nt < 2; ++nt) {
                                    if (nt == 1 && !two) break;
                                    acc[rt][nt] = mfma16x16x32(a1, __builtin_bit_cast(bf16x8, bh[nt][s]), acc[rt][nt]);
                                    acc[rt][nt] = mfma16x16x32(a1, __builtin_bit_cast(bf16x8, bl[nt][s]), acc[rt][nt]);
                                }
                            } else {
                                float sh, sl;
                                split_scale(f16_bits_to_f32(s < 2 ? sc[rt] : (sc[rt] >> 16)), sh, sl);
                                bf16x8 ah, al;
                                e2m1x8_split(cws[s], sh, sl, ah, al);
#pragma unroll
                                for (int nt = 0; nt < 2; ++nt) {
                                    if (nt == 1 && !two) break;
                                    const bf16x8 b0 = __builtin_bit_cast(bf16x8, bh[nt][s]);
                                    const bf16x8 b1 = __builtin_bit_cast(bf16x8, bl[nt][s]);
                                    // all four terms: al can reach 2^-5 of the weight and
                                    // h_lo 2^-8 of h, so al * h_lo is not negligible after
                                    // cancellation in the sum over K
                                    acc[rt][nt] = mfma16x16x32(ah, b0, acc[rt][nt]);
                                    acc[rt][nt] = mfma16x16x32(ah, b1, acc[rt][nt]);
                                    acc[rt][nt] = mfma16x16x32(al, b0, acc[rt][nt]);
                                    acc[rt][nt] = mfma16x16x32(al, b1, acc[rt][nt]);
                                }
                            }
                        }
                    }
                }
                // partials of all waves -> LDS; wave w sums row tile w in wave order
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                        for (int j = 0; j < 4; ++j) red[wv][rt][nt * 4 + j][lane] = acc[rt][nt][j];
                __syncthreads();
                float v[2][4];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float t = red[0][wv][nt * 4 + j][lane];
#pragma unroll
                        for (int w = 1; w < 4; ++w) t += red[w][wv][nt * 4 + j][lane];
                        v[nt][j] = t * gsc;
                    }
                __syncthreads();  // red is reused by the next pass or unit
                if constexpr (TR) {
                    // lane holds columns 4q + j of each tile for row u0 + 16wv + r; the
                    // pair of column c was read by lane c
                    const int row = u0 + 16 * wv + r;
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int p = __shfl(pr[nt], 4 * q + j, 64);
                            if (row < H && n0 + nt * 16 + 4 * q + j < gv.m) a.out[(size_t)p * H + row] = v[nt][j];
                        }
                    continue;
                }
                // lane holds rows u0 + 16wv + 4q + j of column r
                const int rb = u0 + 16 * wv + 4 * q;
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    if (!pv[nt]) continue;
                    float *op = a.out + (size_t)pr[nt] * H + rb;
                    if (rb + 3 < H) {
                        *reinterpret_cast<float4 *>(op) = make_float4(v[nt][0], v[nt][1], v[nt][2], v[nt][3]);
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (rb + j < H) op[j] = v[nt][j];
                    }
                }
            }
        };
        if constexpr (SB) {
            if (sbf) {
                mfma(std::true_type());
                return;
            }
        }
        mfma(std::false_type());
        return;
    }

    // ---- VALU (small groups): 16 rows per wave in load groups of 64/L rows;
    // codes loaded once, then each token: bf16 weights . (h_hi + h_lo)
    const int row0 = tile * 64 + 16 * wv;  // this wave's 16 output rows
    constexpr int NLG = RG >= 16 ? 1 : 16 / RG;
    const int lk = lane % L, rsub = lane / L;
    const int ks = (I + 32 * L - 1) / (32 * L);  // at most KS_VALU (checked by the host)
    uint4 cw[KS_VALU][NLG];
    uint32_t sc[KS_VALU][NLG];
#pragma unroll
    for (int s = 0; s < KS_VALU; ++s)
#pragma unroll
        for (int l = 0; l < NLG; ++l) {
            const int k0 = 32 * (L * s + lk);
            const int rr = row0 + l * RG + rsub;
            const bool v = s < ks && k0 < I && rr < H && (l * RG + rsub) < 16;
            cw[s][l] = ld128(cb, v ? (uint32_t)rr * cs + (uint32_t)(k0 >> 1) : OOB);
            sc[s][l] = ld_scales<FMT>(sb, v ? (uint32_t)rr * ss + scale_col<FMT>(k0) : OOB);
        }
    for (int idx = 0; idx < gv.m; ++idx) {
        if constexpr (FMT == FMT_INT4) {  // as in gw13_unit: the decode stays in the token loop
#pragma unroll
            for (int s = 0; s < KS_VALU; ++s)
#pragma unroll
                for (int l = 0; l < NLG; ++l)
                    asm volatile("" : "+v"(cw[s][l].x), "+v"(cw[s][l].y), "+v"(cw[s][l].z), "+v"(cw[s][l].w));
        }
        const int p = ld_uniform(plist, idx);
        float acc[NLG];
#pragma unroll
        for (int l = 0; l < NLG; ++l) acc[l] = 0.f;
#pragma unroll
        for (int s = 0; s < KS_VALU; ++s) {
            if (s >= ks) break;
            const int k0 = 32 * (L * s + lk);
            const uint32_t ho = (uint32_t)(p * I + k0) * 2u;
            XSlice<FMT> xh, xl;
            load_xslice<FMT>(xh, hhi, k0 < I ? ho : OOB);
            load_xslice<FMT>(xl, hlo, k0 < I ? ho : OOB);
            prep_xslice<FMT>(xh);
            prep_xslice<FMT>(xl);
#pragma unroll
            for (int l = 0; l < NLG; ++l) {
                acc[l] = chunk_dot_bf16<FMT>(cw[s][l], sc[s][l], xh, acc[l]);
                acc[l] = chunk_dot_bf16<FMT>(cw[s][l], sc[s][l], xl, acc[l]);
            }
        }
#pragma unroll
        for (int l = 0; l < NLG; ++l) {
            const float v = group_sum<L>(acc[l]) * gsc;
            const int rr = row0 + l * RG + rsub;
            if (group_leader<L>(lane) && rr < H && (l * RG + rsub) < 16) a.out[(size_t)p * H + rr] = v;
        }
    }
}

template <int FMT, int L, bool SB>
__global__ __launch_bounds__(256, L <= 16 && FMT != FMT_INT4 ? (SB ? 2 : W4_GW_MINBLK) : 1) void k_moe_gw2(GW2Args a) {
    __shared__ float red[4][4][8][64];  // MFMA partials: [wave][row tile][column tile x 4 + j][lane]
    const int nu = unit_count(a.grp, a.s_codes != nullptr, a.tiles);
    for (int u = blockIdx.x; u < nu; u += gridDim.x) {
        const int gs = u / a.tiles;
        gw2_unit<FMT, L, SB>(a, gs, u - gs * a.tiles, red);
    }
}

// ================================================================= prefill (large groups)

// Large batches (groups of tens to hundreds of rows): a block owns 128 weight
// rows of one group (two 16-row tiles per wave) for the whole K and one 64-column
// tile of the group.  The column tile's activations are staged in LDS one
// 128-wide K chunk at a time (double buffered, one barrier per chunk) and shared
// by the 4 waves; each wave keeps its rows' codes in registers (the next chunk's
// are loaded while the current one is multiplied) and owns its outputs
// outright, so no partial sums cross waves.  Operands as in gw13/gw2: every
// dequantised weight is two exact bf16 terms; h is read as its two bf16 terms.
constexpr int PF_COLS = 64;     // columns (pairs) per tile
constexpr int PF_KC = 128;      // K per chunk
constexpr int PF_LROW = PF_KC;  // bf16 per LDS row (256 B); 16-byte units are XOR-swizzled by column
constexpr int PF_ROWS = 128;    // weight rows (W13: h rows) per unit

// LDS address of 16-byte unit j (K elements 8j .. 8j+7) of column c: unit j is
// stored at position j ^ (c % 16), so that the 16 columns an MFMA operand read
// touches (and the 16 lanes of a store) cover all 64 banks once.
__device__ __forceinline__ const bf16x8 *pf_unit_ptr(const uint16_t (*rows)[PF_LROW], int c, int j) {
    return reinterpret_cast<const bf16x8 *>(&rows[c][8 * (j ^ (c & 15))]);
}

// The loader role of thread tid: column tid / 4 of the tile, K elements
// 32 (tid % 4) .. +31 of the chunk (four 16-byte loads).
__device__ __forceinline__ void pf_load(const Buf &b, uint32_t off, bool on, uint4 (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ld128(b, on ? off + 16u * i : OOB);
}
__device__ __forceinline__ void pf_store(uint16_t *row, int c, int lq, const uint4 (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4 *>(row + 8 * ((4 * lq + i) ^ (c & 15))) = v[i];
}

// Work units of the large-batch kernels: (column tile, row tile).  Unit u runs on
// XCD u % 8 (blocks are dealt to the XCDs round-robin and the grid is a multiple
// of 8).  XCD x takes the contiguous column tiles [x nct / 8, (x + 1) nct / 8)
// and walks all row tiles of each: a tile's activations are fetched into one L2
// and reused there, and since a group's tiles are consecutive, the tiles of one
// expert (which read the same weight rows) mostly share an L2 as well.  The
// shared expert's ceil(T/64) tiles follow the routed groups' (group table entry
// 1 + 3 Gmax and the column-tile map).
__device__ __forceinline__ int pf_tile_count(const int32_t *grp, int Gmax, bool shared, int T) {
    return ld_uniform(grp, 1 + 3 * Gmax) + (shared ? (T + PF_COLS - 1) / PF_COLS : 0);
}
__device__ __forceinline__ int pf_unit_count(int nct, int tiles) { return (nct + 7) / 8 * 8 * tiles; }
// false for the padding units of the last round of column tiles
__device__ __forceinline__ bool pf_unit(const int32_t *grp, const int32_t *ctg, int Gmax, bool shared, int nct, int u,
                                        int tiles, int &gs, int &rt, int &n0) {
    const int x = u & 7, j = u >> 3;
    const int ct = ((x * nct) >> 3) + j / tiles;
    rt = j - (j / tiles) * tiles;
    if (ct >= (((x + 1) * nct) >> 3)) return false;
    const int nrc = ld_uniform(grp, 1 + 3 * Gmax);
    if (ct < nrc) {
        gs = ld_uniform(ctg, 2 * ct) + (shared ? 1 : 0);
        n0 = ld_uniform(ctg, 2 * ct + 1);
    } else {
        gs = 0;
        n0 = (ct - nrc) * PF_COLS;
    }
    return true;
}

// FMT, SB as in gw13_unit: E2M1 weights as two exact bf16 terms, NVFP4 as one
// (the global scale multiplies the sums), a bf16 shared expert's rows as they are.
template <int FMT, bool SB>
__device__ __forceinline__ void pf13_unit(const GW13Args &a, int gs, int rt, int n0,
                                          uint16_t (*xs)[PF_COLS][PF_LROW]) {
    using SC = typename std::conditional<FMT == FMT_NVFP4, uint8_t, uint16_t>::type;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H, I = a.I;
    const GroupView<SC> gv = group_view<SC>(a.grp, gs, a.Gmax, a.P, a.T, 2 * I, a.codes, a.scales, a.rl, a.s_codes,
                                            a.s_scales, a.s_rl);
    const uint32_t cs = gv.cs, ss = gv.ss;  // row strides (bytes)
    const bool sbf = SB && gv.e < 0;
    const Buf cb = make_buf(gv.codes, (uint32_t)gv.mat_codes);
    const Buf sb = make_buf(gv.scales, sbf ? 0u : (uint32_t)gv.mat_scales);
    float gsc = 1.f;  // NVFP4 global scale of the matrix
    if constexpr (FMT == FMT_NVFP4) gsc = sbf ? 1.f : gv.e < 0 ? ld_uniform(a.s_gs, 0) : ld_uniform(a.gs, gv.e);
    const Buf xall = make_buf(a.x, (uint32_t)a.T * (uint32_t)H * 2u);
    const int *plist = a.pairs + gv.off;
    const int r = lane & 15, q = lane >> 4;
    const int i0 = rt * PF_ROWS + 32 * wv;  // the wave's first gate row: tiles i0 and i0 + 16
    // code rows: gate tile 0, gate tile 1, up tile 0, up tile 1
    const uint32_t rows[4] = {(uint32_t)(i0 + r), (uint32_t)(i0 + 16 + r), (uint32_t)(I + i0 + r),
                              (uint32_t)(I + i0 + 16 + r)};
    const int lc = tid >> 2, lq = tid & 3;
    const int nch = H / PF_KC;
    const bool lv = n0 + lc < gv.m;
    const uint32_t xo = lv ? (uint32_t)(token_of(plist[n0 + lc], a.P, a.K) * H + 32 * lq) * 2u : 0u;
    uint4 xr[4];
    pf_load(xall, xo, lv, xr);
    uint4 cw[4];
    uint32_t sw[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        cw[t] = ld128(cb, sbf ? OOB : rows[t] * cs + (uint32_t)(16 * q));
        sw[t] = ld_scales<FMT>(sb, sbf ? OOB : rows[t] * ss + scale_col<FMT>(32 * q));
    }
    f32x4 acc[4][4];  // [gate 0, gate 1, up 0, up 1][column tile]
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int ch = 0; ch < nch; ++ch) {
        uint16_t(*xb)[PF_LROW] = xs[ch & 1];
        pf_store(xb[lc], lc, lq, xr);
        __syncthreads();
        uint4 cc[4];
        uint32_t sc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) cc[t] = cw[t], sc[t] = sw[t];
        if (ch + 1 < nch) {  // next chunk: activations to registers, this wave's codes
            const uint32_t kn = (uint32_t)((ch + 1) * PF_KC);
            pf_load(xall, xo + kn * 2u, lv, xr);
            const uint32_t kq = kn + 32u * (uint32_t)q;
            if (!sbf) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    cw[t] = ld128(cb, rows[t] * cs + (kq >> 1));
                    sw[t] = ld_scales<FMT>(sb, rows[t] * ss + scale_col<FMT>((int)kq));
                }
            }
        }
        if constexpr (SB) {
            if (sbf) {  // bf16 rows: 8 weights of each row per MFMA step, read as needed
                const uint32_t kq = (uint32_t)(ch * PF_KC + 32 * q);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    bf16x8 b[4];
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) b[nt] = *pf_unit_ptr(xb, 16 * nt + r, 4 * q + s);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const bf16x8 w = __builtin_bit_cast(
                            bf16x8, ld128(cb, rows[t] * cs + (kq + 8u * (uint32_t)s) * 2u));
#pragma unroll
                        for (int nt = 0; nt < 4; ++nt) acc[t][nt] = mfma16x16x32(w, b[nt], acc[t][nt]);
                    }
                }
                continue;
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 b[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) b[nt] = *pf_unit_ptr(xb, 16 * nt + r, 4 * q + s);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t cws[4] = {cc[t].x, cc[t].y, cc[t].z, cc[t].w};
                if constexpr (FMT == FMT_NVFP4) {
                    const f32x2 sv = block_scales2<FMT>(sc[t]);
                    const bf16x8 a1 = e2m1x8_scaled(cws[s], s < 2 ? sv.x : sv.y);
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) acc[t][nt] = mfma16x16x32(a1, b[nt], acc[t][nt]);
                } else {
                    float hi, lo;
                    split_scale(f16_bits_to_f32(s < 2 ? sc[t] : (sc[t] >> 16)), hi, lo);
                    bf16x8 ah, al;
                    e2m1x8_split(cws[s], hi, lo, ah, al);
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) acc[t][nt] = mfma16x16x32(ah, b[nt], acc[t][nt]);
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) acc[t][nt] = mfma16x16x32(al, b[nt], acc[t][nt]);
                }
            }
        }
    }
    // lane holds rows 4q + j of each 16-row tile, column 16 nt + r
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int idx = n0 + 16 * nt + r;
        if (idx < gv.m) {
            const int p = plist[idx];
#pragma unroll
            for (int ht = 0; ht < 2; ++ht) {
                uint16_t bh[4], bl[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float gg = acc[ht][nt][j] * gsc, uu = acc[2 + ht][nt][j] * gsc;
                    split_bf16((gg / (1.f + expf(-gg))) * uu, bh[j], bl[j]);
                }
                const size_t o = (size_t)p * I + i0 + 16 * ht + 4 * q;
                *reinterpret_cast<uint2 *>(a.h_hi + o) =
                    make_uint2(bh[0] | ((uint32_t)bh[1] << 16), bh[2] | ((uint32_t)bh[3] << 16));
                *reinterpret_cast<uint2 *>(a.h_lo + o) =
                    make_uint2(bl[0] | ((uint32_t)bl[1] << 16), bl[2] | ((uint32_t)bl[3] << 16));
            }
        }
    }
    __syncthreads();  // the LDS buffers are refilled by the next unit
}

template <int FMT, bool SB>
__global__ __launch_bounds__(256) void k_moe_pf13(GW13Args a) {
    __shared__ __align__(16) uint16_t xs[2][PF_COLS][PF_LROW];
    const bool sh = a.s_codes != nullptr;
    const int nct = pf_tile_count(a.grp, a.Gmax, sh, a.T);
    const int nu = pf_unit_count(nct, a.tiles);
    for (int u = blockIdx.x; u < nu; u += gridDim.x) {
        int gs, rt, n0;
        if (pf_unit(a.grp, a.ctg, a.Gmax, sh, nct, u, a.tiles, gs, rt, n0)) pf13_unit<FMT, SB>(a, gs, rt, n0, xs);
    }
}

// FMT, SB as in pf13_unit.
template <int FMT, bool SB>
__device__ __forceinline__ void pf2_unit(const GW2Args &a, int gs, int rt, int n0,
                                         uint16_t (*hs)[2][PF_COLS][PF_LROW]) {
    using SC = typename std::conditional<FMT == FMT_NVFP4, uint8_t, uint16_t>::type;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H, I = a.I;
    const GroupView<SC> gv = group_view<SC>(a.grp, gs, a.Gmax, a.P, a.T, H, a.codes, a.scales, a.rl, a.s_codes,
                                            a.s_scales, a.s_rl);
    const uint32_t cs = gv.cs, ss = gv.ss;  // row strides (bytes)
    const bool sbf = SB && gv.e < 0;
    const Buf cb = make_buf(gv.codes, (uint32_t)gv.mat_codes);
    const Buf sb = make_buf(gv.scales, sbf ? 0u : (uint32_t)gv.mat_scales);
    float gsc = 1.f;  // NVFP4 global scale of the matrix
    if constexpr (FMT == FMT_NVFP4) gsc = sbf ? 1.f : gv.e < 0 ? ld_uniform(a.s_gs, 0) : ld_uniform(a.gs, gv.e);
    const uint32_t hbytes = (uint32_t)(a.P + a.T) * (uint32_t)I * 2u;
    const Buf hhi = make_buf(a.h_hi, hbytes), hlo = make_buf(a.h_lo, hbytes);
    const int *plist = a.pairs + gv.off;
    const int r = lane & 15, q = lane >> 4;
    const int o0 = rt * PF_ROWS + 32 * wv;  // the wave's first output row: tiles o0 and o0 + 16
    const uint32_t rows[2] = {(uint32_t)(o0 + r), (uint32_t)(o0 + 16 + r)};
    const int lc = tid >> 2, lq = tid & 3;
    const int nch = I / PF_KC;
    const bool lv = n0 + lc < gv.m;
    const uint32_t ho = lv ? (uint32_t)(plist[n0 + lc] * I + 32 * lq) * 2u : 0u;
    uint4 hr[4], lr[4];
    pf_load(hhi, ho, lv, hr);
    pf_load(hlo, ho, lv, lr);
    uint4 cw[2];
    uint32_t sw[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        cw[t] = ld128(cb, sbf ? OOB : rows[t] * cs + (uint32_t)(16 * q));
        sw[t] = ld_scales<FMT>(sb, sbf ? OOB : rows[t] * ss + scale_col<FMT>(32 * q));
    }
    f32x4 acc[2][4], acc2[2][4];  // [row tile][column tile]; weight hi / lo terms
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[t][nt] = acc2[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int ch = 0; ch < nch; ++ch) {
        uint16_t(*bh)[PF_LROW] = hs[ch & 1][0];
        uint16_t(*bl)[PF_LROW] = hs[ch & 1][1];
        pf_store(bh[lc], lc, lq, hr);
        pf_store(bl[lc], lc, lq, lr);
        __syncthreads();
        uint4 cc[2];
        uint32_t sc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) cc[t] = cw[t], sc[t] = sw[t];
        if (ch + 1 < nch) {
            const uint32_t kn = (uint32_t)((ch + 1) * PF_KC);
            pf_load(hhi, ho + kn * 2u, lv, hr);
            pf_load(hlo, ho + kn * 2u, lv, lr);
            const uint32_t kq = kn + 32u * (uint32_t)q;
            if (!sbf) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    cw[t] = ld128(cb, rows[t] * cs + (kq >> 1));
                    sw[t] = ld_scales<FMT>(sb, rows[t] * ss + scale_col<FMT>((int)kq));
                }
            }
        }
        if constexpr (SB) {
            if (sbf) {  // bf16 rows, read as needed; h as hi + lo
                const uint32_t kq = (uint32_t)(ch * PF_KC + 32 * q);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    bf16x8 b0[4], b1[4];
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        b0[nt] = *pf_unit_ptr(bh, 16 * nt + r, 4 * q + s);
                        b1[nt] = *pf_unit_ptr(bl, 16 * nt + r, 4 * q + s);
                    }
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const bf16x8 w = __builtin_bit_cast(
                            bf16x8, ld128(cb, rows[t] * cs + (kq + 8u * (uint32_t)s) * 2u));
#pragma unroll
                        for (int nt = 0; nt < 4; ++nt) {
                            acc[t][nt] = mfma16x16x32(w, b0[nt], acc[t][nt]);
                            acc2[t][nt] = mfma16x16x32(w, b1[nt], acc2[t][nt]);
                        }
                    }
                }
                continue;
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 b0[4], b1[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                b0[nt] = *pf_unit_ptr(bh, 16 * nt + r, 4 * q + s);
                b1[nt] = *pf_unit_ptr(bl, 16 * nt + r, 4 * q + s);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint32_t cws[4] = {cc[t].x, cc[t].y, cc[t].z, cc[t].w};
                if constexpr (FMT == FMT_NVFP4) {  // one exact weight term
                    const f32x2 sv = block_scales2<FMT>(sc[t]);
                    const bf16x8 a1 = e2m1x8_scaled(cws[s], s < 2 ? sv.x : sv.y);
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        acc[t][nt] = mfma16x16x32(a1, b0[nt], acc[t][nt]);
                        acc2[t][nt] = mfma16x16x32(a1, b1[nt], acc2[t][nt]);
                    }
                    continue;
                }
                float hi, lo;
                split_scale(f16_bits_to_f32(s < 2 ? sc[t] : (sc[t] >> 16)), hi, lo);
                bf16x8 ah, al;
                e2m1x8_split(cws[s], hi, lo, ah, al);
                // all four terms (al can reach 2^-5 of the weight, h_lo 2^-8 of h)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    acc[t][nt] = mfma16x16x32(ah, b0[nt], acc[t][nt]);
                    acc2[t][nt] = mfma16x16x32(al, b0[nt], acc2[t][nt]);
                }
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    acc[t][nt] = mfma16x16x32(ah, b1[nt], acc[t][nt]);
                    acc2[t][nt] = mfma16x16x32(al, b1[nt], acc2[t][nt]);
                }
            }
        }
    }
    // lane holds rows 4q + j of each 16-row tile, column 16 nt + r
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int idx = n0 + 16 * nt + r;
        if (idx < gv.m) {
            float *op = a.out + (size_t)plist[idx] * H + o0 + 4 * q;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const f32x4 v = (acc[t][nt] + acc2[t][nt]) * gsc;
                *reinterpret_cast<float4 *>(op + 16 * t) = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
    __syncthreads();
}

template <int FMT, bool SB>
__global__ __launch_bounds__(256) void k_moe_pf2(GW2Args a) {
    __shared__ __align__(16) uint16_t hs[2][2][PF_COLS][PF_LROW];  // [buffer][hi, lo][column][K]
    const bool sh = a.s_codes != nullptr;
    const int nct = pf_tile_count(a.grp, a.Gmax, sh, a.T);
    const int nu = pf_unit_count(nct, a.tiles);
    for (int u = blockIdx.x; u < nu; u += gridDim.x) {
        int gs, rt, n0;
        if (pf_unit(a.grp, a.ctg, a.Gmax, sh, nct, u, a.tiles, gs, rt, n0)) pf2_unit<FMT, SB>(a, gs, rt, n0, hs);
    }
}

// ================================================================= MX path

// The MX path (MXFP4 weights, MXFP8 activations) runs every group on gfx950's
// scaled FP4 MFMA (16 x 16 x 128 per instruction, E8M0 scale per 32 K on both
// operands), so its units need no exact split of the scales.  Quantisation of
// activations follows the OCP Microscaling conversion (mx8_exponent, mx8_pack4).

// x bf16 [rows][n] -> MXFP8: one thread per 32-element block.
__global__ __launch_bounds__(256) void k_mx_quant(MXQuantArgs a) {
    const int nb = a.n >> 5;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= a.rows * nb) return;
    const int r = i / nb, b = i - r * nb;
    const uint4 *src = reinterpret_cast<const uint4 *>(a.x + (size_t)r * a.n + 32 * b);
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 u = src[q];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            v[8 * q + 2 * d] = __uint_as_float(w[d] << 16);
            v[8 * q + 2 * d + 1] = __uint_as_float(w[d] & 0xFFFF0000u);
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[e]));
    const int X = mx8_exponent(amax);
    uint32_t o[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] = mx8_pack4(v[4 * d], v[4 * d + 1], v[4 * d + 2], v[4 * d + 3], X);
    uint4 *dst = reinterpret_cast<uint4 *>(a.q + (size_t)r * a.n + 32 * b);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    a.s[i] = (uint8_t)(X + 127);
}

// One unit of the MX W13 launch: group slot gs, gate rows 32 tile .. +32 and the
// matching up rows (four 16-row MFMA tiles), so that each 32-element block of h
// is complete here and is quantised in the epilogue.
__device__ __forceinline__ void mx13_unit(const MX13Args &a, int gs, int tile, float (*red)[32][64]) {
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int H = a.H, I = a.I;
    const GroupView<uint8_t> gv = group_view<uint8_t>(a.grp, gs, a.Gmax, a.P, a.T, 2 * I, a.codes, a.scales, a.rl,
                                                      a.s_codes, a.s_scales, a.s_rl);
    const uint32_t cs = gv.cs, ss = gv.ss;  // row strides (bytes)
    const Buf cb = make_buf(gv.codes, (uint32_t)gv.mat_codes);
    const Buf sb = make_buf(gv.scales, (uint32_t)gv.mat_scales);
    const Buf xqb = make_buf(a.xq, (uint32_t)a.T * (uint32_t)H);
    const Buf xsb = make_buf(a.xs, (uint32_t)a.T * (uint32_t)(H >> 5));
    const int *plist = a.pairs + gv.off;
    const int i0 = tile * 32;
    const int r = lane & 15, g = lane >> 4;
    const uint32_t rows[4] = {(uint32_t)(i0 + r), (uint32_t)(i0 + 16 + r), (uint32_t)(I + i0 + r),
                              (uint32_t)(I + i0 + 16 + r)};
    const int nchunks = H >> 7;
    for (int n0 = 0; n0 < gv.m; n0 += 32) {
        int pr[2], tk[2];
        bool pv[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int idx = n0 + nt * 16 + r;
            pv[nt] = idx < gv.m;
            pr[nt] = pv[nt] ? plist[idx] : 0;
            tk[nt] = token_of(pr[nt], a.P, a.K);
        }
        const bool two = n0 + 16 < gv.m;  // second column tile in use (uniform)
        f32x4 acc[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t][0] = acc[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int c = wv; c < nchunks; c += 4) {
            const int k0 = c * 128;
            uint4 av[4];
            uint32_t as[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                av[t] = ld128(cb, rows[t] * cs + (uint32_t)((k0 + 32 * g) >> 1));
                as[t] = ld8(sb, rows[t] * ss + (uint32_t)(k0 >> 5) + (uint32_t)g);
            }
            uint4 blo[2], bhi[2];
            uint32_t bs[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const bool on = (nt == 0 || two) && pv[nt];
                const uint32_t xo = (uint32_t)(tk[nt] * H + k0 + 16 * g);
                blo[nt] = ld128(xqb, on ? xo : OOB);
                bhi[nt] = ld128(xqb, on ? xo + 64u : OOB);
                bs[nt] = ld8(xsb, on ? (uint32_t)(tk[nt] * (H >> 5) + (k0 >> 5) + g) : OOB);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    if (nt == 1 && !two) break;
                    acc[t][nt] = mfma_mx(av[t], blo[nt], bhi[nt], as[t], bs[nt], acc[t][nt]);
                }
        }
        // fixed-order sum of the four K partials
        if (wv > 0) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) red[wv - 1][t * 8 + nt * 4 + j][lane] = acc[t][nt][j];
        }
        __syncthreads();
        if (wv == 0) {
#pragma unroll
            for (int w = 0; w < 3; ++w)
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[t][nt][j] += red[w][t * 8 + nt * 4 + j][lane];
            // lane holds rows 4g + j of both 16-row halves of column r: h of rows
            // i0 + 4g + j (tile 0) and i0 + 16 + 4g + j (tile 1)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                float h[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float g0 = acc[0][nt][j], u0 = acc[2][nt][j];
                    const float g1 = acc[1][nt][j], u1 = acc[3][nt][j];
                    h[j] = (g0 / (1.f + expf(-g0))) * u0;
                    h[4 + j] = (g1 / (1.f + expf(-g1))) * u1;
                }
                float m = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(h[e]));
                m = fmaxf(m, __shfl_xor(m, 16));  // the 32 rows of column r sit in lanes r, r+16, r+32, r+48
                m = fmaxf(m, __shfl_xor(m, 32));
                const int X = mx8_exponent(m);
                if (pv[nt]) {
                    const size_t o = (size_t)pr[nt] * I + i0 + 4 * g;
                    *reinterpret_cast<uint32_t *>(a.hq + o) = mx8_pack4(h[0], h[1], h[2], h[3], X);
                    *reinterpret_cast<uint32_t *>(a.hq + o + 16) = mx8_pack4(h[4], h[5], h[6], h[7], X);
                    if (g == 0) a.hs[(size_t)pr[nt] * (I >> 5) + (i0 >> 5)] = (uint8_t)(X + 127);
                }
            }
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void k_moe_mx13(MX13Args a) {
    __shared__ float red[3][32][64];  // K partials of waves 1..3
    const int nu = unit_count(a.grp, a.s_codes != nullptr, a.tiles);
    for (int u = blockIdx.x; u < nu; u += gridDim.x) {
        const int gs = u / a.tiles;
        mx13_unit(a, gs, u - gs * a.tiles, red);
    }
}

// One unit of the MX down launch: group slot gs, output rows 64 tile .. +64; the
// waves split K (128-element chunks), each multiplies its chunk into all four
// 16-row tiles, partials summed in wave order through LDS.
__device__ __forceinline__ void mx2_unit(const MX2Args &a, int gs, int tile, float (*red)[4][8][64]) {
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int H = a.H, I = a.I;
    const GroupView<uint8_t> gv = group_view<uint8_t>(a.grp, gs, a.Gmax, a.P, a.T, H, a.codes, a.scales, a.rl,
                                                      a.s_codes, a.s_scales, a.s_rl);
    const uint32_t cs = gv.cs, ss = gv.ss;  // row strides (bytes)
    const Buf cb = make_buf(gv.codes, (uint32_t)gv.mat_codes);
    const Buf sb = make_buf(gv.scales, (uint32_t)gv.mat_scales);
    const uint32_t rowsall = (uint32_t)(a.P + a.T);
    const Buf hqb = make_buf(a.hq, rowsall * (uint32_t)I);
    const Buf hsb = make_buf(a.hs, rowsall * (uint32_t)(I >> 5));
    const int *plist = a.pairs + gv.off;
    const int r = lane & 15, g = lane >> 4;
    const int u0 = tile * 64;
    const int nchunks = I >> 7;
    for (int n0 = 0; n0 < gv.m; n0 += 32) {
        int pr[2];
        bool pv[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int idx = n0 + nt * 16 + r;
            pv[nt] = idx < gv.m;
            pr[nt] = pv[nt] ? plist[idx] : 0;
        }
        const bool two = n0 + 16 < gv.m;
        f32x4 acc[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t][0] = acc[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int c = wv; c < nchunks; c += 4) {
            const int k0 = c * 128;
            uint4 av[4];
            uint32_t as[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t row = (uint32_t)(u0 + 16 * t + r);
                const bool rv = (int)row < H;
                av[t] = ld128(cb, rv ? row * cs + (uint32_t)((k0 + 32 * g) >> 1) : OOB);
                as[t] = ld8(sb, rv ? row * ss + (uint32_t)(k0 >> 5) + (uint32_t)g : OOB);
            }
            uint4 blo[2], bhi[2];
            uint32_t bs[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const bool on = (nt == 0 || two) && pv[nt];
                const uint32_t ho = (uint32_t)(pr[nt] * I + k0 + 16 * g);
                blo[nt] = ld128(hqb, on ? ho : OOB);
                bhi[nt] = ld128(hqb, on ? ho + 64u : OOB);
                bs[nt] = ld8(hsb, on ? (uint32_t)(pr[nt] * (I >> 5) + (k0 >> 5) + g) : OOB);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    if (nt == 1 && !two) break;
                    acc[t][nt] = mfma_mx(av[t], blo[nt], bhi[nt], as[t], bs[nt], acc[t][nt]);
                }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int j = 0; j < 4; ++j) red[wv][t][nt * 4 + j][lane] = acc[t][nt][j];
        __syncthreads();
        float v[2][4];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float sum = red[0][wv][nt * 4 + j][lane];
#pragma unroll
                for (int w = 1; w < 4; ++w) sum += red[w][wv][nt * 4 + j][lane];
                v[nt][j] = sum;
            }
        __syncthreads();
        const int rb = u0 + 16 * wv + 4 * g;  // lane holds rows rb .. rb+3 of column r
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            if (!pv[nt]) continue;
            float *op = a.out + (size_t)pr[nt] * H + rb;
            if (rb + 3 < H) {
                *reinterpret_cast<float4 *>(op) = make_float4(v[nt][0], v[nt][1], v[nt][2], v[nt][3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (rb + j < H) op[j] = v[nt][j];
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_moe_mx2(MX2Args a) {
    __shared__ float red[4][4][8][64];
    const int nu = unit_count(a.grp, a.s_codes != nullptr, a.tiles);
    for (int u = blockIdx.x; u < nu; u += gridDim.x) {
        const int gs = u / a.tiles;
        mx2_unit(a, gs, u - gs * a.tiles, red);
    }
}

// Large batches, MX: the structure of k_moe_pf13 / k_moe_pf2 with fp8
// activations (one byte per element, an E8M0 scale per 32) in the LDS tile and
// the scaled FP4 MFMA (16 x 16 x 128, both block scales fed to the instruction).
// A column's 128-byte chunk is 8 units of 16 bytes stored at j ^ ((c / 2) % 8),
// so the 16 columns one operand read touches cover all 64 banks once.
constexpr int PFX_LROW = PF_KC;  // bytes per LDS row
__device__ __forceinline__ uint4 pfx_unit(const uint8_t (*rows)[PFX_LROW], int c, int j) {
    return *reinterpret_cast<const uint4 *>(&rows[c][16 * (j ^ ((c >> 1) & 7))]);
}
// loader role of thread tid: column tid / 4, bytes 32 (tid % 4) .. +31 of the
// chunk and the column's E8M0 scale byte of block tid % 4
__device__ __forceinline__ void pfx_store(uint8_t *row, int c, int lq, const uint4 (&v)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4 *>(row + 16 * ((2 * lq + i) ^ ((c >> 1) & 7))) = v[i];
}

__device__ __forceinline__ void pfmx13_unit(const MX13Args &a, int gs, int rt, int n0, uint8_t (*xs)[PF_COLS][PFX_LROW],
                                            uint8_t (*xsc)[PF_COLS][4]) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H, I = a.I;
    const GroupView<uint8_t> gv = group_view<uint8_t>(a.grp, gs, a.Gmax, a.P, a.T, 2 * I, a.codes, a.scales, a.rl,
                                                      a.s_codes, a.s_scales, a.s_rl);
    const uint32_t cs = gv.cs, ss = gv.ss;  // row strides (bytes)
    const Buf cb = make_buf(gv.codes, (uint32_t)gv.mat_codes);
    const Buf sb = make_buf(gv.scales, (uint32_t)gv.mat_scales);
    const Buf xqb = make_buf(a.xq, (uint32_t)a.T * (uint32_t)H);
    const Buf xsb = make_buf(a.xs, (uint32_t)a.T * (uint32_t)(H >> 5));
    const int *plist = a.pairs + gv.off;
    const int r = lane & 15, g = lane >> 4;
    const int i0 = rt * PF_ROWS + 32 * wv;  // the wave's 32 h rows: tiles i0, i0 + 16
    const uint32_t rows[4] = {(uint32_t)(i0 + r), (uint32_t)(i0 + 16 + r), (uint32_t)(I + i0 + r),
                              (uint32_t)(I + i0 + 16 + r)};
    const int lc = tid >> 2, lq = tid & 3;
    const int nch = H / PF_KC;
    const bool lv = n0 + lc < gv.m;
    const int tok = lv ? token_of(plist[n0 + lc], a.P, a.K) : 0;
    const uint32_t xo = (uint32_t)(tok * H + 32 * lq), so = (uint32_t)(tok * (H >> 5) + lq);
    uint4 xr[2];
    uint32_t sr;
    xr[0] = ld128(xqb, lv ? xo : OOB);
    xr[1] = ld128(xqb, lv ? xo + 16u : OOB);
    sr = ld8(xsb, lv ? so : OOB);
    uint4 cw[4];
    uint32_t sw[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        cw[t] = ld128(cb, rows[t] * cs + (uint32_t)(16 * g));
        sw[t] = ld8(sb, rows[t] * ss + (uint32_t)g);
    }
    f32x4 acc[4][4];  // [gate 0, gate 1, up 0, up 1][column tile]
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int ch = 0; ch < nch; ++ch) {
        uint8_t(*xb)[PFX_LROW] = xs[ch & 1];
        uint8_t(*xc)[4] = xsc[ch & 1];
        pfx_store(xb[lc], lc, lq, xr);
        xc[lc][lq] = (uint8_t)sr;
        __syncthreads();
        uint4 cc[4];
        uint32_t sc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) cc[t] = cw[t], sc[t] = sw[t];
        if (ch + 1 < nch) {
            const uint32_t kn = (uint32_t)((ch + 1) * PF_KC);
            xr[0] = ld128(xqb, lv ? xo + kn : OOB);
            xr[1] = ld128(xqb, lv ? xo + kn + 16u : OOB);
            sr = ld8(xsb, lv ? so + (kn >> 5) : OOB);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                cw[t] = ld128(cb, rows[t] * cs + ((kn + 32u * (uint32_t)g) >> 1));
                sw[t] = ld8(sb, rows[t] * ss + (kn >> 5) + (uint32_t)g);
            }
        }
        uint4 blo[4], bhi[4];
        uint32_t bs[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            blo[nt] = pfx_unit(xb, 16 * nt + r, g);
            bhi[nt] = pfx_unit(xb, 16 * nt + r, 4 + g);
            bs[nt] = xc[16 * nt + r][g];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) acc[t][nt] = mfma_mx(cc[t], blo[nt], bhi[nt], sc[t], bs[nt], acc[t][nt]);
    }
    // lane holds rows 4g + j of each 16-row tile, column 16 nt + r; the 32 h rows
    // of the wave form one MX block per column, spread over lanes r, r+16, r+32, r+48
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        float h[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float g0 = acc[0][nt][j], u0 = acc[2][nt][j];
            const float g1 = acc[1][nt][j], u1 = acc[3][nt][j];
            h[j] = (g0 / (1.f + expf(-g0))) * u0;
            h[4 + j] = (g1 / (1.f + expf(-g1))) * u1;
        }
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(h[e]));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        const int X = mx8_exponent(m);
        const int idx = n0 + 16 * nt + r;
        if (idx < gv.m) {
            const int p = plist[idx];
            const size_t o = (size_t)p * I + i0 + 4 * g;
            *reinterpret_cast<uint32_t *>(a.hq + o) = mx8_pack4(h[0], h[1], h[2], h[3], X);
            *reinterpret_cast<uint32_t *>(a.hq + o + 16) = mx8_pack4(h[4], h[5], h[6], h[7], X);
            if (g == 0) a.hs[(size_t)p * (I >> 5) + (i0 >> 5)] = (uint8_t)(X + 127);
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void k_moe_pfmx13(MX13Args a) {
    __shared__ __align__(16) uint8_t xs[2][PF_COLS][PFX_LROW];
    __shared__ uint8_t xsc[2][PF_COLS][4];
    const bool sh = a.s_codes != nullptr;
    const int nct = pf_tile_count(a.grp, a.Gmax, sh, a.T);
    const int nu = pf_unit_count(nct, a.tiles);
    for (int u = blockIdx.x; u < nu; u += gridDim.x) {
        int gs, rt, n0;
        if (pf_unit(a.grp, a.ctg, a.Gmax, sh, nct, u, a.tiles, gs, rt, n0)) pfmx13_unit(a, gs, rt, n0, xs, xsc);
    }
}

__device__ __forceinline__ void pfmx2_unit(const MX2Args &a, int gs, int rt, int n0, uint8_t (*hsm)[PF_COLS][PFX_LROW],
                                           uint8_t (*hsc)[PF_COLS][4]) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H, I = a.I;
    const GroupView<uint8_t> gv = group_view<uint8_t>(a.grp, gs, a.Gmax, a.P, a.T, H, a.codes, a.scales, a.rl,
                                                      a.s_codes, a.s_scales, a.s_rl);
    const uint32_t cs = gv.cs, ss = gv.ss;  // row strides (bytes)
    const Buf cb = make_buf(gv.codes, (uint32_t)gv.mat_codes);
    const Buf sb = make_buf(gv.scales, (uint32_t)gv.mat_scales);
    const uint32_t rowsall = (uint32_t)(a.P + a.T);
    const Buf hqb = make_buf(a.hq, rowsall * (uint32_t)I);
    const Buf hsb = make_buf(a.hs, rowsall * (uint32_t)(I >> 5));
    const int *plist = a.pairs + gv.off;
    const int r = lane & 15, g = lane >> 4;
    const int o0 = rt * PF_ROWS + 32 * wv;  // the wave's output rows: tiles o0, o0 + 16
    const uint32_t rows[2] = {(uint32_t)(o0 + r), (uint32_t)(o0 + 16 + r)};
    const int lc = tid >> 2, lq = tid & 3;
    const int nch = I / PF_KC;
    const bool lv = n0 + lc < gv.m;
    const int pr = lv ? plist[n0 + lc] : 0;
    const uint32_t ho = (uint32_t)(pr * I + 32 * lq), so = (uint32_t)(pr * (I >> 5) + lq);
    uint4 hr[2];
    uint32_t sr;
    hr[0] = ld128(hqb, lv ? ho : OOB);
    hr[1] = ld128(hqb, lv ? ho + 16u : OOB);
    sr = ld8(hsb, lv ? so : OOB);
    uint4 cw[2];
    uint32_t sw[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        cw[t] = ld128(cb, rows[t] * cs + (uint32_t)(16 * g));
        sw[t] = ld8(sb, rows[t] * ss + (uint32_t)g);
    }
    f32x4 acc[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int ch = 0; ch < nch; ++ch) {
        uint8_t(*hb)[PFX_LROW] = hsm[ch & 1];
        uint8_t(*hc)[4] = hsc[ch & 1];
        pfx_store(hb[lc], lc, lq, hr);
        hc[lc][lq] = (uint8_t)sr;
        __syncthreads();
        uint4 cc[2];
        uint32_t sc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) cc[t] = cw[t], sc[t] = sw[t];
        if (ch + 1 < nch) {
            const uint32_t kn = (uint32_t)((ch + 1) * PF_KC);
            hr[0] = ld128(hqb, lv ? ho + kn : OOB);
            hr[1] = ld128(hqb, lv ? ho + kn + 16u : OOB);
            sr = ld8(hsb, lv ? so + (kn >> 5) : OOB);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                cw[t] = ld128(cb, rows[t] * cs + ((kn + 32u * (uint32_t)g) >> 1));
                sw[t] = ld8(sb, rows[t] * ss + (kn >> 5) + (uint32_t)g);
            }
        }
        uint4 blo[4], bhi[4];
        uint32_t bs[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            blo[nt] = pfx_unit(hb, 16 * nt + r, g);
            bhi[nt] = pfx_unit(hb, 16 * nt + r, 4 + g);
            bs[nt] = hc[16 * nt + r][g];
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) acc[t][nt] = mfma_mx(cc[t], blo[nt], bhi[nt], sc[t], bs[nt], acc[t][nt]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int idx = n0 + 16 * nt + r;
        if (idx < gv.m) {
            float *op = a.out + (size_t)plist[idx] * H + o0 + 4 * g;
#pragma unroll
            for (int t = 0; t < 2; ++t)
                *reinterpret_cast<float4 *>(op + 16 * t) = make_float4(acc[t][nt][0], acc[t][nt][1], acc[t][nt][2],
                                                                      acc[t][nt][3]);
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void k_moe_pfmx2(MX2Args a) {
    __shared__ __align__(16) uint8_t hsm[2][PF_COLS][PFX_LROW];
    __shared__ uint8_t hsc[2][PF_COLS][4];
    const bool sh = a.s_codes != nullptr;
    const int nct = pf_tile_count(a.grp, a.Gmax, sh, a.T);
    const int nu = pf_unit_count(nct, a.tiles);
    for (int u = blockIdx.x; u < nu; u += gridDim.x) {
        int gs, rt, n0;
        if (pf_unit(a.grp, a.ctg, a.Gmax, sh, nct, u, a.tiles, gs, rt, n0)) pfmx2_unit(a, gs, rt, n0, hsm, hsc);
    }
}

// ================================================================= combine

// Test hook of the scaled FP4 MFMA: out[i][j] = sum_k A[i][k] B[j][k] with A
// MXFP4 (E2M1 codes [n][k/2], E8M0 [n][k/32]) and B MXFP8 (E4M3 [m][k], E8M0
// [m][k/32]), one wave per 16 x 16 output tile, every 128-wide K chunk added
// into the same accumulator: the operand mapping (mfma_mx) and the per-wave
// accumulation chain of the MX expert kernels, on plain matrices.
__global__ __launch_bounds__(64) void k_mx_dot(const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as,
                                               const uint8_t *__restrict__ bc, const uint8_t *__restrict__ bs,
                                               float *__restrict__ out, int n, int m, int k, RowLayout arl) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int row0 = (int)blockIdx.y * 16, col0 = (int)blockIdx.x * 16;
    const Buf ab = make_buf(ac, (uint32_t)n * arl.cs);
    const Buf asb = make_buf(as, (uint32_t)n * arl.ss);
    const Buf bb = make_buf(bc, (uint32_t)m * (uint32_t)k);
    const Buf bsb = make_buf(bs, (uint32_t)m * (uint32_t)(k >> 5));
    const uint32_t row = (uint32_t)(row0 + r), col = (uint32_t)(col0 + r);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < k; k0 += 128) {
        const uint4 av = ld128(ab, row * arl.cs + (uint32_t)((k0 + 32 * g) >> 1));
        const uint32_t sa = ld8(asb, row * arl.ss + (uint32_t)(k0 >> 5) + (uint32_t)g);
        const uint32_t xo = col * (uint32_t)k + (uint32_t)(k0 + 16 * g);
        const uint4 blo = ld128(bb, xo), bhi = ld128(bb, xo + 64u);
        const uint32_t sb = ld8(bsb, col * (uint32_t)(k >> 5) + (uint32_t)(k0 >> 5) + (uint32_t)g);
        acc = mfma_mx(av, blo, bhi, sa, sb, acc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) out[(size_t)(row0 + 4 * g + j) * m + col] = acc[j];
}

__global__ __launch_bounds__(256) void k_moe_gcombine(GCombineArgs a) {
    // four consecutive outputs per thread (H is a multiple of 64); every element
    // is summed in slot order, then the shared expert, as one scalar would be
    const int t = blockIdx.y;
    const int n = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
    if (n >= a.H) return;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < a.K; ++j) {
        const int p = t * a.K + j;
        const int e = ld_uniform(a.ids, p);
        const float w = ld_uniform(a.w, p);
        if (e >= 0 && e < a.E) {
            const float4 o = *reinterpret_cast<const float4 *>(a.out + (size_t)p * a.H + n);
            v.x += w * o.x, v.y += w * o.y, v.z += w * o.z, v.w += w * o.w;
        } else {
            v = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
        }
    }
    if (a.has_shared) {
        const float sig = 1.f / (1.f + expf(-ld_uniform(a.logits, t * a.lstride + a.E)));
        const float4 o = *reinterpret_cast<const float4 *>(a.out + (size_t)(a.P + t) * a.H + n);
        v.x += sig * o.x, v.y += sig * o.y, v.z += sig * o.z, v.w += sig * o.w;
    }
    uint16_t *yp = a.y + (size_t)t * a.H + n;
    if ((reinterpret_cast<uintptr_t>(a.y) & 7) == 0) {  // y needs only 2-byte alignment
        const uint32_t lo = f32_to_bf16_rne(v.x) | ((uint32_t)f32_to_bf16_rne(v.y) << 16);
        const uint32_t hi = f32_to_bf16_rne(v.z) | ((uint32_t)f32_to_bf16_rne(v.w) << 16);
        *reinterpret_cast<uint2 *>(yp) = make_uint2(lo, hi);
    } else {
        yp[0] = f32_to_bf16_rne(v.x), yp[1] = f32_to_bf16_rne(v.y);
        yp[2] = f32_to_bf16_rne(v.z), yp[3] = f32_to_bf16_rne(v.w);
    }
}

}  // namespace w4k

// ================================================================= launchers

namespace w4k {

namespace {
int lanes_for_k(int k) {
    int need = (k + 31) / 32, L = 1;
    while (L < need && L < 64) L <<= 1;
    return L;
}

template <typename F, typename... Args>
void go_ev(hipStream_t st, hipEvent_t e0, hipEvent_t e1, F kernel, dim3 g, dim3 b, uint32_t shm, Args... args) {
    if (e0)
        hipExtLaunchKernelGGL(kernel, g, b, shm, st, e0, e1, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, g, b, shm, st, args...);
}
}  // namespace

size_t grouped_lds_bytes(int E, int P) { return (size_t)(2 * E + 2 * P) * sizeof(int); }

void launch_route_group(GroupArgs &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    const int pl = (a.E + 63) / 64;
    const dim3 g(1), b(1024);
    const uint32_t shm = (uint32_t)grouped_lds_bytes(a.E, a.P);
    if (pl <= 1) go_ev(st, e0, e1, k_moe_route_group<1>, g, b, shm, a);
    else if (pl <= 2) go_ev(st, e0, e1, k_moe_route_group<2>, g, b, shm, a);
    else if (pl <= 4) go_ev(st, e0, e1, k_moe_route_group<4>, g, b, shm, a);
    else if (pl <= 8) go_ev(st, e0, e1, k_moe_route_group<8>, g, b, shm, a);
    else go_ev(st, e0, e1, k_moe_route_group<16>, g, b, shm, a);
}

void launch_rank_group(GroupArgs &a, int32_t *arrive, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    const int pl = (a.E + 63) / 64;
    const dim3 g((unsigned)((a.T + RG_TOKENS - 1) / RG_TOKENS)), b(64 * RG_WAVES);
    const uint32_t shm = (uint32_t)grouped_lds_bytes(a.E, a.P);
    if (pl <= 1) go_ev(st, e0, e1, k_moe_rank_group<1>, g, b, shm, a, arrive);
    else if (pl <= 2) go_ev(st, e0, e1, k_moe_rank_group<2>, g, b, shm, a, arrive);
    else if (pl <= 4) go_ev(st, e0, e1, k_moe_rank_group<4>, g, b, shm, a, arrive);
    else if (pl <= 8) go_ev(st, e0, e1, k_moe_rank_group<8>, g, b, shm, a, arrive);
    else go_ev(st, e0, e1, k_moe_rank_group<16>, g, b, shm, a, arrive);
}

void launch_route_multi(RouteArgs &a, hipStream_t st, hipEvent_t *ev) {
    const int pl = (a.g.E + 63) / 64;
    const dim3 g((unsigned)a.nblk), b(256);
    hipEvent_t e[6] = {};
    if (ev)
        for (int i = 0; i < 6; ++i) e[i] = ev[i];
    if (pl <= 1) go_ev(st, e[0], e[1], k_route_topk<1>, g, b, 0, a);
    else if (pl <= 2) go_ev(st, e[0], e[1], k_route_topk<2>, g, b, 0, a);
    else if (pl <= 4) go_ev(st, e[0], e[1], k_route_topk<4>, g, b, 0, a);
    else if (pl <= 8) go_ev(st, e[0], e[1], k_route_topk<8>, g, b, 0, a);
    else go_ev(st, e[0], e[1], k_route_topk<16>, g, b, 0, a);
    go_ev(st, e[2], e[3], k_route_scan, dim3(1), dim3(1024), 0, a);
    go_ev(st, e[4], e[5], k_route_scatter, g, b, 0, a);
}

// blocks of the grid-stride W13 and down launches
#ifndef W4_GROUPED_BLOCKS
#define W4_GROUPED_BLOCKS 1024
#endif

unsigned grouped_grid(int Gmax, int tiles) {
    const long units = (long)(Gmax + 1) * tiles;
    return (unsigned)(units < W4_GROUPED_BLOCKS ? units : W4_GROUPED_BLOCKS);
}

void launch_gw13(GW13Args &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    a.tiles = (a.I + 15) / 16;
    const dim3 g(grouped_grid(a.Gmax, a.tiles)), b(256);
    auto with_fmt = [&](auto F, auto SBc) {
        constexpr int FMT = decltype(F)::value;
        constexpr bool SB = decltype(SBc)::value;
        switch (lanes_for_k(a.H)) {
        case 1: go_ev(st, e0, e1, k_moe_gw13<FMT, 1, SB>, g, b, 0, a); break;
        case 2: go_ev(st, e0, e1, k_moe_gw13<FMT, 2, SB>, g, b, 0, a); break;
        case 4: go_ev(st, e0, e1, k_moe_gw13<FMT, 4, SB>, g, b, 0, a); break;
        case 8: go_ev(st, e0, e1, k_moe_gw13<FMT, 8, SB>, g, b, 0, a); break;
        case 16: go_ev(st, e0, e1, k_moe_gw13<FMT, 16, SB>, g, b, 0, a); break;
        case 32: go_ev(st, e0, e1, k_moe_gw13<FMT, 32, SB>, g, b, 0, a); break;
        default: go_ev(st, e0, e1, k_moe_gw13<FMT, 64, SB>, g, b, 0, a); break;
        }
    };
    auto with_sb = [&](auto F) {
        if (a.s_bf16) with_fmt(F, std::true_type());
        else with_fmt(F, std::false_type());
    };
    if (a.fmt == FMT_NVFP4) with_sb(std::integral_constant<int, FMT_NVFP4>());
    else if (a.fmt == FMT_INT4) with_sb(std::integral_constant<int, FMT_INT4>());
    else with_sb(std::integral_constant<int, FMT_E2M1>());
}

void launch_gw2(GW2Args &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    a.tiles = (a.H + 63) / 64;
    const dim3 g(grouped_grid(a.Gmax, a.tiles)), b(256);
    auto with_fmt = [&](auto F, auto SBc) {
        constexpr int FMT = decltype(F)::value;
        constexpr bool SB = decltype(SBc)::value;
        switch (lanes_for_k(a.I)) {
        case 1: go_ev(st, e0, e1, k_moe_gw2<FMT, 1, SB>, g, b, 0, a); break;
        case 2: go_ev(st, e0, e1, k_moe_gw2<FMT, 2, SB>, g, b, 0, a); break;
        case 4: go_ev(st, e0, e1, k_moe_gw2<FMT, 4, SB>, g, b, 0, a); break;
        case 8: go_ev(st, e0, e1, k_moe_gw2<FMT, 8, SB>, g, b, 0, a); break;
        case 16: go_ev(st, e0, e1, k_moe_gw2<FMT, 16, SB>, g, b, 0, a); break;
        case 32: go_ev(st, e0, e1, k_moe_gw2<FMT, 32, SB>, g, b, 0, a); break;
        default: go_ev(st, e0, e1, k_moe_gw2<FMT, 64, SB>, g, b, 0, a); break;
        }
    };
    auto with_sb = [&](auto F) {
        if (a.s_bf16) with_fmt(F, std::true_type());
        else with_fmt(F, std::false_type());
    };
    if (a.fmt == FMT_NVFP4) with_sb(std::integral_constant<int, FMT_NVFP4>());
    else if (a.fmt == FMT_INT4) with_sb(std::integral_constant<int, FMT_INT4>());
    else with_sb(std::integral_constant<int, FMT_E2M1>());
}

// blocks of the large-batch launches (grid-stride over the units)
#ifndef W4_PF_BLOCKS
#define W4_PF_BLOCKS 1024  // a multiple of 8: unit u must stay on XCD u % 8
#endif
static_assert(W4_PF_BLOCKS % 8 == 0, "the large-batch unit order assumes a grid that is a multiple of 8");

void launch_pf13(GW13Args &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    a.tiles = a.I / PF_ROWS;
    const dim3 g(W4_PF_BLOCKS), b(256);
    const bool nv = a.fmt == FMT_NVFP4;
    if (a.s_bf16) go_ev(st, e0, e1, nv ? k_moe_pf13<FMT_NVFP4, true> : k_moe_pf13<FMT_E2M1, true>, g, b, 0, a);
    else go_ev(st, e0, e1, nv ? k_moe_pf13<FMT_NVFP4, false> : k_moe_pf13<FMT_E2M1, false>, g, b, 0, a);
}

void launch_pf2(GW2Args &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    a.tiles = a.H / PF_ROWS;
    const dim3 g(W4_PF_BLOCKS), b(256);
    const bool nv = a.fmt == FMT_NVFP4;
    if (a.s_bf16) go_ev(st, e0, e1, nv ? k_moe_pf2<FMT_NVFP4, true> : k_moe_pf2<FMT_E2M1, true>, g, b, 0, a);
    else go_ev(st, e0, e1, nv ? k_moe_pf2<FMT_NVFP4, false> : k_moe_pf2<FMT_E2M1, false>, g, b, 0, a);
}

void launch_mx_quant(MXQuantArgs &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    const int blocks = a.rows * (a.n >> 5);
    go_ev(st, e0, e1, k_mx_quant, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, a);
}

void launch_pfmx13(MX13Args &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    a.tiles = a.I / PF_ROWS;
    go_ev(st, e0, e1, k_moe_pfmx13, dim3(W4_PF_BLOCKS), dim3(256), 0, a);
}

void launch_pfmx2(MX2Args &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    a.tiles = a.H / PF_ROWS;
    go_ev(st, e0, e1, k_moe_pfmx2, dim3(W4_PF_BLOCKS), dim3(256), 0, a);
}

void launch_mx13(MX13Args &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    a.tiles = a.I / 32;
    go_ev(st, e0, e1, k_moe_mx13, dim3(grouped_grid(a.Gmax, a.tiles)), dim3(256), 0, a);
}

void launch_mx2(MX2Args &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    a.tiles = (a.H + 63) / 64;
    go_ev(st, e0, e1, k_moe_mx2, dim3(grouped_grid(a.Gmax, a.tiles)), dim3(256), 0, a);
}

void launch_mx_dot(const uint8_t *ac, const uint8_t *as, RowLayout arl, const uint8_t *bc, const uint8_t *bs,
                   float *out, int n, int m, int k, hipStream_t st) {
    hipLaunchKernelGGL(k_mx_dot, dim3((unsigned)(m / 16), (unsigned)(n / 16)), dim3(64), 0, st, ac, as, bc, bs, out,
                       n, m, k, arl);
}

void launch_gcombine(GCombineArgs &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    const dim3 g((unsigned)((a.H / 4 + 255) / 256), (unsigned)a.T), b(256);
    go_ev(st, e0, e1, k_moe_gcombine, g, b, 0, a);
}

}  // namespace w4k
