// Arguments and launchers of the batched-decode (expert-grouped) MoE kernels,
// shared by the entry points in w4moe_kernels.hip and their definitions in
// w4moe_grouped.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4k {

// Row addressing of one quantised matrix stack: row r of matrix e has its codes
// at e * n * cs + r * cs bytes from the codes base and its block scales at
// e * n * ss + r * ss bytes from the scale base.  Canonical layout: cs = code
// bytes per row, ss = scale bytes per row, separate arrays.  GFX950_V1: one
// record per row, cs = ss = the record size and the scale base = codes + k/2.
// bf16 rows: cs = 2k, no scales.
struct RowLayout {
    uint32_t cs, ss;
};

// Group table layout in the workspace: grp[0] = number of routed groups n,
// grp[1 + g] = expert, grp[1 + Gmax + g] = first pair-list entry,
// grp[1 + 2*Gmax + g] = pair count (g < n).  pairs[0 .. P) holds the routed
// pair ids p = t*k + j grouped by expert; pairs[P + t] = P + t are the shared
// expert's rows.
struct GroupArgs {
    const float *logits;   // [T][lstride] router logits (routed mode)
    const float *bias;     // [E] or null
    const int32_t *ids_in; // [T][k] caller routing (supplied mode)
    int32_t *ids_ws;       // [T][k] routing ids and weights for the combine
    float *w_ws;
    int32_t *ids_user;     // optional caller copies
    float *w_user;
    int32_t *grp;
    int32_t *pairs;
    int E, K, T, P, Gmax, lstride, route;
    int mfma_min;          // one-launch grouping: groups of >= 16 pairs first, then >= mfma_min, then the rest
};

// Column tiles of the large-batch kernels: the routed groups' 64-column tiles in
// group order, ctg[2c] = group index, ctg[2c + 1] = first column; their number
// is grp[1 + 3*Gmax] (the shared expert's ceil(T/64) tiles follow implicitly).
// Large batches group their pairs over three launches (k_route_topk,
// k_route_scan, k_route_scatter) instead of one block: per-block expert
// histograms in cntb [nblk][E], each block's base offset inside each expert's
// list in cbase [nblk][E] (written by the scan, so that every launch reads
// only what an earlier launch wrote and can run again on the same inputs), the
// expert of every pair in e_of [P], each expert's first pair-list entry in
// off_e [E].
struct RouteArgs {
    GroupArgs g;
    int32_t *e_of;
    int32_t *cntb;
    int32_t *cbase;
    int32_t *off_e;
    int32_t *ctg;  // [2 x column tiles]: routed group, first column (see k_route_scan)
    int nblk;
    int tpb;       // tokens per block of k_route_topk / k_route_scatter (<= ROUTE_MAX_TPB)
};
constexpr int ROUTE_MAX_TPB = 16;

struct GW13Args {
    const uint8_t *codes;   // routed W13 [E][2I][H/2]
    const void *scales;     // block scales (canonical array, or inside the row records)
    const uint8_t *s_codes; // shared W13 [2I][H/2] or null
    const void *s_scales;
    const uint16_t *x;      // [T][H]
    const int32_t *grp;
    const int32_t *pairs;
    uint16_t *h_hi;         // [P + T][I] bf16: h = h_hi + h_lo (see split_bf16)
    uint16_t *h_lo;
    int H, I, K, T, P, Gmax, tiles, mfma_min;
    const int32_t *ctg;     // column tiles (large-batch kernels only)
    int fmt;                // FMT_E2M1, FMT_NVFP4 or FMT_INT4 (gw13 / gw2; the large-batch kernels: not INT4)
    const float *gs, *s_gs; // NVFP4 global scales: routed [E], shared [1]
    int s_bf16;             // the shared expert is bf16 (s_codes = bf16 rows, no scales)
    RowLayout rl, s_rl;     // row strides of the routed and shared matrices
};

struct GW2Args {
    const uint8_t *codes;   // routed W2 [E][H][I/2]
    const void *scales;     // block scales (canonical array, or inside the row records)
    const uint8_t *s_codes; // shared W2 [H][I/2] or null
    const void *s_scales;
    const int32_t *grp;
    const int32_t *pairs;
    const uint16_t *h_hi;   // [P + T][I]
    const uint16_t *h_lo;
    float *out;             // [P + T][H]
    int H, I, K, T, P, Gmax, tiles, mfma_min;
    const int32_t *ctg;     // column tiles (large-batch kernels only)
    int fmt;                // as GW13Args
    const float *gs, *s_gs; // NVFP4 global scales: routed [E], shared [1]
    int s_bf16;             // the shared expert is bf16 (s_codes = bf16 rows, no scales)
    RowLayout rl, s_rl;     // row strides of the routed and shared matrices
};

struct GCombineArgs {
    const int32_t *ids;     // [T][k]
    const float *w;         // [T][k]
    const float *logits;    // [T][lstride], column E = shared-gate logit
    const float *out;       // [P + T][H]
    uint16_t *y;            // [T][H] bf16
    int H, E, K, T, P, lstride, has_shared;
};

// MX path (MXFP4 weights, MXFP8 activations): quantised activations in the
// workspace, natural K order: xq [T][H] E4M3 bytes + xs [T][H/32] E8M0 bytes;
// hq [P + T][I] + hs [P + T][I/32] likewise for the SwiGLU intermediate.
struct MXQuantArgs {
    const uint16_t *x;      // [rows][n] bf16
    uint8_t *q;             // [rows][n]
    uint8_t *s;             // [rows][n/32]
    int rows, n;
};

struct MX13Args {
    const uint8_t *codes;   // routed W13 [E][2I][H/2]
    const void *scales;     // E8M0 per 32 (canonical [E][2I][H/32], or inside the row records)
    const uint8_t *s_codes; // shared W13 or null
    const void *s_scales;
    const uint8_t *xq;      // [T][H]
    const uint8_t *xs;      // [T][H/32]
    const int32_t *grp;
    const int32_t *pairs;
    uint8_t *hq;            // [P + T][I]
    uint8_t *hs;            // [P + T][I/32]
    int H, I, K, T, P, Gmax, tiles;
    const int32_t *ctg;     // column tiles (large-batch kernels only)
    RowLayout rl, s_rl;     // row strides of the routed and shared matrices
};

struct MX2Args {
    const uint8_t *codes;   // routed W2 [E][H][I/2]
    const void *scales;     // E8M0 per 32 (canonical [E][H][I/32], or inside the row records)
    const uint8_t *s_codes;
    const void *s_scales;
    const int32_t *grp;
    const int32_t *pairs;
    const uint8_t *hq;
    const uint8_t *hs;
    float *out;             // [P + T][H]
    int H, I, K, T, P, Gmax, tiles;
    const int32_t *ctg;     // column tiles (large-batch kernels only)
    RowLayout rl, s_rl;     // row strides of the routed and shared matrices
};

size_t grouped_lds_bytes(int E, int P);
// large groups (prefill-sized batches): LDS-staged activations, 64-row units
void launch_pf13(GW13Args &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
void launch_pf2(GW2Args &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
void launch_route_multi(RouteArgs &a, hipStream_t st, hipEvent_t *ev);  // ev: 6 events or null
void launch_mx_quant(MXQuantArgs &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
void launch_pfmx13(MX13Args &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1);  // large batches
void launch_pfmx2(MX2Args &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
void launch_mx13(MX13Args &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
void launch_mx2(MX2Args &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
void launch_route_group(GroupArgs &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
// routed batches: ranking over ceil(T / 4) blocks, grouping by the last one to
// finish; `arrive` must read zero when the launch starts (the router zeroes it)
void launch_rank_group(GroupArgs &a, int32_t *arrive, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
void launch_gw13(GW13Args &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
void launch_gw2(GW2Args &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
void launch_gcombine(GCombineArgs &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
// test hook: out [n][m] = A (MXFP4) B^T (MXFP8) on the scaled FP4 MFMA; n, m % 16 == 0, k % 128 == 0
void launch_mx_dot(const uint8_t *ac, const uint8_t *as, RowLayout arl, const uint8_t *bc, const uint8_t *bs,
                   float *out, int n, int m, int k, hipStream_t st);

}  // namespace w4k
