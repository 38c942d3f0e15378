// Arguments and launchers of the decode kernels of an MoE layer whose down
// projections are stored K-tiled (W4_LAYOUT_GFX950_KT16): the gate/up rows and
// the down projection of each 16-value slice of an expert's intermediate run in
// one launch, and a second launch sums the slices.  Shared by the entry points
// in w4moe_kernels.hip and the definitions in w4moe_decode.hip.
#pragma once

#include "w4moe_grouped.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4k {

constexpr int DEC_TILE = 16;     // intermediate values per block (one K tile of the down projection)
constexpr int DEC_WAVES = 8;     // waves per block: 2 gate + 2 up rows each
constexpr int DEC_MAX_H = 4096;  // hidden sizes up to 2 steps of 64 lanes x 32

struct DecArgs {
    const uint8_t *codes13;      // routed W13 [E][2I][H] in a row layout (rows [0,I) gate, [I,2I) up)
    const void *scales13;        // its block scales (canonical array or inside the row records)
    const uint8_t *s_codes13;    // shared W13 (or null)
    const void *s_scales13;
    const uint8_t *codes2;       // routed W2, K-tiled: [E][I/16][tile record of H rows]
    const uint8_t *s_codes2;     // shared W2, K-tiled (or null)
    const uint16_t *x;           // [T][H] bf16
    const float *logits;         // [T][lstride] (routed mode)
    const float *bias;           // [E] or null
    const int32_t *ids_in;       // [T][K] (supplied mode)
    int32_t *ids_ws;             // [T][K] routing for the combine
    float *w_ws;
    int32_t *ids_user;           // optional caller copies
    float *w_user;
    float *part;                 // [T][S][tiles][H] fp32 partial down projections
    const float *gs13, *s_gs13;  // NVFP4 global scales of W13: routed [E], shared [1]
    const float *gs2, *s_gs2;    // of W2
    RowLayout rl13, s_rl13;      // row strides of the W13 matrices
    uint32_t tile_bytes;         // K-tiled record of W2 (same for the shared W2)
    int H, I, E, K, S, T, tiles, lstride, route;
};

struct DecCombineArgs {
    const float *w;              // [T][K] routing weights
    const float *logits;         // [T][lstride], column E = shared-gate logit
    const float *part;           // [T][S][tiles][H]
    uint16_t *y;                 // [T][H] bf16
    int H, E, K, S, T, tiles, lstride, has_shared;
};

// fmt: FMT_E2M1 or FMT_NVFP4
void launch_dec(DecArgs &a, int fmt, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
void launch_dec_combine(DecCombineArgs &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1);

}  // namespace w4k
