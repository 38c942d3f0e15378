/*
 * w4moe.h - C ABI of the W4A16 mixture-of-experts decode layer and the dense
 * W4A16 GEMV for AMD Instinct MI355X (gfx950).
 *
 * Method sources (cited by page title and section):
 *   [LE]   "Lynn Engine" article (zingnex.cn): "Native NVFP4 quantization support"
 *          (W4A16: 4-bit weights, bf16 activations) and "Kernel optimisation
 *          history", stage P1 (packed E2M1 codes + an FP16 scale per 16 K
 *          elements read directly by the matvec; 8192x2048 = 10.00 MiB vs 32.00).
 *   [README] lynn-engine README (GitHub), status notes: P28 gate_up_silu
 *          (grouped packed experts + per-16 scale + top-k ids -> [top_k, I]),
 *          P29 down_weighted_sum ([top_k, I] + routing weights -> [H]),
 *          P45 one-call active-MoE ABI (hidden, expert_ids, routing_weights,
 *          gate_up, down -> out[H]), P46/P48 (no float atomics; output rows owned
 *          by one block), P35 (sorted top-k), P23 (int32 expert ids),
 *          P59 (unknown layouts fail loudly).
 *   [TUT]  lynn-engine tutorials index: note 06 (router = softmax over all experts
 *          -> top-K -> renormalise, plus a sigmoid-gated shared expert) and the
 *          Qwen 3.6 35B-A3B configuration block (hidden 2048, 256 experts, top-8).
 *   [CI]   "cuda_inf" article: "2. INT4 weight quantization" (signed int4, one
 *          scale per group of 128 along K, fp32 accumulate).
 *   NVFP4 variant: lynn-engine README notes P17/P54 (per-16 E4M3 scales), R5-C0
 *          (UE4M3 block-16 scales) and P29 (down projection with packed codes,
 *          scales and a global scale).
 *
 * Conventions (all entry points):
 *   - Status: 0 = W4_OK, negative = error.  Every argument is validated before
 *     anything is launched; on error nothing is launched and w4_last_error()
 *     returns a message for the calling thread.  An unknown format or layout tag
 *     is an error, never a fallback.
 *   - Ownership: the caller owns every buffer.  The library never allocates,
 *     frees or synchronises device memory.
 *   - Device entry points are asynchronous on `stream` (a hipStream_t; NULL is
 *     the default stream): outputs are valid once the stream reaches the work.
 *   - Host entry points (sizes, quantise, pack) never touch the GPU, so they work
 *     on a machine without one.
 *   - bf16 and fp16 values are passed as their 16-bit patterns (uint16_t).
 *   - Results are deterministic: fixed reduction orders, no float atomics.
 *   - Thread safety: no global mutable state besides the thread-local error
 *     message and the per-device scratch address of moe_w4a16_forward_noalloc
 *     (set once under a lock); concurrent calls on distinct streams with
 *     distinct outputs and workspaces are safe.
 */
#ifndef W4MOE_H
#define W4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */
#define W4_OK 0
#define W4_ERR_INVALID_ARG (-1)   /* null pointer, bad size or count            */
#define W4_ERR_LAYOUT (-2)        /* unknown format or layout tag, or mismatch  */
#define W4_ERR_ALIGNMENT (-3)     /* pointer not aligned as documented          */
#define W4_ERR_UNSUPPORTED (-4)   /* valid request the library does not serve   */
#define W4_ERR_WORKSPACE (-5)     /* workspace missing or too small             */
#define W4_ERR_NONFINITE (-6)     /* quantise: Inf or NaN in the input          */
#define W4_ERR_RANGE (-7)         /* quantise: block scale overflows its format */
#define W4_ERR_HIP (-8)           /* a HIP runtime call or launch failed        */

/* ------------------------------------------------------------------ formats */
/* E2M1 codes (OCP MX FP4: 1 sign, 2 exponent bits bias 1, 1 mantissa bit) with
 * one FP16 scale per 16 consecutive K elements [LE stage P1]. */
#define W4_FMT_E2M1_F16S16 1
/* Two's-complement int4 codes in [-8, 7] with one FP16 scale per 128 K
 * elements [CI "2. INT4 weight quantization"]. */
#define W4_FMT_INT4_F16S128 2
/* NVFP4: E2M1 codes with one unsigned E4M3 scale byte (OCP E4M3, sign 0, at
 * most 448) per 16 consecutive K elements and one fp32 global scale per matrix;
 * element value = code x scale x global. */
#define W4_FMT_NVFP4_E4M3S16 3
/* Unquantised bf16 weights: `codes` holds bf16 bit patterns [groups][n][k]
 * (2 bytes per element), no scales.  Accepted for the shared expert of an MoE
 * layer (the pages' engine keeps it in bf16: lynn-engine README P15/P37) and by
 * w4_quantize (round to nearest even); the GEMV and dequant hook reject it. */
#define W4_FMT_BF16 4
/* MXFP4 (OCP Microscaling v1.0): E2M1 codes with one E8M0 scale byte (2^(byte -
 * 127)) per 32 K elements; scales [groups][n][k/32] bytes.  The vendor
 * block-scaled format the pages bridge to (README P17/P54, R5-B "e8m0/group32").
 * In an MoE layer it takes MXFP8 activations: the layer input and the SwiGLU
 * intermediate are quantised to E4M3 elements with an E8M0 scale per 32
 * (X = floor(log2 absmax) - 8, round to nearest even, clamp to +-448), so such a
 * layer computes W4A8 (MX): batches on gfx950's scaled FP4 MFMA, 1-3 tokens on
 * the single-token VALU kernels (exact products, fp32 sums); the dense GEMV
 * does not take this format. */
#define W4_FMT_MXFP4_E8M0S32 5

/* Canonical layout (the quantiser's output and the exchange format):
 *   codes  [groups][n][k/2] bytes, element 2j in the low nibble of byte j and
 *          element 2j+1 in the high nibble;
 *   scales [groups][n][k/G] fp16 bit patterns, G = 16 (E2M1) or 128 (int4);
 *          NVFP4: [groups][n][k/16] UE4M3 bytes; MXFP4: [groups][n][k/32] E8M0;
 *   global_scales (NVFP4 only) [groups] fp32.
 * With y = W x, a row is one output element.  A wave streams 1 KiB of one
 * row's codes per 128-bit load (64 lanes x 16 B = 32 elements per lane, two
 * whole E2M1 scale blocks) and the matching 256 B of scales per 32-bit load. */
#define W4_LAYOUT_CANONICAL 0
/* Device layout for gfx950 (the packed-weight layout of [LE stage P1], the
 * packed codes and their per-16 scales read directly by the matvec, with the
 * scales placed next to the codes they scale):
 *   codes  one record of R bytes per row, rows in [groups][n] order: the row's
 *          k/2 code bytes in the canonical nibble order (the operand order of
 *          gfx950's packed fp4 conversion: byte j's low nibble is element 2j),
 *          then the row's k/G block scales in K order, then zero padding up to
 *          R = the next multiple of 16 (E2M1 at k = 2048: 1024 + 256 = 1280 B);
 *   scales unused (may be NULL): w4_scales_bytes() returns 0;
 *   global_scales (NVFP4) as in the canonical layout.
 * Every load of a row, codes and scales, falls in one contiguous record (one
 * DRAM stream per row instead of two arrays), and the record stride is not a
 * power of two, so the 16-row MFMA tiles of the batched kernels spread over
 * the memory channels.  bf16 matrices have no scales: both layouts coincide.
 * Every entry point that takes a w4_matrix reads it; w4_pack / w4_unpack
 * convert between it and the canonical layout. */
#define W4_LAYOUT_GFX950_V1 1
/* K-tiled device layout for down projections in decode (E2M1 and NVFP4 only):
 *   codes  per group, per 16-wide K tile t (k/16 tiles): one record of the
 *          tile for every row, the n rows' 8 code bytes of elements 16t..16t+15
 *          (canonical nibble order), then the n rows' scale of that tile (FP16
 *          or UE4M3), then zero padding to a multiple of 16 bytes (at n = 2048,
 *          E2M1: 16,384 + 4,096 = 20,480 B per tile);
 *   scales unused (may be NULL); global_scales (NVFP4) as canonical.
 * A block that owns 16 intermediate values of one expert reads its whole
 * share of that expert's down projection as one contiguous record, so the
 * down projection can be split over K (the intermediate dimension) and run in
 * the same launch as the gate/up rows that produce those 16 values.  The MoE
 * layer takes it for w2 and shared_w2 (its decode kernels, any T); the dense
 * GEMV, which dots whole rows, does not. */
#define W4_LAYOUT_GFX950_KT16 2

/* A stack of `groups` quantised matrices W[g] of shape [n][k] (y = W x).
 * Requirements: k % 32 == 0 (E2M1, NVFP4) or k % 128 == 0 (int4); codes
 * 16-byte aligned; scales and global_scales 4-byte aligned; all in device
 * memory for device calls.  global_scales is required for NVFP4 and ignored
 * (may be NULL) for the other formats. */
typedef struct w4_matrix {
    int32_t format;              /* W4_FMT_*                                */
    int32_t layout;              /* W4_LAYOUT_*                             */
    int64_t groups;              /* number of stacked matrices (experts)    */
    int64_t n;                   /* rows per matrix                         */
    int64_t k;                   /* columns = reduction length              */
    const uint8_t *codes;        /* packed codes, see the layout above      */
    const void *scales;          /* fp16 bit patterns, or UE4M3 bytes       */
    const float *global_scales;  /* NVFP4: fp32 [groups]; otherwise unused  */
} w4_matrix;

/* ------------------------------------------------------------------ errors */
/* Name of a status code ("W4_OK", "W4_ERR_LAYOUT", ...); never NULL. */
const char *w4_status_string(int status);
/* Message describing the last failing call on this thread ("" if none). */
const char *w4_last_error(void);
/* Library version string. */
const char *w4_version(void);

/* ------------------------------------------------------------------ sizes (host) */
/* Bytes of packed codes / scales for `groups` matrices of [n][k] in a layout:
 * canonical: codes = groups*n*k/2, scales = groups*n*(k/G)*2 (NVFP4:
 * groups*n*(k/16)); GFX950_V1: codes = groups*n*R (the row record above),
 * scales = 0; GFX950_KT16: codes = groups*(k/16)*(tile record), scales = 0.
 * 8192x2048 E2M1 gives 8,388,608 + 2,097,152 = 10,485,760 B = 10.00 MiB
 * [LE stage P1]; NVFP4 8,388,608 + 1,048,576 = 9.00 MiB (+ 4 B global).
 * Returns 0 for an unknown format/layout or a k the format does not accept. */
size_t w4_codes_bytes(int32_t format, int32_t layout, int64_t groups, int64_t n, int64_t k);
size_t w4_scales_bytes(int32_t format, int32_t layout, int64_t groups, int64_t n, int64_t k);

/* ------------------------------------------------------------------ quantise (host) */
/* Quantise host fp32 weights w[n][k] (row-major, one matrix) into canonical
 * codes [n][k/2] and scales [n][k/G] (host buffers of w4_codes_bytes /
 * w4_scales_bytes with groups = 1).  Offline step before upload [LE stage P1;
 * CI "2. INT4 weight quantization"].  Per block of G elements:
 *   scale = round-to-nearest-even fp16 of (fp32 absmax / 6)   (E2M1)
 *                                        (fp32 absmax / 7)   (int4);
 *   code  = nearest code to fp32(w) / fp32(scale) (IEEE fp32 division), ties to
 *           the even code, saturating at +-6; int4: round half to even, clip to
 *           [-8, 7]; an all-zero block has scale 0 and zero codes; a value that
 *           rounds to magnitude zero is encoded as +0.
 * NVFP4 (the pages name the scale types, not a recipe; this is the common one):
 *   g = fp32(absmax(w)) / 2688 (= 6 x 448), written to *global_scale;
 *   block scale = UE4M3 round-to-nearest-even of fp32(fp32(block absmax) / 6) / g,
 *   saturating at 448; code = nearest E2M1 value to fp32(w) / fp32(scale x g),
 *   ties to even, +0 for zero; an all-zero matrix has g = 0.
 * bf16: codes receives bf16 bit patterns [n][k] (round to nearest even), scales
 * and global_scale are unused.
 * MXFP4: per 32 elements X = floor(log2 absmax) - 2 (limited to [-127, 127]),
 * scale byte X + 127, code = nearest E2M1 value to w / 2^X, ties to even,
 * clamped to +-6, +0 for zero; an all-zero block has byte 0.
 * global_scale may be NULL for the FP16-scale formats.
 * Errors: W4_ERR_NONFINITE (Inf/NaN input), W4_ERR_RANGE (a block scale would
 * overflow fp16), W4_ERR_INVALID_ARG, W4_ERR_LAYOUT.  Synchronous, thread-safe. */
int w4_quantize(int32_t format, const float *w, int64_t n, int64_t k,
                uint8_t *codes, void *scales, float *global_scale);

/* Canonical <-> device layout for a stack of `groups` [n][k] matrices (host
 * buffers, synchronous).  w4_pack reads canonical codes / scales and writes
 * dst_layout (GFX950_V1 / GFX950_KT16: records into codes_out, sized by
 * w4_codes_bytes; scales_out unused and may be NULL; CANONICAL: a copy).  w4_unpack reads
 * src_layout and writes canonical codes and scales.  Bytes are only moved, so
 * the two are exact inverses (the V1 padding is written as zeros and ignored on
 * unpack).  The pages fix no device layout; unknown tags fail loudly
 * (lynn-engine README P59).  Errors: W4_ERR_LAYOUT, W4_ERR_INVALID_ARG. */
int w4_pack(int32_t format, int64_t groups, int64_t n, int64_t k, const uint8_t *codes, const void *scales,
            int32_t dst_layout, uint8_t *codes_out, void *scales_out);
int w4_unpack(int32_t format, int64_t groups, int64_t n, int64_t k, int32_t src_layout, const uint8_t *codes_in,
              const void *scales_in, uint8_t *codes, void *scales);

/* Host helpers between one-nibble-per-byte codes [n][k] (values 0..15) and the
 * packed canonical codes [n][k/2] (low nibble = even element).  Exact inverses
 * for any input; w4_pack_nibbles rejects a nibble > 15 (W4_ERR_INVALID_ARG). */
int w4_pack_nibbles(const uint8_t *nibbles, int64_t n, int64_t k, uint8_t *packed);
int w4_unpack_nibbles(const uint8_t *packed, int64_t n, int64_t k, uint8_t *nibbles);

/* ------------------------------------------------------------------ dense GEMV */
/* y[m][n] = x[m][k] . W[n][k]^T for the single matrix W (groups must be 1):
 * the packed W4A16 matvec of [LE stage P1] (m = 1 for decode).  Codes are
 * dequantised in registers (exactly: code value x fp32(scale)), products are
 * accumulated in fp32 (NVFP4: the row sum is multiplied by the global scale)
 * and each output is rounded once to bf16 (nearest even).
 *   x: device bf16 [m][k], 16-byte aligned;  y: device bf16 [m][n].
 * Supports 1 <= m <= 64.  Errors: W4_ERR_INVALID_ARG, _LAYOUT, _ALIGNMENT,
 * _UNSUPPORTED, _HIP. */
int w4a16_gemv(const w4_matrix *W, const uint16_t *x, int64_t m, uint16_t *y, void *stream);

/* Test hook: dequantise every element of W (all groups) to fp32
 * out[groups][n][k] on the device with the same in-register decode the GEMV
 * and MoE kernels use.  Bit-exact by construction (each product is exact;
 * NVFP4: code x scale is exact and its product with the global scale is
 * rounded once). */
int w4_dequant_device(const w4_matrix *W, float *out, void *stream);

/* Test hook of the MXFP4 path's matrix instruction: out[i][j] = sum_k A[i][k] B[j][k]
 * (fp32 [n][m], row-major) for an MXFP4 matrix A (groups = 1) and an MXFP8 matrix
 * B given as E4M3 codes [m][k] (16-byte aligned) and E8M0 scale bytes [m][k/32],
 * on gfx950's scaled FP4 MFMA with the operand mapping and accumulation chain
 * the MX expert kernels use (each 128-wide K chunk added into one fp32
 * accumulator).  Lets a test pin the instruction's rounding, which the MX
 * parity bounds rely on (lynn-engine README P17/P18: e8m0/32 scale bridges).
 * Needs n, m multiples of 16 and k a multiple of 128.  Errors: W4_ERR_LAYOUT
 * (A not MXFP4), W4_ERR_UNSUPPORTED, W4_ERR_INVALID_ARG, _ALIGNMENT, _HIP. */
int w4_mx_dot_device(const w4_matrix *A, const uint8_t *b_codes, const uint8_t *b_scales, int64_t m, float *out,
                     void *stream);

/* Measurement aid (not a step of the layer): read `bytes` (a multiple of 16) of
 * device memory at src with 128-bit loads spread over the whole GPU, one per
 * thread in as many 256-thread blocks as the buffer needs (the fastest plain read
 * measured on MI355X), and write nothing but, with negligible probability, one word
 * to *sink (device, 4-byte aligned).  Timing it gives the practical HBM read
 * ceiling for a buffer of that size, the second denominator beside the 8 TB/s
 * peak.  Asynchronous on `stream`.  Errors: W4_ERR_INVALID_ARG, _ALIGNMENT, _HIP. */
int w4_bench_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* ------------------------------------------------------------------ MoE layer */
/* One MoE decode layer [TUT note 06 and the 35B-A3B config; README P28/P29/P45].
 *   router_w      bf16 [E][H]                  router weight (logits = Wr x)
 *   router_bias   fp32 [E] or NULL             added to the logits before softmax
 *   w13           groups = E, n = 2I, k = H    rows [0,I) gate, [I,2I) up
 *   w2            groups = E, n = H,  k = I    down projection
 *   has_shared    0/1; if 1:
 *     shared_w13  groups = 1, n = 2*shared_inter, k = H
 *     shared_w2   groups = 1, n = H, k = shared_inter
 *                 in the routed experts' format or both W4_FMT_BF16
 *     shared_gate_w bf16 [H]: sigma = sigmoid(shared_gate_w . x)
 * The library requires shared_inter == inter and H % 64 == 0; the routed experts
 * use one format (NVFP4: one global scale per expert matrix, applied to the
 * gate/up sums and to the down sums), the shared expert that format or bf16
 * (MXFP4: that format only). */
typedef struct moe_w4a16_layer {
    int64_t hidden;              /* H */
    int64_t inter;               /* I (expert intermediate) */
    int64_t num_experts;         /* E */
    int64_t top_k;               /* k */
    int64_t shared_inter;        /* shared expert intermediate (if has_shared) */
    const uint16_t *router_w;
    const float *router_bias;
    w4_matrix w13;
    w4_matrix w2;
    int32_t has_shared;
    w4_matrix shared_w13;
    w4_matrix shared_w2;
    const uint16_t *shared_gate_w;
} moe_w4a16_layer;

/* Bytes of device workspace moe_w4a16_forward / moe_w4a16_experts need for T
 * tokens (0 on invalid arguments).  The caller allocates it (e.g. with torch);
 * its contents need no initialisation and are scratch between calls. */
size_t moe_w4a16_workspace_bytes(const moe_w4a16_layer *L, int64_t T);

/* Full layer for T tokens, 1 <= T <= 16384 (decode: T = 1; batched decode and
 * prefill: T > 1):
 *   logits = Wr x (+ bias); p = softmax over all E; ids = the k largest p,
 *   sorted by descending p, ties to the lower expert id; w = p[ids] / sum
 *   (computed as softmax over the k selected logits, the equal form [TUT 06]);
 *   y = sum_j w_j * W2[e_j] (silu(gate_j) * up_j) + sigma * shared(x),
 *   gate_j/up_j = rows of W13[e_j] x; every intermediate in fp32; y rounded
 *   once to bf16.
 *   x: device bf16 [T][H] (16-byte aligned);  y: device bf16 [T][H].
 *   topk_ids: device int32 [T][k] or NULL;  topk_w: device fp32 [T][k] or NULL.
 *   ws: device workspace of at least moe_w4a16_workspace_bytes(L, T), 256-byte
 *   aligned; its contents need no initialisation (the launches write every
 *   intermediate, including the ranking's arrival counter, before reading it),
 *   and two calls in flight at once must not share it.
 * Errors: W4_ERR_INVALID_ARG, _LAYOUT, _ALIGNMENT, _UNSUPPORTED, _WORKSPACE, _HIP. */
int moe_w4a16_forward(const moe_w4a16_layer *L, const uint16_t *x, int64_t T, uint16_t *y,
                      int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, void *stream);

/* Measurement variant of moe_w4a16_forward: identical work, with each kernel
 * launched through hipExtLaunchKernel so that the runtime records the
 * caller's events at the kernel's start and end on `stream`.  `events` holds
 * 2 * moe_w4a16_stage_count(L, T) hipEvent_t (start/stop per kernel, in launch
 * order; n_events gives the array length).  The router pair is not recorded
 * for a layer whose router is skipped.  Not for use under stream capture.
 * Errors as moe_w4a16_forward, plus W4_ERR_INVALID_ARG for too few or null
 * events. */
int moe_w4a16_forward_timed(const moe_w4a16_layer *L, const uint16_t *x, int64_t T, uint16_t *y,
                            int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, void *stream,
                            void *const *events, int32_t n_events);

/* Number of kernels moe_w4a16_forward launches for T tokens (0 on invalid
 * arguments): 3 for the single-token path (router; grouped W13 + SiLU over
 * every (token, slot); down + combine), 5 for the batched path (router; top-k
 * and grouping of the (token, slot) pairs by expert; W13 + SiLU per expert
 * group, on MFMA for groups of at least 2 tokens; W2 per expert group; ordered
 * combine).  The batched path serves E2M1 and NVFP4 layers with H and I
 * multiples of 128 and at most 4096, T >= 4 and T * top_k <= 65536 (NVFP4: one
 * exact bf16 MFMA term per weight instead of two, the global scales applied to
 * the sums; a bf16 shared expert: its rows are the MFMA operands), and int4
 * layers up to T * top_k = 4096 (the codes on the MFMA, each 128-wide chunk's
 * sums times its scale); other requests take the single-token path.  MXFP4 layers need H and I multiples of 128 and a shared
 * expert in MXFP4 (W4_ERR_UNSUPPORTED otherwise); from T = 4 they run 6
 * kernels (router; x to MXFP8; top-k and grouping; W13 + SiLU with h quantised
 * to MXFP8; W2; ordered combine), below it the 3 single-token kernels, which
 * quantise x and h in registers.  E2M1, NVFP4 and MXFP4 batches of more than
 * 1024 (token, slot) pairs (T > 128 at top-8; at most 65536 pairs, T <= 16384)
 * group their pairs over three launches (per-block top-k and expert
 * histograms; one scan; a scatter) instead of one, so the grouped path takes 7
 * kernels (MXFP4: 8), and run W13 and W2 as grouped GEMMs with LDS-staged
 * activations; int4 batches keep the one-launch grouping and the per-group
 * kernels up to their 4096-pair limit; from T = 160 the router runs on MFMA.  E2M1 requests beyond 65536 pairs take the
 * single-token path; MXFP4 ones fail with W4_ERR_UNSUPPORTED.
 * Sources: lynn-engine README, R5 notes (tokens-per-expert grouping, inverse
 * scatter) and P85-P92 (per-16 scales applied exactly). */
int moe_w4a16_stage_count(const moe_w4a16_layer *L, int64_t T);

/* Size of the scratch array of moe_w4a16_forward_noalloc (per GPU). */
#define W4_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

/* moe_w4a16_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The intermediates live in a scratch array
 * of W4_NOALLOC_SCRATCH_BYTES (8 MiB) that the library keeps in each GPU's
 * memory until the process ends; this call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine).  The first call on a device looks up
 * that device's scratch address (hipGetSymbolAddress) with the device current,
 * so call it with the device of `stream` current.  Arguments and results as
 * moe_w4a16_forward; the caller still owns x, y, topk_ids and topk_w.  A batch
 * whose workspace (moe_w4a16_workspace_bytes) exceeds the scratch fails with
 * W4_ERR_WORKSPACE before anything is launched (about T = 64 tokens at the
 * 35B-A3B shape fit).  Every call on a GPU shares that GPU's scratch: calls
 * that overlap on one GPU (other streams, other threads) race, so serialise
 * them; the scratch keeps the last call's contents, none of which a later call
 * reads before writing it.  Errors as moe_w4a16_forward, plus W4_ERR_HIP if the
 * scratch address cannot be obtained. */
int moe_w4a16_forward_noalloc(const moe_w4a16_layer *L, const uint16_t *x, int64_t T, uint16_t *y,
                              int32_t *topk_ids, float *topk_w, void *stream);

/* Experts and combine only, with caller-supplied routing (the one-call shape of
 * README P45): ids int32 [T][k] in [0, E), w fp32 [T][k] (used as given).  The
 * shared expert, if present, is still added with its sigmoid gate. */
int moe_w4a16_experts(const moe_w4a16_layer *L, const uint16_t *x, int64_t T,
                      const int32_t *ids, const float *w, uint16_t *y,
                      void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* W4MOE_H */
