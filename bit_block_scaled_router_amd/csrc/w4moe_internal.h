// Internal declarations shared by the host and device translation units of the
// w4moe library (status handling and shape checks).
#pragma once

#include "w4moe.h"  // include/ is on the include path

namespace w4 {

// Record a message for w4_last_error() on this thread and return `status`.
int fail(int status, const char *fmt, ...);
void clear_error();

// Scale block length of a format (16, 32 or 128; bf16: 32, its K granule), 0 for
// an unknown tag.
int group_of(int32_t format);

// Bytes per matrix row: codes (bf16: 2 per element), block scales, and the
// GFX950_V1 row record (codes then scales, padded to a multiple of 16).
size_t code_bytes_per_row(int32_t format, int64_t k);
size_t scale_bytes_per_row(int32_t format, int64_t k);
size_t v1_row_bytes(int32_t format, int64_t k);
// GFX950_KT16 tile record of an n-row matrix: n x 8 code bytes, n scales, padded to 16.
size_t kt16_tile_bytes(int32_t format, int64_t n);

// Validate format/layout tags and dimensions of a matrix stack.
int check_shape(int32_t format, int32_t layout, int64_t groups, int64_t n, int64_t k);

}  // namespace w4
