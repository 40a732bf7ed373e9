// Launch arguments shared by the host front end (jpa_norm_rope_host.cpp) and
// the per-head RMSNorm + rotary kernel (jpa_norm_rope.hip).  Plain C++ data.
#ifndef JPA_NORM_ROPE_PARAMS_H
#define JPA_NORM_ROPE_PARAMS_H

#include <stdint.h>

// Index 0 is q, index 1 is k.  Rows are (token, head) pairs: rows
// [0, rows_q) are q's in token-major order, rows [rows_q, rows_total) k's.
struct jpa_norm_rope_params {
    const uint16_t* x[2];        // inputs, bf16 [tokens, heads, head_dim]
    uint16_t* y[2];              // outputs, same shapes (may be the inputs)
    int64_t x_ts[2], y_ts[2];    // token strides (elements)
    int32_t x_hs[2], y_hs[2];    // head strides (elements)
    int32_t heads[2];
    uint32_t div_magic[2];       // row -> token: t = (row * div_magic) >> div_shift, exact
    int32_t div_shift[2];        // for every row < 2^31 (rows of one tensor < 2^31)
    const float* w[2];           // per-channel norm weights, float [head_dim]
    const float* table;          // float [tokens, table_stride]: [cos | sin]
    int64_t table_stride;
    int64_t rows_q, rows_total;
    int32_t rotary_dim;          // even, 0 <= rotary_dim <= head_dim
    int32_t interleaved;         // 1: pairs (2i, 2i+1); 0: pairs (i, i + rotary_dim/2)
    float eps;
};

// Enqueue the kernel for head_dim 64, 128 or 256; returns a hipError_t value.
int jpa_launch_norm_rope(const jpa_norm_rope_params& p, int head_dim, void* stream);

#endif
