// Launch arguments of the cat + pad kernel (jpa_cat_pad.hip), filled by the
// host front end (jpa_cat_pad_host.cpp).  Plain C++ data.
#ifndef JPA_CAT_PAD_PARAMS_H
#define JPA_CAT_PAD_PARAMS_H

#include <stdint.h>

struct jpa_cat_pad_params {
    const uint16_t* x;           // [B, C, frames, height, width], 2-byte elements
    const uint16_t* cache;       // [B, C, cache_frames, height, width] (may be null if none)
    uint16_t* out;               // [B, C, t_out, h_out, w_out]
    int64_t x_numel, cache_numel;
    uint32_t out_numel;          // < 2^31
    uint64_t chunks;             // ceil(out_numel / 8)
    int32_t frames, cache_frames, height, width;
    int32_t t_out, h_out, w_out;
    int32_t pad_w0, pad_h0, pad_t0;   // left pads (right pads follow from the sizes)
    // exact division by w_out, h_out, t_out for dividends below 2^31:
    // n / d = (n * magic) >> shift
    uint32_t w_magic, h_magic, t_magic;
    int32_t w_shift, h_shift, t_shift;
};

int jpa_launch_cat_pad(const jpa_cat_pad_params& p, void* stream);

#endif
