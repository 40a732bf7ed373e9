// Host front end of jpa_causal_cat_pad: argument checks (host only, before
// any HIP call) and the launch.
#include <cstdint>

#include "jpa.h"
#include "jpa_cat_pad.h"
#include "jpa_cat_pad_params.h"

namespace {

// Division by an invariant d (1 <= d <= 2^16) for dividends below 2^31:
// m = ceil(2^(31+l) / d), l = ceil(log2 d) gives floor(n / d) = (n * m) >>
// (31 + l) (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994, theorem 4.2).
void magic_for(int32_t d, uint32_t* magic, int32_t* shift) {
    int l = 0;
    while ((int64_t(1) << l) < d) ++l;
    const uint64_t num = uint64_t(1) << (31 + l);
    *magic = (uint32_t)((num + (uint64_t)d - 1) / (uint64_t)d);
    *shift = 31 + l;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

JPA_API jpa_status jpa_causal_cat_pad(const void* x, const void* cache, int32_t batch, int32_t channels,
                                      int32_t frames, int32_t cache_frames, int32_t height, int32_t width,
                                      const int32_t* padding, void* out, void* stream) {
    if (!padding) return JPA_ERR_NULL;
    if (batch < 0 || channels < 0 || frames < 0 || cache_frames < 0 || height < 0 || width < 0)
        return JPA_ERR_SHAPE;
    for (int i = 0; i < 6; ++i)
        if (padding[i] < 0) return JPA_ERR_VALUE;
    const int64_t w_out = (int64_t)width + padding[0] + padding[1];
    const int64_t h_out = (int64_t)height + padding[2] + padding[3];
    const int64_t t_out = (int64_t)cache_frames + frames + padding[4] + padding[5];
    if (w_out > 65536 || h_out > 65536 || t_out > 65536) return JPA_ERR_SHAPE;
    const int64_t rows = (int64_t)batch * channels;
    const int64_t out_numel = rows * t_out * h_out * w_out;
    if (out_numel >= (int64_t(1) << 31)) return JPA_ERR_SHAPE;
    const int64_t plane = (int64_t)height * width;
    const int64_t x_numel = rows * frames * plane, cache_numel = rows * cache_frames * plane;
    if (out_numel == 0) return JPA_OK;
    if (!out || (x_numel > 0 && !x) || (cache_numel > 0 && !cache)) return JPA_ERR_NULL;
    if (!aligned16(out) || !aligned16(x) || !aligned16(cache)) return JPA_ERR_LAYOUT;
    // the output must not overlap an input
    auto overlap = [](const void* a, int64_t na, const void* b, int64_t nb) {
        if (na == 0 || nb == 0) return false;
        const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
        return pa < pb + 2 * (uintptr_t)nb && pb < pa + 2 * (uintptr_t)na;
    };
    if (overlap(out, out_numel, x, x_numel) || overlap(out, out_numel, cache, cache_numel)) return JPA_ERR_LAYOUT;

    jpa_cat_pad_params p{};
    p.x = static_cast<const uint16_t*>(x);
    p.cache = static_cast<const uint16_t*>(cache);
    p.out = static_cast<uint16_t*>(out);
    p.x_numel = x_numel;
    p.cache_numel = cache_numel;
    p.out_numel = (uint32_t)out_numel;
    p.chunks = (uint64_t)(out_numel + 7) / 8;
    p.frames = frames;
    p.cache_frames = cache_frames;
    p.height = height;
    p.width = width;
    p.t_out = (int32_t)t_out;
    p.h_out = (int32_t)h_out;
    p.w_out = (int32_t)w_out;
    p.pad_w0 = padding[0];
    p.pad_h0 = padding[2];
    p.pad_t0 = padding[4];
    magic_for(p.w_out, &p.w_magic, &p.w_shift);
    magic_for(p.h_out, &p.h_magic, &p.h_shift);
    magic_for(p.t_out, &p.t_magic, &p.t_shift);
    return jpa_launch_cat_pad(p, stream) == 0 ? JPA_OK : JPA_ERR_HIP;
}

}  // extern "C"
