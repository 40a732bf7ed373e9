/*
 * jpa_cat_pad.h -- fused cat + pad + zero-fill of causal Conv3D inputs, C ABI
 * (part of libjpa; uses jpa_status from jpa.h).
 *
 *   sglang PR #29281 review (Cosmos3 VAE decode): before each causal Conv3D
 *   the frames cached from the previous chunk are concatenated with the
 *   current frames along time and the result is zero-padded; the fused op
 *   fused_causal_conv3d_cat_pad(x, cache_x, padding) does both in one pass
 *   (padding listed last dimension first; the time-right pad is 0 in the
 *   pattern the page supports, any value is accepted here).
 *
 * Definition (tensors [B, C, T, H, W], contiguous):
 *     cat = [cache ; x] along T (cache frames first)
 *     out[b, c, t, h, w] = cat[b, c, t - tl, h - hl, w - wl] where that exists,
 *                          0 elsewhere
 *     padding = {wl, wr, hl, hr, tl, tr}; out is [B, C, Tc + T + tl + tr,
 *     H + hl + hr, W + wl + wr].
 * Elements are moved as 2-byte words (bf16 in the pages' decoder; fp16 works
 * the same), so the result is bit-exact and pad elements are +0.0.
 */
#ifndef JPA_CAT_PAD_H
#define JPA_CAT_PAD_H

#include "jpa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * jpa_causal_cat_pad -- enqueue the op on `stream` and return.
 *   x        device [batch, channels, frames, height, width], 2-byte elements
 *   cache    device [batch, channels, cache_frames, height, width]; may be NULL
 *            when cache_frames == 0
 *   padding  host int32[6] = {w_left, w_right, h_left, h_right, t_left, t_right},
 *            each >= 0 (applied to the concatenation: a caller padding for a
 *            causal kernel has already taken the cached frames off t_left)
 *   out      device [batch, channels, cache_frames + frames + t_left + t_right,
 *            height + h_left + h_right, width + w_left + w_right]; must not
 *            overlap x or cache
 *   stream   a hipStream_t (NULL = the default stream)
 * All pointers 16-byte aligned.  Limits: the output below 2^31 elements, each
 * output extent <= 65536.
 * Errors (host checks before any HIP call; nothing enqueued): JPA_ERR_NULL,
 * JPA_ERR_SHAPE (negative sizes, limits), JPA_ERR_VALUE (negative pad),
 * JPA_ERR_LAYOUT (alignment, overlap), JPA_ERR_HIP (launch rejected).  An
 * empty output enqueues nothing and returns JPA_OK.
 */
JPA_API jpa_status jpa_causal_cat_pad(const void* x, const void* cache, int32_t batch, int32_t channels,
                                      int32_t frames, int32_t cache_frames, int32_t height, int32_t width,
                                      const int32_t* padding, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif
