/*
 * jpa_norm_rope.h -- per-head Q/K RMSNorm + rotary embedding, C ABI (part of
 * libjpa; uses jpa_tensor and jpa_status from jpa.h).
 *
 * The step right before attention in a DiT block, producing the attention
 * inputs q and k in the packed [tokens, heads, head_dim] layout jpa_forward
 * takes:
 *   vLLM-Omni diffusion performance-patterns guide, section "Q/K RMSNorm +
 *     RoPE": RMSNorm of q and of k over head_dim with per-channel weights
 *     (separate for q and k) and an epsilon, then the rotary embedding from
 *     one per-token non-interleaved [cos | sin] table; pairs are interleaved
 *     (GPT-J style, is_neox_style=False) or half-split (NeoX style); with a
 *     partial rotary dimension the first rotary_dim channels are rotated and
 *     the rest pass through.
 *   sglang PR #26973 review, Cosmos3 attention snippet: q and k are slices of
 *     a fused QKV projection; rms_norm over head_dim, then rotary, then the
 *     attention call.
 *
 * Definition, per token t and head h of q (and of k, with k_weight):
 *     y_d  = x_d / sqrt(mean_d(x_d^2) + eps) * weight_d
 *     for pair i < rotary_dim/2 with channels (a, b) = (2i, 2i+1) if
 *     interleaved, else (i, i + rotary_dim/2), and
 *     c = table[t*table_stride + i], s = table[t*table_stride + rotary_dim/2 + i]:
 *         out_a = y_a c - y_b s,   out_b = y_b c + y_a s
 *     out_d = y_d for d >= rotary_dim.
 * Arithmetic is fp32; the result is rounded to bf16 (nearest even) once.
 */
#ifndef JPA_NORM_ROPE_H
#define JPA_NORM_ROPE_H

#include "jpa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * jpa_qk_norm_rope -- enqueue the step on `stream` and return.
 *   q, k          bf16 [T, Hq, D] and [T, Hkv, D] (same T; views allowed, e.g.
 *                 the q and k slices of a fused QKV tensor); D is 64, 128 or
 *                 256; the jpa_tensor rules of jpa.h apply (16-byte aligned
 *                 data, strides multiples of 8 elements)
 *   q_weight, k_weight  device float [D], 16-byte aligned
 *   table         device float, row t at table + t*table_stride holding
 *                 [cos_0 .. cos_{r/2-1} | sin_0 .. sin_{r/2-1}], r = rotary_dim;
 *                 4-byte aligned; table_stride >= rotary_dim; may be NULL when
 *                 rotary_dim == 0
 *   rotary_dim    even, 0 <= rotary_dim <= D
 *   interleaved   1: pairs (2i, 2i+1); 0: pairs (i, i + rotary_dim/2)
 *   eps           finite, >= 0 (a zero row with eps == 0 gives NaN, as the
 *                 definition does)
 *   q_out, k_out  bf16, shaped like q and k.  An output is either exactly its
 *                 input (in place, same data and strides) or shares no element
 *                 with either input; the outputs share no element with each
 *                 other.  Views of one buffer with equal token strides whose
 *                 per-token column ranges do not meet count as sharing none.
 *   stream        a hipStream_t (NULL = the default stream)
 * All checks run on the host before any HIP call; nothing is enqueued on
 * error.  Errors: JPA_ERR_NULL (missing pointer), JPA_ERR_DTYPE, JPA_ERR_SHAPE
 * (head_dim, head or token counts, rotary_dim), JPA_ERR_LAYOUT (alignment,
 * strides, overlap, table_stride), JPA_ERR_VALUE (eps, interleaved flag),
 * JPA_ERR_HIP (launch rejected).  T == 0 enqueues nothing and returns JPA_OK.
 */
JPA_API jpa_status jpa_qk_norm_rope(const jpa_tensor* q, const jpa_tensor* k,
                                    const float* q_weight, const float* k_weight,
                                    const float* table, int64_t table_stride,
                                    int32_t rotary_dim, int32_t interleaved, float eps,
                                    const jpa_tensor* q_out, const jpa_tensor* k_out,
                                    void* stream);

#ifdef __cplusplus
}
#endif

#endif
