// Host front end of jpa_qk_norm_rope: argument checks (host only, before any
// HIP call) and the launch.
#include <cmath>
#include <cstdint>

#include "jpa.h"
#include "jpa_norm_rope.h"
#include "jpa_norm_rope_params.h"
#include "jpa_views.h"

namespace {

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

jpa_status check_view(const jpa_tensor* t, int64_t tokens, int32_t heads, int32_t head_dim) {
    if (!t) return JPA_ERR_NULL;
    if (t->dtype != JPA_DTYPE_BF16) return JPA_ERR_DTYPE;
    if (t->head_dim != head_dim || t->heads != heads || t->tokens != tokens || heads <= 0) return JPA_ERR_SHAPE;
    if (!t->data && t->tokens > 0) return JPA_ERR_NULL;
    if (!aligned(t->data, 16)) return JPA_ERR_LAYOUT;
    if (t->token_stride % 8 != 0 || t->head_stride % 8 != 0) return JPA_ERR_LAYOUT;
    if (t->head_stride < t->head_dim) return JPA_ERR_LAYOUT;
    if (t->token_stride < (int64_t)t->heads * t->head_stride) return JPA_ERR_LAYOUT;
    return JPA_OK;
}

// Division by an invariant d (1 <= d <= 2^16) for dividends below 2^31:
// with l = ceil(log2 d) and m = ceil(2^(31+l) / d) < 2^32, floor(n / d) =
// (n * m) >> (31 + l) for every such n (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994, theorem 4.2).
void div_magic(int32_t d, uint32_t* magic, int32_t* shift) {
    int l = 0;
    while ((int64_t(1) << l) < d) ++l;
    const uint64_t num = uint64_t(1) << (31 + l);
    *magic = (uint32_t)((num + (uint64_t)d - 1) / (uint64_t)d);
    *shift = 31 + l;
}

}  // namespace

extern "C" {

JPA_API jpa_status jpa_qk_norm_rope(const jpa_tensor* q, const jpa_tensor* k,
                                    const float* q_weight, const float* k_weight,
                                    const float* table, int64_t table_stride,
                                    int32_t rotary_dim, int32_t interleaved, float eps,
                                    const jpa_tensor* q_out, const jpa_tensor* k_out,
                                    void* stream) {
    if (!q || !k || !q_out || !k_out) return JPA_ERR_NULL;
    const int32_t d = q->head_dim;
    if (d != 64 && d != 128 && d != 256) return JPA_ERR_SHAPE;
    jpa_status st;
    if ((st = check_view(q, q->tokens, q->heads, d)) != JPA_OK) return st;
    if ((st = check_view(k, q->tokens, k->heads, d)) != JPA_OK) return st;
    if ((st = check_view(q_out, q->tokens, q->heads, d)) != JPA_OK) return st;
    if ((st = check_view(k_out, q->tokens, k->heads, d)) != JPA_OK) return st;
    if (!q_weight || !k_weight) return JPA_ERR_NULL;
    if (!aligned(q_weight, 16) || !aligned(k_weight, 16)) return JPA_ERR_LAYOUT;
    if (rotary_dim < 0 || rotary_dim > d || rotary_dim % 2 != 0) return JPA_ERR_SHAPE;
    if (interleaved != 0 && interleaved != 1) return JPA_ERR_VALUE;
    if (!std::isfinite(eps) || eps < 0.f) return JPA_ERR_VALUE;
    if (rotary_dim > 0) {
        if (!table && q->tokens > 0) return JPA_ERR_NULL;
        if (!aligned(table, 4)) return JPA_ERR_LAYOUT;
        if (table_stride < rotary_dim) return JPA_ERR_LAYOUT;
    }
    // outputs: each is its own input, or shares no element with any input;
    // the two outputs share none either
    if (!jpa_same_view(q_out, q) && !(jpa_views_disjoint(q_out, q) && jpa_views_disjoint(q_out, k))) return JPA_ERR_LAYOUT;
    if (!jpa_same_view(k_out, k) && !(jpa_views_disjoint(k_out, k) && jpa_views_disjoint(k_out, q))) return JPA_ERR_LAYOUT;
    if (jpa_same_view(q_out, q) && !jpa_views_disjoint(q_out, k)) return JPA_ERR_LAYOUT;
    if (jpa_same_view(k_out, k) && !jpa_views_disjoint(k_out, q)) return JPA_ERR_LAYOUT;
    if (!jpa_views_disjoint(q_out, k_out)) return JPA_ERR_LAYOUT;
    // rows of one tensor and token strides fit the kernel's 32-bit index math
    if (q->heads > 65536 || k->heads > 65536) return JPA_ERR_SHAPE;
    if (q->tokens * q->heads >= (int64_t(1) << 31) || q->tokens * k->heads >= (int64_t(1) << 31))
        return JPA_ERR_SHAPE;
    const jpa_tensor* all[4] = {q, k, q_out, k_out};
    for (const jpa_tensor* t : all)
        if (t->token_stride >= (int64_t(1) << 32)) return JPA_ERR_LAYOUT;

    jpa_norm_rope_params p{};
    const jpa_tensor* in[2] = {q, k};
    const jpa_tensor* out[2] = {q_out, k_out};
    for (int s = 0; s < 2; ++s) {
        p.x[s] = static_cast<const uint16_t*>(in[s]->data);
        p.y[s] = static_cast<uint16_t*>(out[s]->data);
        p.x_ts[s] = in[s]->token_stride;
        p.y_ts[s] = out[s]->token_stride;
        p.x_hs[s] = in[s]->head_stride;
        p.y_hs[s] = out[s]->head_stride;
        p.heads[s] = in[s]->heads;
        div_magic(in[s]->heads, &p.div_magic[s], &p.div_shift[s]);
    }
    p.w[0] = q_weight;
    p.w[1] = k_weight;
    p.table = table;
    p.table_stride = table_stride;
    p.rows_q = q->tokens * q->heads;
    p.rows_total = p.rows_q + q->tokens * k->heads;
    p.rotary_dim = rotary_dim;
    p.interleaved = interleaved;
    p.eps = eps;
    if (p.rows_total == 0) return JPA_OK;
    return jpa_launch_norm_rope(p, d, stream) == 0 ? JPA_OK : JPA_ERR_HIP;
}

}  // extern "C"
