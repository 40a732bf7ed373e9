// Element extents of jpa_tensor views and overlap tests between them, shared
// by the host front ends (host only; addresses are compared, never read).
#ifndef JPA_VIEWS_H
#define JPA_VIEWS_H

#include <stdint.h>

#include "jpa.h"

// Span of one token's row of heads, and of the whole view, in bf16 elements:
// the view lies in [data, data + span).
inline int64_t jpa_row_span(const jpa_tensor* t) {
    return (int64_t)(t->heads - 1) * t->head_stride + t->head_dim;
}
inline int64_t jpa_view_span(const jpa_tensor* t) {
    return t->tokens == 0 ? 0 : (t->tokens - 1) * t->token_stride + jpa_row_span(t);
}

inline bool jpa_same_view(const jpa_tensor* a, const jpa_tensor* b) {
    return a->data == b->data && a->tokens == b->tokens && a->heads == b->heads &&
           a->token_stride == b->token_stride && a->head_stride == b->head_stride &&
           a->head_dim == b->head_dim;
}

// True when no element of a is an element of b.  Views of one buffer with the
// same token stride (e.g. the q, k and v slices of a fused QKV tensor) are
// disjoint when their per-token column windows do not meet; other views must
// not share any address range.
inline bool jpa_views_disjoint(const jpa_tensor* a, const jpa_tensor* b) {
    if (a->tokens == 0 || b->tokens == 0) return true;
    const intptr_t pa = reinterpret_cast<intptr_t>(a->data), pb = reinterpret_cast<intptr_t>(b->data);
    const intptr_t ea = pa + 2 * jpa_view_span(a), eb = pb + 2 * jpa_view_span(b);
    if (ea <= pb || eb <= pa) return true;
    if (a->token_stride != b->token_stride) return false;
    if ((pb - pa) % 2 != 0) return false;
    const int64_t ts = a->token_stride;
    int64_t d = ((pb - pa) / 2) % ts;          // b's window starts d columns into a's token row
    if (d < 0) d += ts;
    // windows [0, wa) and [d, d + wb) modulo ts must not intersect
    return jpa_row_span(a) <= d && d + jpa_row_span(b) <= ts;
}

// True when the byte range [p, p + nbytes) shares no byte with view t.
inline bool jpa_bytes_disjoint(const void* p, int64_t nbytes, const jpa_tensor* t) {
    if (nbytes <= 0 || t->tokens == 0) return true;
    const intptr_t a = reinterpret_cast<intptr_t>(p), ta = reinterpret_cast<intptr_t>(t->data);
    return a + nbytes <= ta || ta + 2 * jpa_view_span(t) <= a;
}

#endif
