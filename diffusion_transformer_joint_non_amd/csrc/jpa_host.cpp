// Host front end of libjpa: argument validation, segment decoding, launch
// planning.  Everything here runs on the host and never reads device memory
// (varlen metadata is host-side, so a call needs no device readback: vLLM-Omni
// performance-patterns guide, section on removing per-layer syncs).
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#include <algorithm>

#include "jpa.h"
#include "jpa_params.h"
#include "jpa_scratch.h"
#include "jpa_views.h"

namespace {

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

jpa_status check_offsets(const int32_t* cu, int32_t n) {
    if (cu[0] != 0) return JPA_ERR_SEGMENTS;
    for (int32_t i = 0; i + 1 < n; ++i)
        if (cu[i + 1] < cu[i]) return JPA_ERR_SEGMENTS;
    return JPA_OK;
}

// Decode row b (the pad of a row is segment 2b+1 of cu_suffix_real: sglang PR
// #30107 review, implementation breakdown item 4).
jpa_row_plan decode_row(int32_t b, const int32_t* cu_q, const int32_t* cu_prefix,
                        const int32_t* cu_suffix_real) {
    jpa_row_plan r;
    r.q_start = cu_q[b];
    r.q_slots = cu_q[b + 1] - cu_q[b];
    r.prefix_start = cu_prefix[b];
    r.prefix_len = cu_prefix[b + 1] - cu_prefix[b];
    r.suffix_start = cu_suffix_real[2 * b];
    r.suffix_real = cu_suffix_real[2 * b + 1] - cu_suffix_real[2 * b];
    r.suffix_pad = cu_suffix_real[2 * b + 2] - cu_suffix_real[2 * b + 1];
    r.q_real = r.q_slots - r.suffix_pad;
    r.keys = r.prefix_len + r.suffix_real;
    return r;
}

jpa_status check_segments(int32_t batch, const int32_t* cu_q, const int32_t* cu_prefix,
                          const int32_t* cu_suffix_real) {
    if (batch < 0) return JPA_ERR_VALUE;
    if (!cu_q || !cu_prefix || !cu_suffix_real) return JPA_ERR_NULL;
    jpa_status st;
    if ((st = check_offsets(cu_q, batch + 1)) != JPA_OK) return st;
    if ((st = check_offsets(cu_prefix, batch + 1)) != JPA_OK) return st;
    if ((st = check_offsets(cu_suffix_real, 2 * batch + 1)) != JPA_OK) return st;
    for (int32_t b = 0; b < batch; ++b) {
        const jpa_row_plan r = decode_row(b, cu_q, cu_prefix, cu_suffix_real);
        if (r.suffix_pad > r.q_slots) return JPA_ERR_SEGMENTS;
        // int32 sum: both terms are differences of non-decreasing int32 offsets
        if ((int64_t)r.prefix_len + r.suffix_real > INT32_MAX) return JPA_ERR_SEGMENTS;
        if (r.q_real > 0 && (int64_t)r.prefix_len + r.suffix_real == 0) return JPA_ERR_SEGMENTS;
    }
    return JPA_OK;
}

// K/V rows are addressed as a 32-bit multiple of the token stride in bytes
// computed with a 24-bit multiply: token strides must stay below 2^23 elements.
constexpr int64_t kMaxKvTokenStride = int64_t(1) << 23;

jpa_status check_tensor(const jpa_tensor* t, int64_t tokens, int32_t heads, int32_t head_dim,
                        bool kv = false) {
    if (!t) return JPA_ERR_NULL;
    if (t->dtype != JPA_DTYPE_BF16) return JPA_ERR_DTYPE;
    if (t->head_dim != head_dim || t->heads != heads || t->tokens != tokens) return JPA_ERR_SHAPE;
    if (!t->data && t->tokens > 0) return JPA_ERR_NULL;
    if (!aligned16(t->data)) return JPA_ERR_LAYOUT;
    if (t->token_stride % 8 != 0 || t->head_stride % 8 != 0) return JPA_ERR_LAYOUT;
    if (t->head_stride < t->head_dim) return JPA_ERR_LAYOUT;
    if (t->token_stride < (int64_t)t->heads * t->head_stride) return JPA_ERR_LAYOUT;
    if (kv && t->token_stride >= kMaxKvTokenStride) return JPA_ERR_LAYOUT;
    return JPA_OK;
}

jpa_status validate(const jpa_tensor* q, const jpa_tensor* k_prefix, const jpa_tensor* v_prefix,
                    const jpa_tensor* k_suffix, const jpa_tensor* v_suffix, int32_t batch,
                    const int32_t* cu_q, const int32_t* cu_prefix, const int32_t* cu_suffix_real,
                    float scale, const jpa_tensor* out, const float* lse) {
    if (!q || !k_prefix || !v_prefix || !k_suffix || !v_suffix || !out) return JPA_ERR_NULL;
    if (!std::isfinite(scale) || scale < 0.f) return JPA_ERR_VALUE;
    jpa_status st = check_segments(batch, cu_q, cu_prefix, cu_suffix_real);
    if (st != JPA_OK) return st;
    const int32_t d = q->head_dim;
    if (d != 64 && d != 128) return JPA_ERR_SHAPE;
    const int32_t hq = q->heads, hkv = k_prefix->heads;
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return JPA_ERR_SHAPE;
    const int64_t tq = cu_q[batch], tp = cu_prefix[batch], ts = cu_suffix_real[2 * batch];
    if ((st = check_tensor(q, tq, hq, d)) != JPA_OK) return st;
    if ((st = check_tensor(out, tq, hq, d)) != JPA_OK) return st;
    if ((st = check_tensor(k_prefix, tp, hkv, d, true)) != JPA_OK) return st;
    if ((st = check_tensor(v_prefix, tp, hkv, d, true)) != JPA_OK) return st;
    if ((st = check_tensor(k_suffix, ts, hkv, d, true)) != JPA_OK) return st;
    if ((st = check_tensor(v_suffix, ts, hkv, d, true)) != JPA_OK) return st;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return JPA_ERR_LAYOUT;
    // Outputs share no element with the keys and values (other workgroups keep
    // reading every key while rows are written) nor with each other.  out may
    // be q itself, the same view: a workgroup reads only its own query rows,
    // all of them before it writes any, and a row cut between workgroups is
    // written by the merge launch after every piece is done.
    const jpa_tensor* kv[4] = {k_prefix, v_prefix, k_suffix, v_suffix};
    for (const jpa_tensor* t : kv)
        if (!jpa_views_disjoint(out, t)) return JPA_ERR_LAYOUT;
    if (!jpa_same_view(out, q) && !jpa_views_disjoint(out, q)) return JPA_ERR_LAYOUT;
    if (lse) {
        const int64_t lse_bytes = 4 * (int64_t)hq * tq;
        const jpa_tensor* all[6] = {q, k_prefix, v_prefix, k_suffix, v_suffix, out};
        for (const jpa_tensor* t : all)
            if (!jpa_bytes_disjoint(lse, lse_bytes, t)) return JPA_ERR_LAYOUT;
    }
    return JPA_OK;
}

// Compute units of the current device.
jpa_status device_cus(int* cus) {
    *cus = jpa_device_cus();
    return *cus > 0 ? JPA_OK : JPA_ERR_HIP;
}

// Work split of one launch over `wgs` compute units (0: one workgroup per
// item).  Items are (query head, query tile); a real item weighs its key
// tiles, an all-pad item 1.  Whole rounds of wgs items run one item per
// workgroup; the items of the last, partial round are cut into wgs balanced
// ranges of key tiles, whose cut items a second kernel merges.
constexpr int kMinTilesPerRange = 8;

void plan_split(jpa_kernel_params& p, int wgs, bool forced, char* ws, int head_dim) {
    const int64_t items = (int64_t)p.total_tiles * p.hq;
    int64_t head_units = 0;
    std::vector<int64_t> tile_units(p.total_tiles);
    for (int b = 0; b < p.nrows; ++b) {
        const jpa_kernel_row& r = p.rows[b];
        const int nt = (r.q_slots + JPA_BLOCK_M - 1) / JPA_BLOCK_M;
        const int nr = (r.q_real + JPA_BLOCK_M - 1) / JPA_BLOCK_M;
        const int nk = (r.keys + 63) / 64;
        for (int t = 0; t < nt; ++t) tile_units[r.tile_start + t] = t < nr ? nk : 1;
        head_units += (int64_t)nr * nk + (nt - nr);
    }
    p.head_units = head_units;
    p.n_dp = (int32_t)items;
    p.sk_wgs = 0;
    p.tail_unit0 = p.tail_units = 0;
    p.ws_o = nullptr;
    p.ws_lse = nullptr;
    if (wgs <= 0 || items % wgs == 0) return;
    // Unless asked for, split only when the last round would leave more than
    // half of the units idle: cut pieces each pay a prologue and a merge, so a
    // nearly full last round is faster uncut.
    if (!forced && 2 * (items % wgs) > wgs) return;
    const int64_t n_dp = items / wgs * wgs;
    int64_t unit0 = 0, tail = 0;
    for (int64_t it = 0; it < items; ++it) {
        const int64_t u = tile_units[it % p.total_tiles];
        if (it < n_dp) unit0 += u; else tail += u;
    }
    // ... and only when every range gets enough key tiles to amortise its
    // pieces' prologues and the merge launch (tiny problems stay uncut)
    if (!forced && tail < (int64_t)kMinTilesPerRange * wgs) return;
    p.n_dp = (int32_t)n_dp;
    p.sk_wgs = (int32_t)std::min<int64_t>(wgs, tail);
    p.tail_unit0 = unit0;
    p.tail_units = tail;
    p.ws_o = reinterpret_cast<float*>(ws);
    p.ws_lse = reinterpret_cast<float*>(ws + jpa_ws_o_bytes(wgs, head_dim));
}

jpa_status enqueue(const jpa_tensor* q, const jpa_tensor* k_prefix, const jpa_tensor* v_prefix,
                   const jpa_tensor* k_suffix, const jpa_tensor* v_suffix, int32_t batch,
                   const int32_t* cu_q, const int32_t* cu_prefix, const int32_t* cu_suffix_real,
                   float scale, const jpa_tensor* out, float* lse, void* workspace, int wgs,
                   bool forced, void* stream);

}  // namespace

extern "C" {

JPA_API jpa_status jpa_validate(const jpa_tensor* q, const jpa_tensor* k_prefix,
                                const jpa_tensor* v_prefix, const jpa_tensor* k_suffix,
                                const jpa_tensor* v_suffix, int32_t batch, const int32_t* cu_q,
                                const int32_t* cu_prefix, const int32_t* cu_suffix_real,
                                float scale, const jpa_tensor* out, const float* lse) {
    return validate(q, k_prefix, v_prefix, k_suffix, v_suffix, batch, cu_q, cu_prefix,
                    cu_suffix_real, scale, out, lse);
}

JPA_API jpa_status jpa_plan(int32_t batch, const int32_t* cu_q, const int32_t* cu_prefix,
                            const int32_t* cu_suffix_real, int32_t heads_q, int32_t head_dim,
                            jpa_row_plan* rows, int64_t* valid_flops) {
    jpa_status st = check_segments(batch, cu_q, cu_prefix, cu_suffix_real);
    if (st != JPA_OK) return st;
    if (heads_q < 0 || head_dim < 0) return JPA_ERR_VALUE;
    int64_t flops = 0;
    for (int32_t b = 0; b < batch; ++b) {
        const jpa_row_plan r = decode_row(b, cu_q, cu_prefix, cu_suffix_real);
        if (rows) rows[b] = r;
        flops += (int64_t)heads_q * 4 * head_dim * (int64_t)r.q_real * (int64_t)r.keys;
    }
    if (valid_flops) *valid_flops = flops;
    return JPA_OK;
}

JPA_API size_t jpa_workspace_bytes(int32_t head_dim, int32_t split_wgs) {
    if (head_dim != 64 && head_dim != 128) return 0;
    int wgs = split_wgs;
    if (wgs <= 0 && device_cus(&wgs) != JPA_OK) return 0;
    return jpa_ws_o_bytes(wgs, head_dim) + jpa_ws_lse_bytes(wgs);
}

JPA_API jpa_status jpa_forward(const jpa_tensor* q, const jpa_tensor* k_prefix,
                               const jpa_tensor* v_prefix, const jpa_tensor* k_suffix,
                               const jpa_tensor* v_suffix, int32_t batch, const int32_t* cu_q,
                               const int32_t* cu_prefix, const int32_t* cu_suffix_real,
                               float scale, const jpa_tensor* out, float* lse, void* stream) {
    return jpa_forward_ws(q, k_prefix, v_prefix, k_suffix, v_suffix, batch, cu_q, cu_prefix,
                          cu_suffix_real, scale, out, lse, nullptr, 0, 0, stream);
}

JPA_API jpa_status jpa_forward_ws(const jpa_tensor* q, const jpa_tensor* k_prefix,
                                  const jpa_tensor* v_prefix, const jpa_tensor* k_suffix,
                                  const jpa_tensor* v_suffix, int32_t batch, const int32_t* cu_q,
                                  const int32_t* cu_prefix, const int32_t* cu_suffix_real,
                                  float scale, const jpa_tensor* out, float* lse,
                                  void* workspace, size_t workspace_bytes, int32_t split_wgs,
                                  void* stream) {
    jpa_status st = validate(q, k_prefix, v_prefix, k_suffix, v_suffix, batch, cu_q, cu_prefix,
                             cu_suffix_real, scale, out, lse);
    if (st != JPA_OK) return st;
    int wgs = 0;
    if (workspace) {
        if (split_wgs < 0) return JPA_ERR_VALUE;
        if (reinterpret_cast<uintptr_t>(workspace) & 255u) return JPA_ERR_LAYOUT;
        wgs = split_wgs;
        if (wgs == 0 && device_cus(&wgs) != JPA_OK) return JPA_ERR_HIP;
        if (workspace_bytes < jpa_ws_o_bytes(wgs, q->head_dim) + jpa_ws_lse_bytes(wgs))
            return JPA_ERR_VALUE;
    }
    return enqueue(q, k_prefix, v_prefix, k_suffix, v_suffix, batch, cu_q, cu_prefix,
                   cu_suffix_real, scale, out, lse, workspace, wgs, split_wgs > 0, stream);
}

JPA_API jpa_status jpa_forward_scratch(const jpa_tensor* q, const jpa_tensor* k_prefix,
                                       const jpa_tensor* v_prefix, const jpa_tensor* k_suffix,
                                       const jpa_tensor* v_suffix, int32_t batch,
                                       const int32_t* cu_q, const int32_t* cu_prefix,
                                       const int32_t* cu_suffix_real, float scale,
                                       const jpa_tensor* out, float* lse, int32_t split_wgs,
                                       void* stream) {
    jpa_status st = validate(q, k_prefix, v_prefix, k_suffix, v_suffix, batch, cu_q, cu_prefix,
                             cu_suffix_real, scale, out, lse);
    if (st != JPA_OK) return st;
    if (split_wgs < 0) return JPA_ERR_VALUE;
    if (split_wgs > JPA_SCRATCH_MAX_WGS) return JPA_ERR_SCRATCH;
    int wgs = split_wgs;
    if (wgs == 0 && device_cus(&wgs) != JPA_OK) return JPA_ERR_HIP;
    if (wgs > JPA_SCRATCH_MAX_WGS) return JPA_ERR_SCRATCH;
    // the scratch of JPA_SCRATCH_MAX_WGS ranges at head_dim 128 holds any
    // smaller request
    if (jpa_ws_o_bytes(wgs, q->head_dim) + jpa_ws_lse_bytes(wgs) > jpa_scratch_bytes())
        return JPA_ERR_SCRATCH;
    void* ws = nullptr;
    if (jpa_scratch_address(&ws) != 0) return JPA_ERR_HIP;
    return enqueue(q, k_prefix, v_prefix, k_suffix, v_suffix, batch, cu_q, cu_prefix,
                   cu_suffix_real, scale, out, lse, ws, wgs, split_wgs > 0, stream);
}

}  // extern "C"

namespace {

// The launches of one validated forward call: one per JPA_MAX_ROWS batch
// rows, the last round of work items cut over `wgs` key ranges through the
// workspace `ws` when the split rule (or `forced`) says so.
jpa_status enqueue(const jpa_tensor* q, const jpa_tensor* k_prefix, const jpa_tensor* v_prefix,
                   const jpa_tensor* k_suffix, const jpa_tensor* v_suffix, int32_t batch,
                   const int32_t* cu_q, const int32_t* cu_prefix, const int32_t* cu_suffix_real,
                   float scale, const jpa_tensor* out, float* lse, void* workspace, int wgs,
                   bool forced, void* stream) {
    jpa_kernel_params p;
    std::memset(&p, 0, sizeof(p));
    p.q = static_cast<const uint16_t*>(q->data);
    p.kp = static_cast<const uint16_t*>(k_prefix->data);
    p.vp = static_cast<const uint16_t*>(v_prefix->data);
    p.ks = static_cast<const uint16_t*>(k_suffix->data);
    p.vs = static_cast<const uint16_t*>(v_suffix->data);
    p.out = static_cast<uint16_t*>(out->data);
    p.lse = lse;
    p.q_ts = q->token_stride;
    p.kp_ts = k_prefix->token_stride;
    p.vp_ts = v_prefix->token_stride;
    p.ks_ts = k_suffix->token_stride;
    p.vs_ts = v_suffix->token_stride;
    p.o_ts = out->token_stride;
    p.q_hs = q->head_stride;
    p.kp_hs = k_prefix->head_stride;
    p.vp_hs = v_prefix->head_stride;
    p.ks_hs = k_suffix->head_stride;
    p.vs_hs = v_suffix->head_stride;
    p.o_hs = out->head_stride;
    p.lse_ld = cu_q[batch];
    p.hq = q->heads;
    p.group = q->heads / k_prefix->heads;
    // Softmax in base 2: the kernel scales scores by c = scale * log2(e).  c is
    // kept >= 1e-30 so that masked scores (-FLT_MAX) still map to zero weight;
    // below that the weights are uniform to fp32 precision anyway.
    p.c = std::fmax(scale * 1.4426950408889634f, 1e-30f);

    // One launch per JPA_MAX_ROWS batch rows; rows with no query slots are
    // dropped from the plan.
    int32_t b = 0;
    while (b < batch) {
        p.nrows = 0;
        p.total_tiles = 0;
        for (; b < batch && p.nrows < JPA_MAX_ROWS; ++b) {
            const jpa_row_plan r = decode_row(b, cu_q, cu_prefix, cu_suffix_real);
            if (r.q_slots == 0) continue;
            jpa_kernel_row& kr = p.rows[p.nrows++];
            kr.q_start = r.q_start;
            kr.q_slots = r.q_slots;
            kr.q_real = r.q_real;
            kr.p_start = r.prefix_start;
            kr.p_len = r.prefix_len;
            kr.s_start = r.suffix_start;
            kr.keys = r.keys;
            kr.tile_start = p.total_tiles;
            p.total_tiles += (r.q_slots + JPA_BLOCK_M - 1) / JPA_BLOCK_M;
        }
        if (p.nrows == 0) continue;
        if ((int64_t)p.total_tiles * p.hq > INT32_MAX) return JPA_ERR_SHAPE;
        plan_split(p, workspace ? wgs : 0, forced, static_cast<char*>(workspace), q->head_dim);
        if (jpa_launch_kernel(p, q->head_dim, stream) != 0) return JPA_ERR_HIP;
    }
    return JPA_OK;
}

}  // namespace

extern "C" {

JPA_API const char* jpa_status_str(jpa_status status) {
    switch (status) {
        case JPA_OK: return "JPA_OK";
        case JPA_ERR_NULL: return "JPA_ERR_NULL: a required pointer is NULL";
        case JPA_ERR_DTYPE: return "JPA_ERR_DTYPE: tensors must be bf16";
        case JPA_ERR_SHAPE: return "JPA_ERR_SHAPE: inconsistent heads, head_dim or token extents";
        case JPA_ERR_LAYOUT: return "JPA_ERR_LAYOUT: misaligned pointer or stride, or overlapping rows";
        case JPA_ERR_SEGMENTS: return "JPA_ERR_SEGMENTS: invalid segment offsets";
        case JPA_ERR_VALUE: return "JPA_ERR_VALUE: scale must be finite and >= 0, batch >= 0";
        case JPA_ERR_HIP: return "JPA_ERR_HIP: the HIP runtime rejected the launch";
        case JPA_ERR_SCRATCH:
            return "JPA_ERR_SCRATCH: more key ranges than the static scratch holds (JPA_SCRATCH_MAX_WGS)";
    }
    return "JPA_ERR_UNKNOWN";
}

JPA_API int32_t jpa_abi_version(void) { return JPA_ABI_VERSION; }

}  // extern "C"
