// Host-only sequence-parallel tail-pad shard plan and segment offsets
// (sglang PR #30107 review, sp_shard_utils: build_shard_plan, the SpShard
// facts, tail_attn_meta; the pad of each rank is its own varlen segment).
#include <cstdint>
#include <limits>

#include "jpa.h"
#include "jpa_shard.h"

extern "C" {

JPA_API jpa_status jpa_shard_plan(int64_t seq_len, int32_t sp_size, int32_t sp_rank, jpa_shard* out) {
    if (!out) return JPA_ERR_NULL;
    if (seq_len < 0 || sp_size < 1 || sp_rank < 0 || sp_rank >= sp_size) return JPA_ERR_VALUE;
    jpa_shard s{};
    s.orig_len = seq_len;
    s.sp_size = sp_size;
    s.sp_rank = sp_rank;
    if (sp_size == 1) {
        s.local_len = seq_len;
        s.local_real_len = seq_len;
        *out = s;
        return JPA_OK;
    }
    s.local_len = seq_len / sp_size + (seq_len % sp_size != 0 ? 1 : 0);
    if (s.local_len > std::numeric_limits<int64_t>::max() / sp_size) return JPA_ERR_VALUE;
    const int64_t total = s.local_len * sp_size;
    s.num_pad = total - seq_len;
    // the chunk [start, end) of this rank against the global pad block [seq_len, total)
    const int64_t start = (int64_t)sp_rank * s.local_len, end = start + s.local_len;
    const int64_t pad_from = start > seq_len ? start : seq_len;
    s.local_pad = end > pad_from ? end - pad_from : 0;
    s.local_real_len = s.local_len - s.local_pad;
    *out = s;
    return JPA_OK;
}

JPA_API jpa_status jpa_tail_attn_meta(const jpa_shard* shard, int32_t seqlen_multiplier,
                                      int32_t* has_tail, int64_t* valid_len, int64_t* max_seqlen_tail) {
    if (!shard || !has_tail || !valid_len || !max_seqlen_tail) return JPA_ERR_NULL;
    if (seqlen_multiplier < 1 || shard->local_real_len < 0) return JPA_ERR_VALUE;
    if (shard->local_real_len > std::numeric_limits<int64_t>::max() / seqlen_multiplier) return JPA_ERR_VALUE;
    *has_tail = shard->num_pad > 0 ? 1 : 0;
    *valid_len = shard->local_real_len * seqlen_multiplier;
    *max_seqlen_tail = *valid_len > shard->num_pad ? *valid_len : shard->num_pad;
    return JPA_OK;
}

JPA_API jpa_status jpa_tail_segments(const jpa_shard* shard, int32_t seqlen_multiplier, int32_t batch,
                                     const int32_t* prefix_lens, int32_t queries_include_prefix,
                                     int32_t* cu_q, int32_t* cu_prefix, int32_t* cu_suffix_real) {
    if (!shard || !cu_q || !cu_prefix || !cu_suffix_real) return JPA_ERR_NULL;
    if (batch < 0 || seqlen_multiplier < 1) return JPA_ERR_VALUE;
    if (queries_include_prefix != 0 && queries_include_prefix != 1) return JPA_ERR_VALUE;
    if (shard->local_len < 0 || shard->local_pad < 0 || shard->local_pad > shard->local_len) return JPA_ERR_VALUE;
    const int64_t lim = std::numeric_limits<int32_t>::max();
    if (shard->local_len > lim / seqlen_multiplier) return JPA_ERR_SEGMENTS;
    const int64_t slots = shard->local_len * seqlen_multiplier;
    const int64_t real = shard->local_real_len * seqlen_multiplier;
    int64_t q = 0, p = 0, s = 0;
    cu_q[0] = 0;
    cu_prefix[0] = 0;
    cu_suffix_real[0] = 0;
    for (int32_t b = 0; b < batch; ++b) {
        const int64_t pl = prefix_lens ? prefix_lens[b] : 0;
        if (pl < 0) return JPA_ERR_VALUE;
        q += slots + (queries_include_prefix ? pl : 0);
        p += pl;
        if (q > lim || p > lim || s + slots > lim) return JPA_ERR_SEGMENTS;
        cu_q[b + 1] = (int32_t)q;
        cu_prefix[b + 1] = (int32_t)p;
        cu_suffix_real[2 * b + 1] = (int32_t)(s + real);
        s += slots;
        cu_suffix_real[2 * b + 2] = (int32_t)s;
    }
    return JPA_OK;
}

}  // extern "C"
