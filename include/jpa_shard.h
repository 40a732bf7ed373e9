/*
 * jpa_shard.h -- host-side sequence-parallel tail-pad shard plan and the
 * attention segment offsets it implies, C ABI (part of libjpa; uses
 * jpa_status from jpa.h).  Integer only; never touches a device.
 *
 *   sglang PR #30107 review, the sp_shard_utils module: a sequence of seq_len
 *   real tokens is split evenly over sp_size ranks (local_len =
 *   ceil(seq_len / sp_size) rows each, num_pad = local_len * sp_size - seq_len
 *   pad rows in all); layout invariant: the gathered sequence is the real
 *   tokens followed by one contiguous pad block at its global tail, so each
 *   rank's chunk is [valid | pad]; tail_attn_meta gives the valid length
 *   (local_real_len times a sequence-length multiplier) and
 *   max_seqlen_tail = max(valid, num_pad); implementation item 4: the pad is
 *   its own varlen segment of the attention call, exactly jpa_forward's
 *   cu_suffix_real form.
 *
 * Reading where the page is at odds with itself: its per-rank property puts
 * all num_pad rows on the last rank, which matches the invariant only while
 * num_pad <= local_len.  Here a rank's pad rows are its chunk's overlap with
 * the global pad block [seq_len, local_len * sp_size), which equals the page's
 * value in that case and stays right otherwise (e.g. seq_len = 1, sp_size = 4:
 * ranks 1..3 each hold one pad row).
 */
#ifndef JPA_SHARD_H
#define JPA_SHARD_H

#include "jpa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct jpa_shard {
    int64_t orig_len;        /* real tokens, global                              */
    int64_t local_len;       /* rows per rank (equal on every rank)             */
    int64_t num_pad;         /* pad rows in all, at the global tail             */
    int32_t sp_size;
    int32_t sp_rank;
    int64_t local_pad;       /* pad rows in this rank's chunk (its tail)        */
    int64_t local_real_len;  /* real rows in this rank's chunk                  */
} jpa_shard;

/*
 * jpa_shard_plan -- the shard facts of rank sp_rank for seq_len tokens over
 * sp_size ranks.  sp_size == 1: no pad, local_len = seq_len.
 * Errors: JPA_ERR_NULL (out), JPA_ERR_VALUE (seq_len < 0, sp_size < 1,
 * sp_rank outside [0, sp_size), local_len * sp_size beyond int64).
 */
JPA_API jpa_status jpa_shard_plan(int64_t seq_len, int32_t sp_size, int32_t sp_rank, jpa_shard* out);

/*
 * jpa_tail_attn_meta -- *valid_len = local_real_len * seqlen_multiplier and
 * *max_seqlen_tail = max(valid_len, num_pad); *has_tail = (num_pad > 0) (the
 * page returns no metadata then).  Pointers may not be NULL.
 * Errors: JPA_ERR_NULL, JPA_ERR_VALUE (seqlen_multiplier < 1, overflow).
 */
JPA_API jpa_status jpa_tail_attn_meta(const jpa_shard* shard, int32_t seqlen_multiplier,
                                      int32_t* has_tail, int64_t* valid_len, int64_t* max_seqlen_tail);

/*
 * jpa_tail_segments -- the host offsets of one rank's jpa_forward call: batch
 * row b has prefix_lens[b] prefix tokens (prefix_lens may be NULL: no prefix)
 * and a suffix of local_len * m slots whose last local_pad * m are pad
 * (m = seqlen_multiplier); its query slots are its suffix slots, preceded by
 * its prefix tokens when queries_include_prefix is 1.  Writes (caller arrays)
 *   cu_q[batch + 1], cu_prefix[batch + 1], cu_suffix_real[2 * batch + 1]
 * in jpa_forward's encoding.
 * Errors: JPA_ERR_NULL (shard or an output), JPA_ERR_VALUE (batch < 0, m < 1,
 * queries_include_prefix not 0/1, a negative prefix length), JPA_ERR_SEGMENTS
 * (an offset beyond int32).
 */
JPA_API jpa_status jpa_tail_segments(const jpa_shard* shard, int32_t seqlen_multiplier, int32_t batch,
                                     const int32_t* prefix_lens, int32_t queries_include_prefix,
                                     int32_t* cu_q, int32_t* cu_prefix, int32_t* cu_suffix_real);

#ifdef __cplusplus
}
#endif

#endif
