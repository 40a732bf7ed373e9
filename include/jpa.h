/*
 * jpa.h -- joint prefix/suffix attention for diffusion transformers, C ABI.
 *
 * One operation: the bidirectional (non-causal) attention forward of a DiT
 * block whose keys/values arrive as two separate tensors that are never
 * concatenated -- a prefix (text or conditioning tokens) and a suffix (image
 * or video tokens) -- and whose suffix ends, per batch row, with a block of
 * tail-pad slots that is treated as a segment of its own and skipped.
 *
 *   sglang PR #26973 review, core-logic snippet of the attention layer:
 *     forward_with_replicated_kv_prefix(q, k_prefix, v_prefix, k_suffix,
 *     v_suffix); without sequence parallelism it is attention over the
 *     sequence-axis concatenation [prefix, suffix] (prefix first).
 *   sglang PR #30107 review, implementation breakdown item 4 and the
 *     sp_shard_utils layout-invariant docstring: every batch row is laid out
 *     as [valid | pad]; the pad is its own varlen segment, so there is no
 *     repacking and no mask compute.
 *   vLLM-Omni performance-patterns guide, shared attention wiring: non-causal,
 *     BSND layout, softmax scale head_dim**-0.5 (taken here as an argument);
 *     USP section: Q heads must be a multiple of KV heads; section on removing
 *     per-layer syncs: varlen metadata lives on the host, so a call never
 *     reads the device back.
 *
 * Definition.  For batch row b, query head h (kv head h / (Hq/Hkv)) and real
 * query slot i of that row:
 *     K_b = [k_prefix rows of b ; real k_suffix rows of b]   (pad rows excluded)
 *     s_ij = scale * <q_i, k_j>,  LSE_i = ln sum_j exp(s_ij)
 *     out_i = sum_j exp(s_ij - LSE_i) v_j
 * Pad query slots get out = +0.0 and LSE = -inf.
 *
 * Threading / ownership: the library allocates nothing; the only state it
 * keeps between calls is a per-device cache of the compute-unit count, filled
 * on first use and read atomically, so calls from several host threads are
 * safe.  The caller
 * owns every buffer and the stream.  Every entry point validates all its
 * arguments on the host before touching the device; none throws or aborts
 * across the ABI.  All functions return a jpa_status.
 */
#ifndef JPA_H
#define JPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define JPA_API __attribute__((visibility("default")))
#else
#define JPA_API
#endif

#define JPA_ABI_VERSION 1

typedef enum jpa_status {
    JPA_OK = 0,
    JPA_ERR_NULL = 1,      /* a required pointer is NULL                          */
    JPA_ERR_DTYPE = 2,     /* tensor dtype is not JPA_DTYPE_BF16                  */
    JPA_ERR_SHAPE = 3,     /* head_dim not 64/128, Hq % Hkv != 0, head counts or
                              token extents inconsistent with each other or with
                              the segment offsets                                 */
    JPA_ERR_LAYOUT = 4,    /* misaligned pointer/stride, or an output overlapping
                              an input or the other output                        */
    JPA_ERR_SEGMENTS = 5,  /* bad offsets: cu[0] != 0, decreasing, pad_b > Lq_b,
                              or real queries with no keys                        */
    JPA_ERR_VALUE = 6,     /* scale not finite or negative; batch < 0             */
    JPA_ERR_HIP = 7,       /* the HIP runtime rejected the launch (no device,
                              no gfx950 code object, bad stream, ...)             */
    JPA_ERR_SCRATCH = 8    /* jpa_forward_scratch: more key ranges than its
                              static scratch holds (JPA_SCRATCH_MAX_WGS)          */
} jpa_status;

typedef enum jpa_dtype {
    JPA_DTYPE_BF16 = 1
} jpa_dtype;

/*
 * A packed token-major tensor [tokens, heads, head_dim] (BSND with the batch
 * folded into the token axis).  Element (t, h, d) lives at
 *     ((uint16_t*)data) + t * token_stride + h * head_stride + d
 * (strides in elements; head_dim is contiguous).  Views are allowed: e.g. V
 * as a token-strided slice of a fused QKV projection output (sglang PR
 * #26973 review, Cosmos3 cross-attention snippet).
 * Requirements: data 16-byte aligned; token_stride and head_stride multiples
 * of 8; head_stride >= head_dim; token_stride >= heads * head_stride; for the
 * four K/V tensors token_stride < 2^23 (8 Mi elements per token).
 * data may be NULL only when tokens == 0.
 */
typedef struct jpa_tensor {
    void*   data;          /* device address (host address for jpa_validate) */
    int64_t tokens;
    int64_t token_stride;
    int32_t heads;
    int32_t head_stride;
    int32_t head_dim;
    int32_t dtype;         /* jpa_dtype */
} jpa_tensor;

/*
 * Per-row bookkeeping decoded from the offsets (all token counts).
 */
typedef struct jpa_row_plan {
    int32_t q_start;       /* first query slot of the row                       */
    int32_t q_slots;       /* Lq_b: query slots, pad slots included             */
    int32_t q_real;        /* Nq_b = Lq_b - pad_b                               */
    int32_t prefix_start;  /* first k_prefix/v_prefix token of the row          */
    int32_t prefix_len;    /* P_b                                               */
    int32_t suffix_start;  /* first k_suffix/v_suffix slot of the row           */
    int32_t suffix_real;   /* R_b                                               */
    int32_t suffix_pad;    /* pad_b                                             */
    int32_t keys;          /* Nk_b = P_b + R_b                                  */
} jpa_row_plan;

/*
 * Segment offsets (HOST int32 arrays, read during the call only):
 *   cu_q           batch+1 entries: row b owns query slots [cu_q[b], cu_q[b+1])
 *   cu_prefix      batch+1 entries: row b owns prefix tokens [cu_prefix[b], cu_prefix[b+1])
 *   cu_suffix_real 2*batch+1 entries, alternating boundaries
 *                  [s_0, s_0+R_0, s_1, s_1+R_1, ..., end]: segment 2b is row b's
 *                  real suffix, segment 2b+1 its tail pad (pad_b slots); the pad
 *                  slots are never read.
 * The last pad_b query slots of row b are its pad rows (queries end with the
 * row's suffix slots); they are never read and get out = 0, LSE = -inf.
 *
 * The offsets are taken as host arrays only; no device copy is passed or
 * needed.  This follows the vLLM-Omni performance-patterns guide, section on
 * removing per-layer syncs: varlen metadata is built once on the host, so the
 * forward never reads anything back from the device.  The host decodes each
 * row's lengths and passes them to the kernel inside its launch arguments.
 */

/*
 * jpa_forward -- enqueue the attention forward on `stream` and return.
 *
 *   q         [Tq, Hq, D]  bf16, Tq = cu_q[batch]
 *   k_prefix  [Tp, Hkv, D] bf16, Tp = cu_prefix[batch]; v_prefix likewise
 *   k_suffix  [Ts, Hkv, D] bf16, Ts = cu_suffix_real[2*batch]; v_suffix likewise
 *   scale     softmax scale (finite, >= 0; head_dim**-0.5 in every DiT above);
 *             scale*log2(e) below 1e-30 is treated as 1e-30 (uniform weights)
 *   out       [Tq, Hq, D]  bf16, written entirely (pad rows as +0.0), rounded
 *             to nearest even; shares no element with k_prefix, v_prefix,
 *             k_suffix or v_suffix, and either is q itself (the same view:
 *             in place) or shares no element with q (JPA_ERR_LAYOUT)
 *   lse       fp32 [Hq, Tq] (element (h, t) at lse[h*Tq + t]), natural log of
 *             the softmax denominator, -inf on pad rows; may be NULL; shares
 *             no byte with any tensor argument (JPA_ERR_LAYOUT)
 *   stream    a hipStream_t (NULL = the default stream)
 * D is 64 or 128; Hq % Hkv == 0.  The call is asynchronous: it validates the
 * arguments on the host, enqueues one or more kernel launches (one per 32
 * batch rows) and returns without synchronising or reading device memory.
 * On any error nothing is enqueued and a status other than JPA_OK is returned
 * (JPA_ERR_HIP if the runtime rejects a launch; batches already enqueued by
 * that call are not undone).
 */
JPA_API jpa_status jpa_forward(const jpa_tensor* q,
                               const jpa_tensor* k_prefix, const jpa_tensor* v_prefix,
                               const jpa_tensor* k_suffix, const jpa_tensor* v_suffix,
                               int32_t batch,
                               const int32_t* cu_q, const int32_t* cu_prefix,
                               const int32_t* cu_suffix_real,
                               float scale,
                               const jpa_tensor* out, float* lse,
                               void* stream);

/*
 * jpa_forward_ws -- jpa_forward with a workspace that lets the last, partial
 * round of work items be balanced over every compute unit.
 *
 * Work items are (query head, 256-query tile).  When their number is not a
 * multiple of the compute-unit count, the last round would leave units idle;
 * with a workspace, the key tiles of that round's items are cut into
 * split_wgs equal ranges, one per workgroup, and every item cut between
 * ranges is merged from per-piece
 * partial results by a second kernel (the standard log-sum-exp merge of
 * softmax partials, in a fixed order, so results do not depend on timing).
 * The attention computed is the same as jpa_forward's; values may differ from
 * it by rounding only.
 *
 *   workspace        device memory of at least jpa_workspace_bytes(head_dim,
 *                    split_wgs) bytes, 256-byte aligned, or NULL (then this is
 *                    jpa_forward).  No contents are needed between calls; the
 *                    pieces' partial results pass through it to a second
 *                    kernel enqueued on the same stream, so calls that may run
 *                    at the same time need distinct workspaces.
 *   workspace_bytes  its size; a smaller size than required is JPA_ERR_VALUE.
 *   split_wgs        0: ranges = compute units, and the last round is cut
 *                    only when it would leave more than half of them idle
 *                    and every range gets at least 8 key tiles (each cut
 *                    piece pays a prologue and a merge); > 0: that
 *                    many ranges, always cut (a tuning and testing knob).
 * Errors as jpa_forward, plus JPA_ERR_LAYOUT for a misaligned workspace and
 * JPA_ERR_HIP when the device cannot be queried.
 */
JPA_API jpa_status jpa_forward_ws(const jpa_tensor* q,
                                  const jpa_tensor* k_prefix, const jpa_tensor* v_prefix,
                                  const jpa_tensor* k_suffix, const jpa_tensor* v_suffix,
                                  int32_t batch,
                                  const int32_t* cu_q, const int32_t* cu_prefix,
                                  const int32_t* cu_suffix_real,
                                  float scale,
                                  const jpa_tensor* out, float* lse,
                                  void* workspace, size_t workspace_bytes, int32_t split_wgs,
                                  void* stream);

/*
 * jpa_forward_scratch -- jpa_forward_ws for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same launches, with the cut items' partial
 * results in a static device array of the library instead of a caller
 * workspace.  No allocation of any kind is made by this call.
 *
 *   split_wgs  as in jpa_forward_ws (0: the device's compute units, cut only
 *              when the split rule says so; > 0: that many ranges, always
 *              cut); at most JPA_SCRATCH_MAX_WGS.
 * The array holds the workspace of JPA_SCRATCH_MAX_WGS ranges at head_dim 128
 * (64.5 MiB); every device the library runs on keeps its own copy until the
 * process ends.  Nothing in it needs to start at zero.  All calls on one
 * device share it, so two calls that may run at the same time on one device
 * (different streams without ordering between them) race and corrupt each
 * other's results; calls on one stream are ordered and safe.  Results equal
 * jpa_forward_ws's with the same split_wgs, bit for bit.
 * Errors as jpa_forward_ws, plus JPA_ERR_SCRATCH when split_wgs (or, for 0,
 * the device's compute units) exceeds JPA_SCRATCH_MAX_WGS; JPA_ERR_HIP when
 * the device or the array's address cannot be queried.
 */
#define JPA_SCRATCH_MAX_WGS 256
JPA_API jpa_status jpa_forward_scratch(const jpa_tensor* q,
                                       const jpa_tensor* k_prefix, const jpa_tensor* v_prefix,
                                       const jpa_tensor* k_suffix, const jpa_tensor* v_suffix,
                                       int32_t batch,
                                       const int32_t* cu_q, const int32_t* cu_prefix,
                                       const int32_t* cu_suffix_real,
                                       float scale,
                                       const jpa_tensor* out, float* lse,
                                       int32_t split_wgs,
                                       void* stream);

/*
 * jpa_workspace_bytes -- workspace size jpa_forward_ws needs for head_dim
 * (64 or 128) and split_wgs (0: the current device's compute units); 0 for an
 * unsupported head_dim or when the device cannot be queried.
 */
JPA_API size_t jpa_workspace_bytes(int32_t head_dim, int32_t split_wgs);

/*
 * jpa_validate -- every check jpa_forward performs, on the host only; never
 * touches the device (tensor data pointers are only checked for alignment).
 */
JPA_API jpa_status jpa_validate(const jpa_tensor* q,
                                const jpa_tensor* k_prefix, const jpa_tensor* v_prefix,
                                const jpa_tensor* k_suffix, const jpa_tensor* v_suffix,
                                int32_t batch,
                                const int32_t* cu_q, const int32_t* cu_prefix,
                                const int32_t* cu_suffix_real,
                                float scale,
                                const jpa_tensor* out, const float* lse);

/*
 * jpa_plan -- decode the offsets into per-row bookkeeping (rows[0..batch),
 * caller-allocated) and the valid-token work count
 *     *valid_flops = sum_b heads_q * 4 * head_dim * Nq_b * Nk_b
 * (2*D multiply-adds for QK^T and PV per query/key pair).  Host only.
 * rows and valid_flops may each be NULL to skip that output.
 */
JPA_API jpa_status jpa_plan(int32_t batch,
                            const int32_t* cu_q, const int32_t* cu_prefix,
                            const int32_t* cu_suffix_real,
                            int32_t heads_q, int32_t head_dim,
                            jpa_row_plan* rows, int64_t* valid_flops);

/* Static string naming a status (never NULL). */
JPA_API const char* jpa_status_str(jpa_status status);

/* JPA_ABI_VERSION of the built library. */
JPA_API int32_t jpa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* JPA_H */
