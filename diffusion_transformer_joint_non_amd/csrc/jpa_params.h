// Internal launch parameters shared by the host front end (jpa_host.cpp) and
// the gfx950 kernel (jpa_kernel.hip).  Not part of the public ABI.
#ifndef JPA_PARAMS_H
#define JPA_PARAMS_H

#include <stddef.h>
#include <stdint.h>

// Batch rows carried by one launch (their plan travels in the kernel
// argument block, so the kernel never reads offsets from device memory).
#define JPA_MAX_ROWS 32
// Query rows per workgroup: 4 waves x 2 blocks of 32 queries.
#define JPA_BLOCK_M 256

struct jpa_kernel_row {
    int32_t q_start;     // first query slot
    int32_t q_slots;     // Lq_b
    int32_t q_real;      // Nq_b
    int32_t p_start;     // first prefix token
    int32_t p_len;       // P_b
    int32_t s_start;     // first suffix slot
    int32_t keys;        // Nk_b = P_b + R_b
    int32_t tile_start;  // first query tile of this row within the launch
};

struct jpa_kernel_params {
    const uint16_t* q;
    const uint16_t* kp;
    const uint16_t* vp;
    const uint16_t* ks;
    const uint16_t* vs;
    uint16_t* out;
    float* lse;                 // may be null
    int64_t q_ts, kp_ts, vp_ts, ks_ts, vs_ts, o_ts;   // token strides (elements)
    int64_t lse_ld;             // Tq: row length of lse [Hq, Tq]
    int32_t q_hs, kp_hs, vp_hs, ks_hs, vs_hs, o_hs;   // head strides (elements)
    int32_t hq;                 // query heads
    int32_t group;              // Hq / Hkv
    int32_t nrows;              // rows in this launch
    int32_t total_tiles;        // query tiles over those rows (per head)
    float c;                    // scale * log2(e)
    // Work split.  The first n_dp workgroups each take one whole item (query
    // head, query tile) in an XCD-grouped order.  The next sk_wgs workgroups
    // split the remaining items (n_dp .. hq*total_tiles-1) into balanced
    // contiguous ranges of "units": a real item counts its key tiles, an
    // all-pad item counts 1.  The pieces of an item cut between ranges leave
    // partial results in the workspace, merged by a second kernel.
    int32_t n_dp;               // whole-item workgroups
    int32_t sk_wgs;             // balanced-range workgroups (0: none)
    int64_t head_units;         // units of one query head (all rows of the launch)
    int64_t tail_unit0;         // absolute unit of item n_dp (hq*head_units + ..)
    int64_t tail_units;         // units of items n_dp ..
    float* ws_o;                // [2*sk_wgs][JPA_BLOCK_M][head_dim] partial outputs
    float* ws_lse;              // [2*sk_wgs][JPA_BLOCK_M] partial LSE (log2 units)
    jpa_kernel_row rows[JPA_MAX_ROWS];
};

// Workspace layout for up to `wgs` balanced-range workgroups (bytes; every
// part 256-byte aligned).
inline size_t jpa_ws_o_bytes(int wgs, int head_dim) {
    return (size_t)2 * wgs * JPA_BLOCK_M * head_dim * sizeof(float);
}
inline size_t jpa_ws_lse_bytes(int wgs) { return (size_t)2 * wgs * JPA_BLOCK_M * sizeof(float); }

// Enqueue one launch; returns the hipError_t of the launch as an int.
int jpa_launch_kernel(const jpa_kernel_params& p, int head_dim, void* stream);
// Compute units of the current device, or 0 if the runtime reports none.
int jpa_device_cus();

#endif
