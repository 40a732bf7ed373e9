// Internal launch parameters shared by the host front end (jpa_host.cpp) and
// the gfx950 kernel (jpa_kernel.hip).  Not part of the public ABI.
#ifndef JPA_PARAMS_H
#define JPA_PARAMS_H

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
    jpa_kernel_row rows[JPA_MAX_ROWS];
};

// Enqueue one launch; returns the hipError_t of the launch as an int.
int jpa_launch_kernel(const jpa_kernel_params& p, int head_dim, void* stream);

#endif
