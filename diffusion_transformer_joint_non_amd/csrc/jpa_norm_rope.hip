// gfx950 kernel: per-head RMSNorm of q and k followed by the rotary
// embedding, producing the attention inputs in their packed [tokens, heads,
// head_dim] layout (vLLM-Omni diffusion performance-patterns guide, section
// "Q/K RMSNorm + RoPE": norm over head_dim with a per-channel weight, then
// rotation of the first rotary_dim channels with a per-token [cos | sin]
// table, interleaved or half-split pairs, remaining channels passed through;
// the Cosmos3 attention snippet of sglang PR #26973's review applies the same
// two steps to q and k right before attention).
//
// The step moves 2 x head_dim x 2 bytes per (token, head) row and does a few
// flops per byte, so it is bound by HBM bandwidth.  Design:
// * a row is head_dim/8 lanes, 16 contiguous bytes each (one dwordx4 load and
//   one store per lane), so a wave covers 64*8/head_dim whole rows and every
//   memory instruction is fully coalesced;
// * the mean square is an in-lane sum of 8 squares plus a DPP reduction over
//   the row's lanes; the reciprocal square root is the hardware one (about
//   one fp32 ulp, far below the bf16 rounding); everything is fp32 and the
//   result is rounded to bf16 once;
// * interleaved pairs sit inside a lane; half-split partners are read back
//   from the wave's own LDS copy of the normalised row;
// * when rotary_dim and the table layout allow it (VEC), the table is read
//   as float4s and the partner as a whole 8-channel chunk; otherwise per
//   channel;
// * one launch covers q and k: rows [0, rows_q) are q's, the rest k's, in
//   token-major order so that a token's table row is read by neighbouring
//   lanes; a grid-stride loop over groups of rows, each lane issuing the
//   loads of kUnroll rows (and their table entries) before using any, so
//   enough bytes are in flight to cover HBM latency.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jpa_norm_rope_params.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 4;                     // rows per lane with loads in flight together

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Sum over each aligned group of LANES lanes (8, 16 or 32), every lane of a
// group getting the same value: DPP quad permutations, then the half-row and
// row mirrors (the lanes being mirrored already hold equal partial sums, so
// a mirror pairs the two halves), then one cross-row exchange for 32.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int LANES>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp_mov<0xB1>(v);                   // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);                   // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);                  // row_half_mirror
    if constexpr (LANES >= 16) v += dpp_mov<0x140>(v);   // row_mirror
    if constexpr (LANES >= 32) v += __shfl_xor(v, 16, 64);
    return v;
}

template <int D, bool VEC>
__global__ __launch_bounds__(kThreads) void jpa_norm_rope_kernel(const jpa_norm_rope_params p) {
    constexpr int kLanes = D / 8;              // lanes per row
    constexpr int kRowsPerWave = 64 / kLanes;
    constexpr int kRowsPerBlock = kRowsPerWave * kWaves;
    __shared__ __attribute__((aligned(16))) float stage[kWaves][kRowsPerWave * D];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane / kLanes;             // row of the wave
    const int e0 = 8 * (lane % kLanes);        // first channel of this lane
    const int rot = p.rotary_dim;
    const int half = rot >> 1;
    const bool il = p.interleaved != 0;
    float* const srow = stage[wave] + sub * D;
    // VEC: this lane's 8 channels are all rotated or all passed through, and
    // (half-split) all in the first or all in the second half
    const bool rotated = e0 < rot;
    const bool first_half = e0 < half;
    const int i0 = il ? (e0 >> 1) : (first_half ? e0 : e0 - half);      // first pair index

    float wt[2][8];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < 8; j += 4) {
            const float4 v = *reinterpret_cast<const float4*>(p.w[s] + e0 + j);
            wt[s][j] = v.x; wt[s][j + 1] = v.y; wt[s][j + 2] = v.z; wt[s][j + 3] = v.w;
        }

    const int64_t step = (int64_t)gridDim.x * kRowsPerBlock * kUnroll;
    for (int64_t base = (int64_t)blockIdx.x * kRowsPerBlock * kUnroll; base < p.rows_total; base += step) {
        // issue every load of the group first: kUnroll rows per lane in flight
        bool act[kUnroll];
        int sel[kUnroll], hh[kUnroll];
        int64_t tt[kUnroll];
        u32x4_t xv[kUnroll];
        float4 tc[kUnroll][2], ts[kUnroll][2];       // VEC table values (cos, sin)
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t r = base + u * kRowsPerBlock + wave * kRowsPerWave + sub;
            act[u] = r < p.rows_total;
            sel[u] = r >= p.rows_q ? 1 : 0;
            // row of its tensor (< 2^31) -> (token, head) by multiply-shift
            const uint32_t rr = act[u] ? (uint32_t)(sel[u] ? r - p.rows_q : r) : 0u;
            // per-lane choice between the two tensors' scalar arguments (never
            // an indexed read of the argument block, which would be a memory load)
            const bool k_row = sel[u] != 0;
            const uint32_t magic = k_row ? p.div_magic[1] : p.div_magic[0];
            const int shift = k_row ? p.div_shift[1] : p.div_shift[0];
            const uint32_t t32 = (uint32_t)(((uint64_t)rr * magic) >> shift);
            tt[u] = t32;
            hh[u] = (int)(rr - t32 * (uint32_t)(k_row ? p.heads[1] : p.heads[0]));
            xv[u] = u32x4_t{0u, 0u, 0u, 0u};
            if (act[u]) {
                const uint16_t* const xb = k_row ? p.x[1] : p.x[0];
                const uint32_t xts = (uint32_t)(k_row ? p.x_ts[1] : p.x_ts[0]);
                const uint32_t xhs = (uint32_t)(k_row ? p.x_hs[1] : p.x_hs[0]);
                // q/k rows are read once: a streaming (non-temporal) load
                xv[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4_t*>(xb + (uint64_t)t32 * xts + ((uint32_t)hh[u] * xhs + (uint32_t)e0)));
            }
            if constexpr (VEC) {
                if (act[u] && rotated) {
                    const float* const tab = p.table + (uint64_t)(uint32_t)tt[u] * (uint64_t)p.table_stride;
                    tc[u][0] = *reinterpret_cast<const float4*>(tab + i0);
                    ts[u][0] = *reinterpret_cast<const float4*>(tab + half + i0);
                    if (!il) {
                        tc[u][1] = *reinterpret_cast<const float4*>(tab + i0 + 4);
                        ts[u][1] = *reinterpret_cast<const float4*>(tab + half + i0 + 4);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int s = sel[u];
            float y[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) { y[2 * j] = bf16_lo(xv[u][j]); y[2 * j + 1] = bf16_hi(xv[u][j]); }
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) ss = fmaf(y[j], y[j], ss);
            ss = group_sum<kLanes>(ss);
            const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.eps);
#pragma unroll
            for (int j = 0; j < 8; ++j) y[j] = y[j] * inv * (s ? wt[1][j] : wt[0][j]);

            if (rot > 0) {
                float part[8];
                if (il) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) part[j] = y[j ^ 1];
                } else {
                    // the row's normalised channels through this wave's LDS rows
                    *reinterpret_cast<float4*>(srow + e0) = make_float4(y[0], y[1], y[2], y[3]);
                    *reinterpret_cast<float4*>(srow + e0 + 4) = make_float4(y[4], y[5], y[6], y[7]);
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    if constexpr (VEC) {
                        const int pe = first_half ? e0 + half : e0 - half;
                        if (rotated) {
                            const float4 a4 = *reinterpret_cast<const float4*>(srow + pe);
                            const float4 b4 = *reinterpret_cast<const float4*>(srow + pe + 4);
                            part[0] = a4.x; part[1] = a4.y; part[2] = a4.z; part[3] = a4.w;
                            part[4] = b4.x; part[5] = b4.y; part[6] = b4.z; part[7] = b4.w;
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const int e = e0 + j;
                            part[j] = e < half ? srow[e + half] : (e < rot ? srow[e - half] : 0.f);
                        }
                    }
                    // the reads are done before the next row overwrites the stage
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                }
                if constexpr (VEC) {
                    if (rotated && act[u]) {
                        float cs[8], sn[8];
                        if (il) {
                            const float cc[4] = {tc[u][0].x, tc[u][0].y, tc[u][0].z, tc[u][0].w};
                            const float sv[4] = {ts[u][0].x, ts[u][0].y, ts[u][0].z, ts[u][0].w};
#pragma unroll
                            for (int j = 0; j < 8; ++j) { cs[j] = cc[j >> 1]; sn[j] = sv[j >> 1]; }
                        } else {
                            const float cc[8] = {tc[u][0].x, tc[u][0].y, tc[u][0].z, tc[u][0].w,
                                                 tc[u][1].x, tc[u][1].y, tc[u][1].z, tc[u][1].w};
                            const float sv[8] = {ts[u][0].x, ts[u][0].y, ts[u][0].z, ts[u][0].w,
                                                 ts[u][1].x, ts[u][1].y, ts[u][1].z, ts[u][1].w};
#pragma unroll
                            for (int j = 0; j < 8; ++j) { cs[j] = cc[j]; sn[j] = sv[j]; }
                        }
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const bool a = il ? (j & 1) == 0 : first_half;
                            y[j] = a ? y[j] * cs[j] - part[j] * sn[j] : y[j] * cs[j] + part[j] * sn[j];
                        }
                    }
                } else if (act[u]) {
                    const float* const tab = p.table + (uint64_t)(uint32_t)tt[u] * (uint64_t)p.table_stride;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int e = e0 + j;
                        if (e < rot) {
                            const bool a = il ? (e & 1) == 0 : e < half;
                            const int i = il ? (e >> 1) : (a ? e : e - half);
                            const float c = tab[i], sv = tab[half + i];
                            y[j] = a ? y[j] * c - part[j] * sv : y[j] * c + part[j] * sv;
                        }
                    }
                }
            }
            if (act[u]) {
                const u32x4_t o = {pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]),
                                   pack_bf16(y[6], y[7])};
                uint16_t* const yb = s ? p.y[1] : p.y[0];
                const uint32_t yts = (uint32_t)(s ? p.y_ts[1] : p.y_ts[0]);
                const uint32_t yhs = (uint32_t)(s ? p.y_hs[1] : p.y_hs[0]);
                // written once: a streaming store (5% faster back to back than
                // cached loads and stores of q/k; the table stays cached, every
                // head of a token reads its row)
                __builtin_nontemporal_store(
                    o, reinterpret_cast<u32x4_t*>(yb + (uint64_t)(uint32_t)tt[u] * yts + ((uint32_t)hh[u] * yhs + (uint32_t)e0)));
            }
        }
    }
}

template <int D>
int launch_d(const jpa_norm_rope_params& p, bool vec, hipStream_t s) {
    constexpr int kRowsPerBlock = (64 / (D / 8)) * kWaves * kUnroll;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    const int64_t groups = (p.rows_total + kRowsPerBlock - 1) / kRowsPerBlock;
    const int64_t cap = (int64_t)(cus > 0 ? cus : 256) * 8;
    const int grid = (int)(groups < cap ? groups : cap);
    if (vec)
        hipLaunchKernelGGL((jpa_norm_rope_kernel<D, true>), dim3(grid), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((jpa_norm_rope_kernel<D, false>), dim3(grid), dim3(kThreads), 0, s, p);
    return (int)hipGetLastError();
}

}  // namespace

int jpa_launch_norm_rope(const jpa_norm_rope_params& p, int head_dim, void* stream) {
    if (p.rows_total == 0) return (int)hipSuccess;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // float4 table reads and whole-chunk partners need every lane's 8 channels
    // on one side of every boundary and 16-byte aligned table rows
    const bool vec = ((reinterpret_cast<uintptr_t>(p.table) & 15u) == 0) && (p.table_stride % 4 == 0) &&
                     (p.interleaved ? p.rotary_dim % 8 == 0 : p.rotary_dim % 16 == 0);
    switch (head_dim) {
        case 64: return launch_d<64>(p, vec, s);
        case 128: return launch_d<128>(p, vec, s);
        default: return launch_d<256>(p, vec, s);
    }
}
