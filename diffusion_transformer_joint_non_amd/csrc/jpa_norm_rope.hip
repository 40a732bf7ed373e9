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
// * the mean square is an in-lane sum of 8 squares plus a butterfly over the
//   row's lanes; everything is fp32 and the result is rounded to bf16 once;
// * interleaved pairs sit inside a lane; half-split partners are read back
//   from the wave's own LDS copy of the normalised row;
// * when rotary_dim and the table layout allow it (VEC), the table is read
//   as float4s and the partner as a whole 8-channel chunk; otherwise per
//   channel;
// * one launch covers q and k: rows [0, rows_q) are q's, the rest k's, in
//   token-major order so that a token's table row is read by neighbouring
//   lanes; a grid-stride loop over groups of rows.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jpa_norm_rope_params.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (the inputs here are finite or NaN;
// NaN stays NaN).
__device__ __forceinline__ uint32_t to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
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
    float* const srow = stage[wave] + sub * D;

    float wt[2][8];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < 8; j += 4) {
            const float4 v = *reinterpret_cast<const float4*>(p.w[s] + e0 + j);
            wt[s][j] = v.x; wt[s][j + 1] = v.y; wt[s][j + 2] = v.z; wt[s][j + 3] = v.w;
        }

    for (int64_t base = (int64_t)blockIdx.x * kRowsPerBlock; base < p.rows_total;
         base += (int64_t)gridDim.x * kRowsPerBlock) {
        const int64_t r = base + wave * kRowsPerWave + sub;
        const bool active = r < p.rows_total;
        const int s = r >= p.rows_q ? 1 : 0;
        const int64_t rr = s ? r - p.rows_q : r;
        const int heads = p.heads[s];
        const int64_t t = active ? rr / heads : 0;
        const int h = active ? (int)(rr - t * heads) : 0;

        float y[8];
        if (active) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p.x[s] + t * p.x_ts[s] + (int64_t)h * p.x_hs[s] + e0);
#pragma unroll
            for (int j = 0; j < 4; ++j) { y[2 * j] = bf16_lo(v[j]); y[2 * j + 1] = bf16_hi(v[j]); }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) y[j] = 0.f;
        }
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fmaf(y[j], y[j], ss);
#pragma unroll
        for (int m = kLanes / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
        const float inv = 1.0f / sqrtf(ss * (1.0f / D) + p.eps);
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = y[j] * inv * (s ? wt[1][j] : wt[0][j]);

        if (rot > 0) {
            const float* const tab = p.table + t * p.table_stride;
            float part[8], cs[8], sn[8];
            if (p.interleaved) {
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
                    if (e0 < rot) {
                        const int pe = e0 < half ? e0 + half : e0 - half;
                        const float4 a = *reinterpret_cast<const float4*>(srow + pe);
                        const float4 b = *reinterpret_cast<const float4*>(srow + pe + 4);
                        part[0] = a.x; part[1] = a.y; part[2] = a.z; part[3] = a.w;
                        part[4] = b.x; part[5] = b.y; part[6] = b.z; part[7] = b.w;
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int e = e0 + j;
                        part[j] = e < half ? srow[e + half] : (e < rot ? srow[e - half] : 0.f);
                    }
                }
                // the reads are done before the next group overwrites the rows
                __builtin_amdgcn_wave_barrier();
            }
            if constexpr (VEC) {
                if (e0 < rot && active) {
                    const int i0 = p.interleaved ? (e0 >> 1) : (e0 < half ? e0 : e0 - half);
                    if (p.interleaved) {
                        const float4 c4 = *reinterpret_cast<const float4*>(tab + i0);
                        const float4 s4 = *reinterpret_cast<const float4*>(tab + half + i0);
                        const float cc[4] = {c4.x, c4.y, c4.z, c4.w}, ssn[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                        for (int j = 0; j < 8; ++j) { cs[j] = cc[j >> 1]; sn[j] = ssn[j >> 1]; }
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; j += 4) {
                            const float4 c4 = *reinterpret_cast<const float4*>(tab + i0 + j);
                            const float4 s4 = *reinterpret_cast<const float4*>(tab + half + i0 + j);
                            cs[j] = c4.x; cs[j + 1] = c4.y; cs[j + 2] = c4.z; cs[j + 3] = c4.w;
                            sn[j] = s4.x; sn[j + 1] = s4.y; sn[j + 2] = s4.z; sn[j + 3] = s4.w;
                        }
                    }
                    const bool first = p.interleaved ? true : e0 < half;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const bool a = p.interleaved ? (j & 1) == 0 : first;
                        y[j] = a ? y[j] * cs[j] - part[j] * sn[j] : y[j] * cs[j] + part[j] * sn[j];
                    }
                }
            } else {
                if (active) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int e = e0 + j;
                        if (e < rot) {
                            const bool a = p.interleaved ? (e & 1) == 0 : e < half;
                            const int i = p.interleaved ? (e >> 1) : (a ? e : e - half);
                            const float c = tab[i], sv = tab[half + i];
                            y[j] = a ? y[j] * c - part[j] * sv : y[j] * c + part[j] * sv;
                        }
                    }
                }
            }
        }
        if (active) {
            const u32x4_t o = {to_bf16(y[0]) | (to_bf16(y[1]) << 16), to_bf16(y[2]) | (to_bf16(y[3]) << 16),
                               to_bf16(y[4]) | (to_bf16(y[5]) << 16), to_bf16(y[6]) | (to_bf16(y[7]) << 16)};
            *reinterpret_cast<u32x4_t*>(p.y[s] + t * p.y_ts[s] + (int64_t)h * p.y_hs[s] + e0) = o;
        }
    }
}

template <int D>
int launch_d(const jpa_norm_rope_params& p, bool vec, hipStream_t s) {
    constexpr int kRowsPerBlock = (64 / (D / 8)) * kWaves;
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
