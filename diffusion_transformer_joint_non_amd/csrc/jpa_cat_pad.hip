// gfx950 kernel: fused concatenation of cached frames and current frames
// along time plus zero padding of all three axes, for causal Conv3D inputs
// (sglang PR #29281 review, Cosmos3 VAE decode: cat + pad + zero-fill in one
// pass, 16-byte vectorised stores over the flat output, each output
// coordinate recovered from its flat index).
//
//   out[b, c, t, h, w] = src[b, c, t - tl, h - hl, w - wl]   inside, else 0,
//   src = [cache ; x] along time (cache frames first).
//
// Pure data movement, bound by HBM.  Design:
// * one thread writes one aligned 16-byte chunk (8 elements) of the flat
//   output; it finds the chunk's row (b, c, t, h) with multiply-shift
//   divisions (constants from the host) and its first column;
// * a chunk inside one output row whose 8 source elements all exist reads
//   two aligned 16-byte source chunks and shifts them into place
//   (v_alignbyte_b32), so a row shifted by the left pad is still read with
//   16-byte loads; chunks at row edges or across rows go element by element;
//   chunks of pad rows are stored as zeros without any load;
// * each thread handles kChunks chunks spaced a grid apart, loads first, so
//   several 16-byte loads per lane are in flight.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jpa_cat_pad_params.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChunks = 4;

__device__ __forceinline__ uint32_t divm(uint32_t n, uint32_t magic, int shift) {
    return (uint32_t)(((uint64_t)n * magic) >> shift);
}

// Source element of output element (row, col), or -1 for padding.  row is
// the flat output row (b, c, t, h); the source flat index is returned.
__device__ __forceinline__ int64_t source_of(const jpa_cat_pad_params& p, uint32_t row, int col,
                                             const uint16_t*& src) {
    const uint32_t r1 = divm(row, p.h_magic, p.h_shift);       // (b, c, t)
    const int h = (int)(row - r1 * (uint32_t)p.h_out);
    const uint32_t n = divm(r1, p.t_magic, p.t_shift);         // b * C + c
    const int t = (int)(r1 - n * (uint32_t)p.t_out);
    const int tt = t - p.pad_t0, hh = h - p.pad_h0, ww = col - p.pad_w0;
    if (tt < 0 || tt >= p.cache_frames + p.frames || hh < 0 || hh >= p.height || ww < 0 || ww >= p.width)
        return -1;
    const bool from_cache = tt < p.cache_frames;
    src = from_cache ? p.cache : p.x;
    const int64_t frames = from_cache ? p.cache_frames : p.frames;
    const int64_t ts = from_cache ? tt : tt - p.cache_frames;
    return (((int64_t)n * frames + ts) * p.height + hh) * p.width + ww;
}

__global__ __launch_bounds__(kThreads) void jpa_cat_pad_kernel(const jpa_cat_pad_params p) {
    // chunk c0 + u * stride (u < kChunks) of a pass: every pass tiles
    // stride * kChunks consecutive chunks, each u-slice of it over the grid
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    for (uint64_t c0 = (uint64_t)blockIdx.x * kThreads + threadIdx.x; c0 < p.chunks; c0 += stride * kChunks) {
        u32x4_t val[kChunks];
        bool live[kChunks];
#pragma unroll
        for (int u = 0; u < kChunks; ++u) {
            const uint64_t chunk = c0 + (uint64_t)u * stride;
            live[u] = chunk < p.chunks;
            val[u] = u32x4_t{0u, 0u, 0u, 0u};
            if (!live[u]) continue;
            const uint32_t o = (uint32_t)(chunk * 8);              // out_numel < 2^31
            const uint32_t row = divm(o, p.w_magic, p.w_shift);
            const int col = (int)(o - row * (uint32_t)p.w_out);
            const bool one_row = col + 8 <= p.w_out && o + 8 <= p.out_numel;
            const uint16_t* src = nullptr;
            if (one_row) {
                const int64_t s0 = source_of(p, row, col, src);
                const bool interior = s0 >= 0 && col - p.pad_w0 + 7 < p.width;
                if (interior) {
                    const int64_t a = s0 & ~(int64_t)7;
                    const int off = (int)(s0 - a);
                    const int64_t numel = src == p.cache ? p.cache_numel : p.x_numel;
                    if (off == 0) {
                        val[u] = *reinterpret_cast<const u32x4_t*>(src + a);
                        continue;
                    }
                    if (a + 16 <= numel) {
                        const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(src + a);
                        const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(src + a + 8);
                        uint32_t d[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        // window of 5 dwords starting at dword off/2, then a
                        // 2-byte shift when off is odd
                        const int k = off >> 1;
                        uint32_t wv[5];
#pragma unroll
                        for (int i = 0; i < 5; ++i) {
                            uint32_t v = d[i];
                            v = k == 1 ? d[i + 1] : v;
                            v = k == 2 ? d[i + 2] : v;
                            v = k == 3 ? d[(i + 3) & 7] : v;
                            wv[i] = v;
                        }
                        const uint32_t sh = (uint32_t)(off & 1) * 2;
#pragma unroll
                        for (int i = 0; i < 4; ++i) val[u][i] = __builtin_amdgcn_alignbyte(wv[i + 1], wv[i], sh);
                        continue;
                    }
                }
            }
            // general chunk: element by element (row edges, rows crossed, the
            // tensor's last elements)
            uint16_t e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                e[j] = 0;
                const uint32_t oj = o + j;
                if (oj >= p.out_numel) continue;
                const uint32_t rj = divm(oj, p.w_magic, p.w_shift);
                const int cj = (int)(oj - rj * (uint32_t)p.w_out);
                const uint16_t* sj = nullptr;
                const int64_t s = source_of(p, rj, cj, sj);
                if (s >= 0) e[j] = sj[s];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) val[u][i] = (uint32_t)e[2 * i] | ((uint32_t)e[2 * i + 1] << 16);
        }
#pragma unroll
        for (int u = 0; u < kChunks; ++u) {
            if (!live[u]) continue;
            const uint64_t chunk = c0 + (uint64_t)u * stride;
            const uint32_t o = (uint32_t)(chunk * 8);
            if (o + 8 <= p.out_numel) {
                *reinterpret_cast<u32x4_t*>(p.out + o) = val[u];
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (o + j < p.out_numel) p.out[o + j] = (uint16_t)(val[u][j >> 1] >> (16 * (j & 1)));
            }
        }
    }
}

}  // namespace

int jpa_launch_cat_pad(const jpa_cat_pad_params& p, void* stream) {
    if (p.chunks == 0) return (int)hipSuccess;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    const uint64_t per_block = (uint64_t)kThreads * kChunks;
    const uint64_t blocks = (p.chunks + per_block - 1) / per_block;
    const uint64_t cap = (uint64_t)(cus > 0 ? cus : 256) * 16;
    const int grid = (int)(blocks < cap ? blocks : cap);
    hipLaunchKernelGGL(jpa_cat_pad_kernel, dim3(grid), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}
