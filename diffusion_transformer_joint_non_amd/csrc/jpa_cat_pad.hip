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
//   16-byte loads; chunks at row edges or running into the next row go
//   element by element with each row's source located once (no division per
//   element); pad elements are zeros without any load;
// * the upper aligned source chunk of a shifted read is, for consecutive
//   chunks of one row, the lower chunk of the next lane: it comes from that
//   lane by a DPP wave shift (checked by an address tag), so a shifted row
//   costs one 16-byte load per chunk, not two;
// * each thread handles kChunks chunks spaced a grid apart, loads first, so
//   several 16-byte loads per lane are in flight.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jpa_cat_pad_params.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChunks = 2;

__device__ __forceinline__ uint32_t divm(uint32_t n, uint32_t magic, int shift) {
    return (uint32_t)(((uint64_t)n * magic) >> shift);
}

// First source element of output row `row` (flat (b, c, t, h)) at column
// pad_w0, or -1 when the whole row is padding; *cache_row says which tensor.
// Source tensors hold fewer than 2^31 elements.
__device__ __forceinline__ int32_t source_row(const jpa_cat_pad_params& p, uint32_t row, bool* cache_row) {
    const uint32_t r1 = divm(row, p.h_magic, p.h_shift);       // (b, c, t)
    const int h = (int)(row - r1 * (uint32_t)p.h_out);
    const uint32_t n = divm(r1, p.t_magic, p.t_shift);         // b * C + c
    const int t = (int)(r1 - n * (uint32_t)p.t_out);
    const int tt = t - p.pad_t0, hh = h - p.pad_h0;
    if (tt < 0 || tt >= p.cache_frames + p.frames || hh < 0 || hh >= p.height) return -1;
    const bool from_cache = tt < p.cache_frames;
    *cache_row = from_cache;
    const uint32_t frames = (uint32_t)(from_cache ? p.cache_frames : p.frames);
    const uint32_t ts = (uint32_t)(from_cache ? tt : tt - p.cache_frames);
    return (int32_t)(((n * frames + ts) * (uint32_t)p.height + (uint32_t)hh) * (uint32_t)p.width);
}

// The 8 elements from flat source index s0 (any alignment) with two aligned
// 16-byte loads and a byte shift; a + 16 elements must lie inside src.
__device__ __forceinline__ u32x4_t load8_shifted(const uint16_t* src, uint32_t s0) {
    const uint32_t a = s0 & ~7u;
    const uint32_t off = s0 - a;
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(src + a);
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(src + a + 8);
    const uint32_t d[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const uint32_t k = off >> 1;                       // first dword, then a 2-byte shift if off is odd
    uint32_t wv[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const uint32_t lo2 = (k & 1) ? d[i + 1] : d[i];
        const uint32_t hi2 = (k & 1) ? d[i + 3] : d[i + 2];
        wv[i] = (k & 2) ? hi2 : lo2;
    }
    const uint32_t sh = (off & 1) * 2;
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_alignbyte(wv[i + 1], wv[i], sh);
    return r;
}

// One 16-byte output chunk at flat element o.  Lanes of a wave hold
// consecutive chunks, so the upper aligned source chunk a lane needs is
// usually the lower one its right neighbour loads: it is taken from that
// lane (DPP wave shift) and loaded only where the neighbour's differs.
__device__ __forceinline__ u32x4_t chunk_value(const jpa_cat_pad_params& p, uint32_t o, bool live) {
    const uint32_t row = divm(o, p.w_magic, p.w_shift);
    const int col = (int)(o - row * (uint32_t)p.w_out);
    bool c0 = false, c1 = false;
    const int32_t b0 = live ? source_row(p, row, &c0) : -1;
    const int w0 = col - p.pad_w0;                     // source column of element 0
    const bool fast = b0 >= 0 && w0 >= 0 && w0 + 8 <= p.width;
    const uint16_t* src = c0 ? p.cache : p.x;
    const uint32_t s0 = fast ? (uint32_t)b0 + (uint32_t)w0 : 0u;
    const uint32_t a = s0 & ~7u;
    u32x4_t lo = u32x4_t{0u, 0u, 0u, 0u};
    if (fast) lo = *reinterpret_cast<const u32x4_t*>(src + a);
    // the right neighbour's lower chunk and its address tag (every lane runs the shifts)
    const uint32_t tag = fast ? (a | (c0 ? 1u : 0u)) : 0xFFFFFFFFu;
    const uint32_t ntag = (uint32_t)__builtin_amdgcn_mov_dpp((int)tag, 0x130, 0xF, 0xF, false);   // wave_shl:1
    u32x4_t hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) hi[i] = (uint32_t)__builtin_amdgcn_mov_dpp((int)lo[i], 0x130, 0xF, 0xF, false);
    if (fast) {
        const uint32_t off = s0 - a;
        if (off == 0) return lo;
        const int64_t numel = c0 ? p.cache_numel : p.x_numel;
        const bool shared = (threadIdx.x & 63) != 63 && ntag == ((a + 8) | (c0 ? 1u : 0u));
        if (shared || (int64_t)a + 16 <= numel) {
            if (!shared) hi = *reinterpret_cast<const u32x4_t*>(src + a + 8);
            const uint32_t d[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const uint32_t k = off >> 1;
            uint32_t wv[5];
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                const uint32_t l2 = (k & 1) ? d[i + 1] : d[i];
                const uint32_t h2 = (k & 1) ? d[i + 3] : d[i + 2];
                wv[i] = (k & 2) ? h2 : l2;
            }
            const uint32_t sh = (off & 1) * 2;
            u32x4_t r;
#pragma unroll
            for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_alignbyte(wv[i + 1], wv[i], sh);
            return r;
        }
    }
    uint16_t e[8];
    if (p.w_out >= 8) {
        const int32_t b1 = live && col + 8 > p.w_out ? source_row(p, row + 1, &c1) : -1;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            e[j] = 0;
            const bool next = col + j >= p.w_out;
            const int32_t base = next ? b1 : b0;
            const int w = (next ? col + j - p.w_out : col + j) - p.pad_w0;
            if (live && o + j < p.out_numel && base >= 0 && w >= 0 && w < p.width)
                e[j] = ((next ? c1 : c0) ? p.cache : p.x)[base + w];
        }
    } else {
        for (int j = 0; j < 8; ++j) {
            e[j] = 0;
            const uint32_t oj = o + j;
            if (!live || oj >= p.out_numel) continue;
            const uint32_t rj = divm(oj, p.w_magic, p.w_shift);
            const int w = (int)(oj - rj * (uint32_t)p.w_out) - p.pad_w0;
            bool cj = false;
            const int32_t base = source_row(p, rj, &cj);
            if (base >= 0 && w >= 0 && w < p.width) e[j] = (cj ? p.cache : p.x)[base + w];
        }
    }
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (uint32_t)e[2 * i] | ((uint32_t)e[2 * i + 1] << 16);
    return r;
}

__global__ __launch_bounds__(kThreads) void jpa_cat_pad_kernel(const jpa_cat_pad_params p) {
    // chunk c0 + u * stride (u < kChunks) of a pass: every pass tiles
    // stride * kChunks consecutive chunks, each u-slice of it over the grid
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    for (uint64_t c0 = (uint64_t)blockIdx.x * kThreads + threadIdx.x; c0 < p.chunks; c0 += stride * kChunks) {
        u32x4_t val[kChunks];
#pragma unroll
        for (int u = 0; u < kChunks; ++u) {
            const uint64_t chunk = c0 + (uint64_t)u * stride;
            // every lane calls it (the wave shift needs all lanes), dead ones idle
            val[u] = chunk_value(p, (uint32_t)(chunk < p.chunks ? chunk * 8 : 0), chunk < p.chunks);
        }
#pragma unroll
        for (int u = 0; u < kChunks; ++u) {
            const uint64_t chunk = c0 + (uint64_t)u * stride;
            if (chunk >= p.chunks) continue;
            const uint32_t o = (uint32_t)(chunk * 8);      // out_numel < 2^31
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
