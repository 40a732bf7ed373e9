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
// * one thread owns one aligned 16-byte chunk (8 elements) of the flat
//   output; it finds the chunk's row (b, c, t, h) with multiply-shift
//   divisions (constants from the host) and its first column;
// * a chunk inside one output row whose 8 source elements all exist reads
//   two aligned 16-byte source chunks and shifts them into place
//   (v_alignbyte_b32), so a row shifted by the left pad is still read with
//   16-byte loads; a chunk of zeros (a padded row, a run of pad columns)
//   loads nothing;
// * the upper aligned source chunk of a shifted read is, for consecutive
//   chunks of one row, the lower chunk of the next lane: it comes from that
//   lane by a DPP wave shift (checked by an address tag), so a shifted row
//   costs one 16-byte load per chunk, not two;
// * every other chunk (a row edge with pad columns, a chunk across two rows,
//   the tensor's last chunk) is an edge chunk: the wave collects its edge
//   chunks by ballot and writes them with all 64 lanes at once, eight lanes
//   per chunk, one element per lane, so a row edge does not hold the rest of
//   the wave on an element-by-element path;
// * a lane's loads (lower chunk, own upper chunk, edge element) are all
//   issued before any is waited for: whether the upper chunk comes from the
//   neighbour follows from the two lanes' plans, not from loaded data;
// * the tensor pointers live in scalar registers: a per-lane choice between
//   two kernel arguments compiles to a per-lane load of the argument block,
//   which had cost a dependent memory round trip per chunk;
// * one chunk per thread per pass, and a grid of about a quarter of the
//   chunks' threads, so each thread makes ~4 passes, measured best (kChunks
//   chunks spaced a grid apart are supported).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jpa_cat_pad_params.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChunks = 1;
constexpr int kPassesPerThread = 4;

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

// A wave-uniform 64-bit value held in scalar registers.  Per-lane choices
// between two kernel arguments (x or cache) are made on such copies: a
// choice between the arguments themselves compiles to a per-lane load from
// the argument block.
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Global-memory views (address space 1), so loads stay global loads.
typedef const __attribute__((address_space(1))) uint16_t g_u16;
typedef const __attribute__((address_space(1))) u32x4_t g_u32x4;

// The two source tensors as such scalar copies.
struct sources {
    g_u16* x;
    g_u16* cache;
    int64_t x_numel, cache_numel;
};

// How the 16-byte output chunk at flat element o is written.  "data": the
// chunk lies inside one output row and holds 8 source elements of one source
// row, read as the aligned source chunk at a (plus the next one when off,
// the misalignment, is not 0).  "zero": inside one row and all padding (a
// padded row, a run of pad columns).  Anything else -- a row edge with pad
// columns, a chunk across two rows, a shifted read at a tensor's last chunk
// -- is an edge chunk.  No memory is touched.
struct chunk_plan {
    g_u16* src;
    uint32_t a, off, tag;    // tag: a | tensor bit for data chunks, else ~0
    bool data, edge;
};

__device__ __forceinline__ chunk_plan plan_chunk(const jpa_cat_pad_params& p, const sources& sv, uint32_t o,
                                                 bool live) {
    const uint32_t row = divm(o, p.w_magic, p.w_shift);
    const int col = (int)(o - row * (uint32_t)p.w_out);
    const bool in_row = live && col + 8 <= p.w_out;   // then o + 8 <= out_numel
    bool c0 = false;
    const int32_t b0 = in_row ? source_row(p, row, &c0) : -1;
    const int w0 = col - p.pad_w0;                     // source column of element 0
    const bool zero = in_row && (b0 < 0 || w0 + 8 <= 0 || w0 >= p.width);
    const uint32_t s0 = (uint32_t)b0 + (uint32_t)w0;
    chunk_plan pl;
    pl.src = c0 ? sv.cache : sv.x;
    pl.a = s0 & ~7u;
    pl.off = s0 - pl.a;
    const int64_t numel = c0 ? sv.cache_numel : sv.x_numel;
    pl.data = b0 >= 0 && w0 >= 0 && w0 + 8 <= p.width && (pl.off == 0 || (int64_t)pl.a + 16 <= numel);
    pl.edge = live && !pl.data && !zero;
    pl.tag = pl.data ? (pl.a | (c0 ? 1u : 0u)) : 0xFFFFFFFFu;
    return pl;
}

// Output element o (< out_numel), located on its own.
__device__ __forceinline__ uint16_t element_value(const jpa_cat_pad_params& p, const sources& sv, uint32_t o) {
    const uint32_t row = divm(o, p.w_magic, p.w_shift);
    const int w = (int)(o - row * (uint32_t)p.w_out) - p.pad_w0;
    bool c = false;
    const int32_t base = source_row(p, row, &c);
    return (base >= 0 && w >= 0 && w < p.width) ? (c ? sv.cache : sv.x)[base + w] : (uint16_t)0;
}

// Edge chunks are written by the whole wave at once, eight at a time: lane l
// takes element l % 8 of the (l / 8)-th lowest remaining bit of m (a wave
// ballot, bit = lane of the chunk), so eight lanes write one chunk's 16
// contiguous bytes.  Removes those bits from m; returns this lane's chunk
// lane, or -1.  m is wave-uniform, so is the loop.
__device__ __forceinline__ int take_eight(uint64_t& m) {
    const int lane = threadIdx.x & 63;
    int mine = -1;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if (m) {
            const int pos = __builtin_ctzll(m);
            m &= m - 1;
            if ((lane >> 3) == k) mine = pos;
        }
    }
    return mine;
}

__global__ __launch_bounds__(kThreads) void jpa_cat_pad_kernel(const jpa_cat_pad_params p) {
    const sources sv = {(g_u16*)uniform64(reinterpret_cast<uintptr_t>(p.x)),
                        (g_u16*)uniform64(reinterpret_cast<uintptr_t>(p.cache)),
                        (int64_t)uniform64((uint64_t)p.x_numel), (int64_t)uniform64((uint64_t)p.cache_numel)};
    // chunk c0 + u * stride (u < kChunks) of a pass: every pass tiles
    // stride * kChunks consecutive chunks, each u-slice of it over the grid;
    // a wave holds 64 consecutive chunks of each slice and stays in the loop
    // as a whole (the condition is the same for all its lanes)
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    const uint64_t lane = threadIdx.x & 63;
    for (uint64_t c0 = (uint64_t)blockIdx.x * kThreads + threadIdx.x; c0 - lane < p.chunks; c0 += stride * kChunks) {
        chunk_plan pl[kChunks];
#pragma unroll
        for (int u = 0; u < kChunks; ++u) {
            const uint64_t chunk = c0 + (uint64_t)u * stride;
            pl[u] = plan_chunk(p, sv, (uint32_t)(chunk < p.chunks ? chunk * 8 : 0), chunk < p.chunks);
        }
        // the first eight edge chunks of each slice: their loads go out with the others
        uint64_t em[kChunks];
        int mine[kChunks];
        uint16_t ev[kChunks];
#pragma unroll
        for (int u = 0; u < kChunks; ++u) {
            em[u] = __builtin_amdgcn_ballot_w64(pl[u].edge);
            mine[u] = take_eight(em[u]);
            const uint64_t o = (c0 - lane + (uint64_t)u * stride + (uint64_t)mine[u]) * 8 + (lane & 7);
            if (mine[u] < 0 || o >= p.out_numel) mine[u] = -1;
            ev[u] = mine[u] >= 0 ? element_value(p, sv, (uint32_t)o) : (uint16_t)0;
        }
        // whether a lane's upper source chunk is its right neighbour's lower one
        // follows from the plans alone (address tags by DPP wave shift), so
        // every load of the pass is issued before any is waited for
        bool own_hi[kChunks];
#pragma unroll
        for (int u = 0; u < kChunks; ++u) {
            const uint32_t ntag = (uint32_t)__builtin_amdgcn_mov_dpp((int)pl[u].tag, 0x130, 0xF, 0xF, false);  // wave_shl:1
            own_hi[u] = pl[u].data && pl[u].off != 0 && !(lane != 63 && ntag == pl[u].tag + 8);
        }
        u32x4_t lo[kChunks], hi[kChunks];
#pragma unroll
        for (int u = 0; u < kChunks; ++u) {
            lo[u] = u32x4_t{0u, 0u, 0u, 0u};
            if (pl[u].data) lo[u] = *reinterpret_cast<g_u32x4*>(pl[u].src + pl[u].a);
            if (own_hi[u]) hi[u] = *reinterpret_cast<g_u32x4*>(pl[u].src + pl[u].a + 8);
        }
#pragma unroll
        for (int u = 0; u < kChunks; ++u) {
            u32x4_t nb;                                    // the right neighbour's lower chunk
#pragma unroll
            for (int i = 0; i < 4; ++i) nb[i] = (uint32_t)__builtin_amdgcn_mov_dpp((int)lo[u][i], 0x130, 0xF, 0xF, false);
            if (!own_hi[u]) hi[u] = nb;
        }
#pragma unroll
        for (int u = 0; u < kChunks; ++u) {
            const uint64_t chunk = c0 + (uint64_t)u * stride;
            u32x4_t val = lo[u];
            if (pl[u].off != 0) {                          // shift (data chunks; the rest store lo = 0)
                const uint32_t d[8] = {lo[u][0], lo[u][1], lo[u][2], lo[u][3], hi[u][0], hi[u][1], hi[u][2], hi[u][3]};
                const uint32_t k = pl[u].off >> 1;      // first dword, then a 2-byte shift if off is odd
                uint32_t wv[5];
#pragma unroll
                for (int i = 0; i < 5; ++i) {
                    const uint32_t l2 = (k & 1) ? d[i + 1] : d[i];
                    const uint32_t h2 = (k & 1) ? d[i + 3] : d[i + 2];
                    wv[i] = (k & 2) ? h2 : l2;
                }
                const uint32_t sh = (pl[u].off & 1) * 2;
#pragma unroll
                for (int i = 0; i < 4; ++i) val[i] = __builtin_amdgcn_alignbyte(wv[i + 1], wv[i], sh);
            }
            if (!pl[u].data) val = u32x4_t{0u, 0u, 0u, 0u};
            if (chunk < p.chunks && !pl[u].edge)          // a whole in-row chunk: o + 8 <= out_numel
                *reinterpret_cast<u32x4_t*>(p.out + chunk * 8) = val;
        }
#pragma unroll
        for (int u = 0; u < kChunks; ++u) {
            const uint64_t base = c0 - lane + (uint64_t)u * stride;
            if (mine[u] >= 0) p.out[(base + (uint64_t)mine[u]) * 8 + (lane & 7)] = ev[u];
            while (em[u]) {                                // more than eight edge chunks in the slice
                const int more = take_eight(em[u]);
                const uint64_t o = (base + (uint64_t)more) * 8 + (lane & 7);
                if (more >= 0 && o < p.out_numel) p.out[o] = element_value(p, sv, (uint32_t)o);
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
    // about kPassesPerThread passes of the grid-stride loop per thread (one
    // pass per thread, or 17 on the largest decoder shape, both measured
    // 6-9% slower), and at least 8 workgroups per CU when there is the work
    const uint64_t per_pass = (uint64_t)kThreads * kChunks;
    const uint64_t need = (p.chunks + per_pass - 1) / per_pass;              // one pass each
    const uint64_t spread = (p.chunks + per_pass * kPassesPerThread - 1) / (per_pass * kPassesPerThread);
    const uint64_t floor8 = (uint64_t)(cus > 0 ? cus : 256) * 8;
    uint64_t g = spread > floor8 ? spread : (need < floor8 ? need : floor8);
    const int grid = (int)(g < (uint64_t)(1u << 30) ? g : (uint64_t)(1u << 30));
    hipLaunchKernelGGL(jpa_cat_pad_kernel, dim3(grid), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}
