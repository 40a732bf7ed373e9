// gfx950 (CDNA4) kernel: split prefix/suffix K/V, tail-pad-skipping,
// non-causal attention forward with LSE.
//
// What it computes is fixed by the pages (sglang PR #26973 review: attention
// over [prefix ; suffix] keys, prefix first; sglang PR #30107 review,
// implementation item 4: each row is [valid | pad] and the pad segment is
// skipped with no mask and no repacking; vLLM-Omni performance-patterns guide:
// non-causal, BSND, scale head_dim**-0.5, Hq a multiple of Hkv).  How it is
// computed is this file's own design for gfx950:
//
// * One workgroup = 4 wave64s = 256 query rows of one (batch row, query head);
//   each wave owns 64 queries as two 32-query MFMA column blocks.
// * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//   a lane then holds one query and 16 keys per 32x32 block, so the row max
//   and row sum are in-lane reductions plus one exchange between the two
//   32-lane halves (v_permlane32_swap).
// * The K rows feeding MFMA row i are permuted (bits 2 and 3 of i swapped) so
//   that the accumulator registers of a lane, read eight at a time, are eight
//   consecutive keys: they become the bf16 B operand of O^T += V^T P^T with
//   no data movement.
// * K and V tiles are copied global -> LDS by direct-to-LDS loads (16 bytes
//   per lane, no staging registers) into [key][d] tiles laid out as 1 KB
//   blocks of rows with a 16-byte pad after each block; the V^T operand is
//   read with the gfx950 LDS transpose load ds_read_b64_tr_b16.  XOR
//   swizzles of the 16-byte chunks keep the reads free of bank conflicts,
//   and because the pad shifts each block by one bank group, a wave's
//   copies of one tensor in one tile share one per-lane offset and one m0.
//   Four K and four V tile buffers, each its own LDS array: tile t+3 is
//   fetched while tile t is computed (its loads issued from the MFMA slots),
//   and the per-tile barrier leaves only that newest copy in flight.
// * Software pipeline inside each wave over 32-key units: the QK^T MFMAs of
//   unit u+1 are issued alongside the weights of unit u (second query
//   block), and the PV MFMAs of unit u alongside the first query block's
//   weights of unit u+1, one score register per MFMA slot.
// * Keys are walked in 64-key tiles drawn from both tensors, per row, so the
//   two tensors are never concatenated and no pad slot is ever loaded.  The
//   order of keys is free (the attention is non-causal): the P_b mod 64
//   first prefix keys and the R_b mod 64 last real suffix keys go first, in
//   one or two mixed tiles (only the first one partial, its tail masked),
//   then every full 64-key tile of the prefix, then of the suffix.  So every
//   tile inside the loop is a full run of 64 consecutive rows of one tensor.
// * Online softmax in the log2 domain, fp32, with a lazy rescale: weights
//   are formed against a running reference without computing the unit's max;
//   only when a lane's partial sum exceeds 2^8 does the wave move the
//   reference to the unit's max, rescale O and form the weights again (so
//   P <= 2^8 and the fp32 accumulators are safe).  The common path has no
//   row max at all and almost never rescales.
// * Work items are mapped so that the workgroups resident on one XCD (blocks
//   are dealt round-robin over the 8 XCDs) cover consecutive query tiles of
//   the same head, which then stream the same K/V through that XCD's L2.
// * Optional balanced last round: when the item count leaves the last round
//   of workgroups mostly idle, the items of that round are laid end to end
//   as a run of key tiles and cut into one equal range per workgroup.  A
//   range that covers an item whole writes it directly; pieces of an item
//   write fp32 O, row sum and log2 LSE to a workspace, and a second small
//   kernel on the same stream merges each split item's (at most a few)
//   pieces in key order.  No cross-workgroup synchronisation inside a launch.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>
#include <utility>

#include "jpa_params.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQB = 2;                       // 32-query blocks per wave
constexpr int kBM = kWaves * kQB * 32;       // query rows per workgroup
constexpr int kBN = 64;                      // keys per tile
constexpr int kKB = kBN / 32;                // 32-key blocks per tile
constexpr float kBound = 256.0f;             // largest weight let into the PV product (2^8)

static_assert(kBM == JPA_BLOCK_M, "host and kernel tile height differ");

// MFMA row i of the score product reads K row pi(i): bits 2 and 3 swapped,
// so that accumulator registers 8t..8t+7 of lane half h hold keys
// 16t + 8h .. 16t + 8h + 7 -- exactly the B operand of the PV product.
__device__ __forceinline__ int perm_k(int i) {
    return (i & 0x13) | ((i & 4) << 1) | ((i & 8) >> 1);
}
// LDS tile layout.  A K or V tile is copied by wave-wide 16-byte-per-lane
// loads, each filling one block of 512 / D consecutive key rows (1 KB); the
// blocks sit kBlockPad elements (16 bytes) apart.  The pad moves each block
// by one 16-byte bank group, so a chunk's bank group is (block + position)
// mod 16, and the swizzle below only has to separate the rows inside one
// block.  That keeps a lane's copy offsets the same for every block of a
// tile: one voffset and one m0 per tensor and tile, the blocks told apart by
// the instruction offset (LDS) and the scalar offset (global memory).
constexpr int kBlockPad = 8;
template <int D>
__host__ __device__ constexpr int row_elems(int r) {      // element offset of tile row r
    constexpr int kRowsPerBlock = 512 / D;
    return (r / kRowsPerBlock) * (kRowsPerBlock * D + kBlockPad) + (r % kRowsPerBlock) * D;
}
// 16-byte chunk c of K row r sits at position k_pos(c, r) of its LDS row (an
// XOR, so the same function gives the chunk a copy lane fetches for a
// position).  D = 128 (4 rows a block): the row's block position a moves bits
// 2-3 of the position; a read by 16 lanes of 16 rows (4 blocks x 4 positions)
// then lands in 16 distinct bank groups.  D = 64 (8 rows a block): bits 1-2
// by a / 2; the 16 rows of a read (2 blocks, rows of 128 bytes) again fill
// 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int k_pos(int c, int r) {
    constexpr int kRowsPerBlock = 512 / D;
    const int a = r % kRowsPerBlock;
    return (c ^ (D == 128 ? 4 * a : (a & 6))) & (D / 8 - 1);
}

// V tiles: the 16-byte chunk c of key row r sits at chunk v_pos(c, r) of
// its LDS row.  The row term spreads the four rows one transposed read
// touches; for D = 128 the second term also sends the upper 16 features of
// each 32-feature block to the other half of the 256-byte row, so the 32
// lanes an LDS cycle serves hit 32 different 8-byte bank pairs.  Both terms
// are XORs, so the inverse (the chunk a DMA lane fetches for position p) is
// v_chunk_at(p, r).
template <int D>
__device__ __forceinline__ int v_pos(int c, int r) {
    const int kc = D / 8;
    return ((D == 128 ? (c ^ (((c >> 1) & 1) << 3)) : c) ^ (2 * (r & 3))) & (kc - 1);
}
template <int D>
__device__ __forceinline__ int v_chunk_at(int p, int r) {
    const int kc = D / 8;
    const int x = (p ^ (2 * (r & 3))) & (kc - 1);
    return D == 128 ? (x ^ (((x >> 1) & 1) << 3)) : x;
}

__device__ __forceinline__ float other_half_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float other_half_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Compile-time loop: f(std::integral_constant<int, 0>{}) ... f(<N-1>{}).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}
template <int V>
using ic = std::integral_constant<int, V>;

// 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4).  Written as
// inline asm so that the compiler does not track it; the kernel's own
// s_waitcnt vmcnt(N) before each barrier orders it.  m0 holds the LDS base.
__device__ __forceinline__ void lds_copy16(const void* gaddr, const void* lds_dst) {
    const uint32_t m0v = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_dst;
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(gaddr), "{m0}"(m0v) : "memory");
}

// Buffer resource for raw 16-byte loads: base address, no stride, num_records
// bytes in range (lanes at or past it read nothing and write zeros to LDS).
__device__ __forceinline__ u32x4_t make_rsrc(uintptr_t base, uint32_t num_records) {
    return u32x4_t{(uint32_t)base, (uint32_t)(base >> 32) & 0xFFFFu, num_records, 0x00020000u};
}
__device__ __forceinline__ u32x4_t uniform_rsrc(u32x4_t r) {
    return u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane(r[0]), (uint32_t)__builtin_amdgcn_readfirstlane(r[1]),
                   (uint32_t)__builtin_amdgcn_readfirstlane(r[2]), (uint32_t)__builtin_amdgcn_readfirstlane(r[3])};
}
// 16-byte-per-lane buffer -> LDS copies (buffer_load_dwordx4 ... lds);
// untracked like lds_copy16.  Lane l lands at LDS byte m0 + OFF + 16 l and
// reads global memory at base + soff + voff + OFF.  A run of copies shares
// one m0: the first sets it (lds_base + M0OFF, with the wait state a DMA
// needs after an m0 write) and hands it out, the rest take it back in, each
// placed by its own OFF (below 4096) and a soff that subtracts OFF again.
template <int M0OFF>
__device__ __forceinline__ uint32_t lds_copy16_buf_m0(u32x4_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds_base) {
    uint32_t m0_out;
    asm volatile("s_add_u32 m0, %4, %5\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 : "={m0}"(m0_out)
                 : "v"(voff), "s"(uniform_rsrc(rsrc)), "s"(soff), "s"(lds_base), "n"(M0OFF)
                 : "memory", "scc");
    return m0_out;
}
template <int OFF>
__device__ __forceinline__ void lds_copy16_buf_at(u32x4_t rsrc, uint32_t voff, uint32_t soff, uint32_t m0v) {
    static_assert(OFF >= 0 && OFF < 4096, "12-bit instruction offset");
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%4 lds"
                 :: "v"(voff), "s"(uniform_rsrc(rsrc)), "s"(soff), "{m0}"(m0v), "n"(OFF) : "memory");
}

// A wave-uniform 64-bit value in scalar registers.
__device__ __forceinline__ uintptr_t uniform64(uintptr_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((uintptr_t)hi << 32) | lo;
}

__device__ __forceinline__ u32x4_t load16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
}

typedef __attribute__((address_space(3))) uint16_t lds_u16;

// One wave's 64 output rows as bf16.  Register r of o[qb][db] in lane
// (j, h) is row 32*qb + j, feature 32*db + 8*(r/4) + 4*h + r%4; it is scaled
// by scale[qb] and rounded to nearest even.  The fragments go through the
// wave's own LDS region (64 x D bf16, 16-byte chunks XOR-swizzled by row) so
// that every global store writes whole rows, 16 contiguous bytes a lane,
// instead of 8-byte pieces of 32 rows.  Rows at or past n_real are written
// as +0.0, rows at or past n_slots are not written.
template <int D>
__device__ __forceinline__ void store_rows_bf16(const f32x16_t (&o)[kQB][D / 32], const float (&scale)[kQB],
                                                lds_u16* lds, uint16_t* out_row0, int64_t o_ts,
                                                int n_real, int n_slots, int lane) {
    constexpr int kCH = D / 8;               // 16-byte chunks per row
    constexpr int kDB = D / 32;
    constexpr int kRowsPerRead = 64 / kCH;
    const int j = lane & 31, h = lane >> 5;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int row = 32 * qb + j;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = 4 * db + g;
                const u32x2_t w = {pack_bf16(o[qb][db][4 * g] * scale[qb], o[qb][db][4 * g + 1] * scale[qb]),
                                   pack_bf16(o[qb][db][4 * g + 2] * scale[qb], o[qb][db][4 * g + 3] * scale[qb])};
                *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>(
                    lds + row * D + ((c ^ (row & (kCH - 1))) * 8) + 4 * h) = w;
            }
    }
    // the reads below see this wave's own writes (LDS operations of a wave
    // complete in order); the clobber keeps the compiler from moving them
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < kCH; ++i) {
        const int row = i * kRowsPerRead + lane / kCH;
        const int c = lane % kCH;
        u32x4_t v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
            lds + row * D + ((c ^ (row & (kCH - 1))) * 8));
        if (row < n_slots) {
            if (row >= n_real) v = u32x4_t{0u, 0u, 0u, 0u};        // pad row: +0.0
            *reinterpret_cast<u32x4_t*>(out_row0 + (int64_t)row * o_ts + 8 * c) = v;
        }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads, 1)
void jpa_fwd_kernel(const jpa_kernel_params p) {
    constexpr int kDS = D / 16;              // 16-wide k-steps of QK^T
    constexpr int kDB = D / 32;              // 32-row blocks of O^T
    constexpr int kCH = D / 8;               // 16-byte chunks per K/V row
    constexpr int kBlockElems = 512 + kBlockPad;     // one copy block (512 / D rows) and its pad
    constexpr int kTile = kBN / (512 / D) * kBlockElems;   // elements of one K or V tile buffer
    constexpr int kRowsPerOp = 512 / D;      // rows filled by one wave-wide 16 B/lane load
    constexpr int kOpsPerWave = kBN / kRowsPerOp / kWaves;
    constexpr int kXSlots = kDS * kQB;       // QK MFMAs per 32-key unit
    constexpr int kYSlots = kDB * 2 * kQB;   // PV MFMAs per 32-key unit
    static_assert(kYSlots / 2 == 2 * kOpsPerWave, "one copy job per odd Y slot");

    // Barrier that lets the most recent tile prefetch (2*kOpsPerWave loads
    // of this wave) stay in flight: s_waitcnt vmcnt(N) lgkmcnt(0); s_barrier.
    // gfx9 s_waitcnt fields: vmcnt[3:0] bits 3:0, expcnt bits 6:4,
    // lgkmcnt bits 11:8, vmcnt[5:4] bits 15:14.
#ifndef JPA_STRICT_WAITS
    constexpr int kWaitVm = 2 * kOpsPerWave;
#else
    // Check build: every copy, the newest prefetch included, lands before each
    // barrier.  The arithmetic is unchanged, so its results must equal the
    // release build's bit for bit; a difference would mean a tile was read
    // before its copy had landed.
    constexpr int kWaitVm = 0;
#endif
    constexpr int kWaitImm = (kWaitVm & 15) | (7 << 4) | (0 << 8) | ((kWaitVm >> 4) << 14);
    auto tile_barrier = [&]() __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kWaitImm);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // Four K and four V tile buffers.  The tile copies are untracked inline
    // asm, so no compiler-inserted wait depends on how they are laid out.
    static_assert(kBM / kWaves * D <= kTile, "a wave stages its output rows in one K tile buffer");
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[4 * kTile];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[4 * kTile];
    auto kbuf = [&](auto SLOT) __attribute__((always_inline)) -> uint16_t* {
        return lds_k + decltype(SLOT)::value * kTile;
    };
    auto vbuf = [&](auto SLOT) __attribute__((always_inline)) -> uint16_t* {
        return lds_v + decltype(SLOT)::value * kTile;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31;                 // query column inside a 32-block
    const int h = lane >> 5;                 // lane half

    // ---- work split (jpa_kernel_params): per row of the launch, a real query
    //      tile counts its key tiles as units, an all-pad query tile counts 1.
    auto row_counts = [&](int rb, int& nt, int& nr, int& nk) __attribute__((always_inline)) {
        nt = (p.rows[rb].q_slots + kBM - 1) / kBM;
        nr = (p.rows[rb].q_real + kBM - 1) / kBM;
        nk = (p.rows[rb].keys + kBN - 1) / kBN;
    };
    // absolute unit of the first key tile of item it
    auto item_unit = [&](int it) __attribute__((always_inline)) -> int64_t {
        const int hq_ = it / p.total_tiles, tile_ = it - hq_ * p.total_tiles;
        int64_t acc = (int64_t)hq_ * p.head_units;
        for (int rb = 0; rb < p.nrows; ++rb) {
            int nt, nr, nk;
            row_counts(rb, nt, nr, nk);
            const int tr = tile_ - p.rows[rb].tile_start;
            if (tr < nt) {
                acc += tr < nr ? (int64_t)tr * nk : (int64_t)nr * nk + (tr - nr);
                break;
            }
            acc += (int64_t)nr * nk + (nt - nr);
        }
        return acc;
    };
    // item and key-tile offset of absolute unit U
    auto locate = [&](int64_t U, int& it, int& off) __attribute__((always_inline)) {
        const int hq_ = (int)(U / p.head_units);
        int64_t r = U - (int64_t)hq_ * p.head_units;
        it = hq_ * p.total_tiles;
        off = 0;
        for (int rb = 0; rb < p.nrows; ++rb) {
            int nt, nr, nk;
            row_counts(rb, nt, nr, nk);
            const int64_t ru = (int64_t)nr * nk + (nt - nr);
            if (r < ru || rb + 1 == p.nrows) {
                const int64_t realu = (int64_t)nr * nk;
                int tr;
                if (r < realu) {
                    tr = (int)(r / nk);
                    off = (int)(r - (int64_t)tr * nk);
                } else {
                    tr = nr + (int)(r - realu);
                }
                it += p.rows[rb].tile_start + tr;
                break;
            }
            r -= ru;
        }
    };
    // balanced ranges: range w covers tail units [rstart(w), rstart(w + 1))
    auto rstart = [&](int64_t w) __attribute__((always_inline)) -> int64_t {
        return w * p.tail_units / p.sk_wgs;
    };
    // XCD-grouped order: the workgroups resident on one XCD (blocks are dealt
    // round-robin over the 8 XCDs) take consecutive items or ranges, which
    // then stream the same K/V through that XCD's L2.
    auto xcd_order = [&](int l, int n) __attribute__((always_inline)) {
        const int x = l & 7, per = n >> 3, rem = n & 7;
        return x * per + min(x, rem) + (l >> 3);
    };

    const int bid = blockIdx.x;
    const bool dp = bid < p.n_dp;
    int w_me = 0;
    int64_t u_next = 0, u_end = 0;
    if (!dp) {
        w_me = xcd_order(bid - p.n_dp, p.sk_wgs);
        u_next = rstart(w_me);
        u_end = rstart(w_me + 1);
    }
    // ---- one piece per iteration: a whole item, or key tiles [t0, t1) of one
    for (bool first_piece = true;; first_piece = false) {
    int item, t0 = 0;
    if (dp) {
        if (!first_piece) break;
        item = xcd_order(bid, p.n_dp);
    } else {
        if (u_next >= u_end) break;
        locate(p.tail_unit0 + u_next, item, t0);
    }
    if (!first_piece) __syncthreads();      // the previous piece is done with LDS
    const int hq = item / p.total_tiles;
    const int tile = item - hq * p.total_tiles;
    int b = 0;
    while (b + 1 < p.nrows && p.rows[b + 1].tile_start <= tile) ++b;
    const int q_start = p.rows[b].q_start;
    const int q_slots = p.rows[b].q_slots;
    const int q_real = p.rows[b].q_real;
    const int m0 = (tile - p.rows[b].tile_start) * kBM;

    uint16_t* const out_h = p.out + (int64_t)hq * p.o_hs;

    if (m0 >= q_real) {
        // Whole tile is tail pad: zero rows and -inf LSE, nothing is read.
        const int rows = min(kBM, q_slots - m0);
        for (int idx = tid; idx < rows * kCH; idx += kThreads) {
            const int r = idx / kCH, c = idx - r * kCH;
            *reinterpret_cast<u32x4_t*>(out_h + (int64_t)(q_start + m0 + r) * p.o_ts + c * 8) =
                u32x4_t{0u, 0u, 0u, 0u};
        }
        if (p.lse)
            for (int r = tid; r < rows; r += kThreads)
                p.lse[(int64_t)hq * p.lse_ld + q_start + m0 + r] = -INFINITY;
        u_next += 1;
        continue;
    }

    const int hk = hq / p.group;
    const int P = p.rows[b].p_len;
    const int Nk = p.rows[b].keys;
    const uint16_t* const kp = p.kp + (int64_t)hk * p.kp_hs;
    const uint16_t* const vp = p.vp + (int64_t)hk * p.vp_hs;
    const uint16_t* const ks = p.ks + (int64_t)hk * p.ks_hs;
    const uint16_t* const vs = p.vs + (int64_t)hk * p.vs_hs;
    const int R = Nk - P;
    const int64_t p_row0 = p.rows[b].p_start;      // prefix token of prefix key 0
    const int64_t s_row0 = p.rows[b].s_start;      // suffix slot of suffix key 0
    // Token strides as scalars: a per-lane choice between them must select
    // registers, never re-read the kernel arguments per lane.
    int64_t kp_ts = p.kp_ts, ks_ts = p.ks_ts, vp_ts = p.vp_ts, vs_ts = p.vs_ts;
    asm("" : "+s"(kp_ts), "+s"(ks_ts), "+s"(vp_ts), "+s"(vs_ts));
    // Tile order: npart mixed tiles holding the headP = P mod 64 first prefix
    // keys and the tailR = R mod 64 last suffix keys (tile 0 holds n0 of
    // them, the rest masked; tile 1, if any, is full), then Pf full prefix
    // tiles (prefix keys headP + 64i ..), then Rf full suffix tiles.
    const int headP = P & (kBN - 1), Pf = P / kBN;
    const int tailR = R & (kBN - 1), Rf = R / kBN;
    const int X = headP + tailR;
    const int npart = X == 0 ? 0 : (X <= kBN ? 1 : 2);
    const int n0 = npart == 0 ? kBN : (npart == 1 ? X : X - kBN);
    const int ntiles = npart + Pf + Rf;
    // This piece: key tiles [t0, t1); it is the whole item unless cut.
    const int t1 = dp ? ntiles : (int)min((int64_t)ntiles, (int64_t)t0 + (u_end - u_next));
    u_next += t1 - t0;
    const int nt = t1 - t0;
    const bool whole = t0 == 0 && t1 == ntiles;
    const bool mask_first = t0 == 0;           // only absolute tile 0 has masked rows

    // ---- Q fragments (B operand of S^T = K Q^T): lane (j, h) holds
    //      q[row j][16*ds + 8*h .. +7] for every k-step ds.  Rows past the
    //      real queries re-read the last real row (never a pad slot); their
    //      results are discarded.
    bf16x8_t qf[kQB][kDS];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int qi = min(m0 + wave * (kQB * 32) + qb * 32 + j, q_real - 1);
        const uint16_t* src = p.q + (int64_t)(q_start + qi) * p.q_ts + (int64_t)hq * p.q_hs + 8 * h;
#pragma unroll
        for (int ds = 0; ds < kDS; ++ds) qf[qb][ds] = __builtin_bit_cast(bf16x8_t, load16(src + 16 * ds));
    }

    // ---- global -> LDS tile loads, 16 bytes per lane straight into LDS
    //      (lane l of a wave lands at base + 16*l).  A wave instruction (an
    //      "op") fills kRowsPerOp consecutive key rows of the tile; each lane
    //      fetches the global chunk that belongs at its physical LDS slot,
    //      which realises the XOR swizzles.
    //  Mixed tiles (tile 0, maybe tile 1: loaded before the loop): each lane
    //  forms its own row address.  Rows of tile 0 past n0 re-read the first
    //  mixed key; their scores are masked.
    auto dma_op = [&](int t, auto SLOT, int i) __attribute__((always_inline)) {
        const int row0 = (wave * kOpsPerWave + i) * kRowsPerOp;
        const int row = row0 + lane / kCH;
        const int pc = lane % kCH;
        int pi = t == 0 ? row : n0 + row;            // index among the mixed keys
        pi = (t == 0 && row >= n0) ? 0 : pi;
        const bool pre = pi < headP;
        const int64_t tp = p_row0 + pi;
        const int64_t ts = s_row0 + (int64_t)Rf * kBN + (pi - headP);
        const uint16_t* gk = pre ? kp + tp * kp_ts : ks + ts * ks_ts;
        const uint16_t* gv = pre ? vp + tp * vp_ts : vs + ts * vs_ts;
        lds_copy16(gk + k_pos<D>(pc, row) * 8, kbuf(SLOT) + row_elems<D>(row0));
        lds_copy16(gv + v_chunk_at<D>(pc, row) * 8, vbuf(SLOT) + row_elems<D>(row0));
    };
    //  Full tiles: a buffer resource whose base is the tile's row 0 (less
    //  kCopyBias bytes), one per-lane offset per tensor (the lane's row in its
    //  block times the token stride, plus its chunk), and per op a scalar
    //  offset: op i of a wave fills block (wave * kOpsPerWave + i), so its
    //  rows start i * kRowsPerOp rows further on, and it carries the
    //  instruction offset i * kBlockBytes, which the scalar offset takes back
    //  off the global address.  The loop advances the base by 64 rows per
    //  tile and switches tensor once; its look-ahead past the last tile uses
    //  an empty resource (every lane out of range: nothing is read, zeros
    //  land in a buffer nobody reads).
    constexpr int kBlockBytes = 2 * kBlockElems;
    // Keeps every scalar offset non-negative: token strides are at least D
    // elements, so a block's rows span at least 1024 bytes of global memory.
    constexpr uint32_t kCopyBias = 64;
    static_assert((kOpsPerWave - 1) * (kBlockBytes - 1024) <= (int)kCopyBias, "scalar offsets stay non-negative");
    const int lane_row = lane / kCH;
    const int lane_pc = lane % kCH;
    const uint32_t r_lane0 = (uint32_t)(wave * kOpsPerWave * kRowsPerOp + lane_row);   // tile row in op 0
    const uint32_t kch = (uint32_t)k_pos<D>(lane_pc, lane_row) << 4;
    const uint32_t vch = (uint32_t)v_chunk_at<D>(lane_pc, lane_row) << 4;

    uint64_t kbase = 0, vbase = 0;            // K and V tile bases of the current full tile (less the bias)
    uint32_t nrec = 0;                        // records in range (0: the empty look-ahead)
    uint32_t step_k = 0, step_v = 0;          // 64 rows of the current tensor, bytes
    uint32_t kblk = 0, vblk = 0;              // kRowsPerOp rows of the current tensor less kBlockBytes
    uint32_t koff = 0, voff = 0;
    // Point the copy state at full tile t (npart <= t < ntiles).
    auto set_full_tile = [&](int t) __attribute__((always_inline)) {
        const bool suf = t >= npart + Pf;
        const int64_t tp = p_row0 + headP + (int64_t)(t - npart) * kBN;
        const int64_t tsf = s_row0 + (int64_t)(t - npart - Pf) * kBN;
        const uintptr_t kb_p = reinterpret_cast<uintptr_t>(kp) + 2 * tp * kp_ts;
        const uintptr_t kb_s = reinterpret_cast<uintptr_t>(ks) + 2 * tsf * ks_ts;
        const uintptr_t vb_p = reinterpret_cast<uintptr_t>(vp) + 2 * tp * vp_ts;
        const uintptr_t vb_s = reinterpret_cast<uintptr_t>(vs) + 2 * tsf * vs_ts;
        const uint32_t ksb = 2u * (uint32_t)(suf ? ks_ts : kp_ts);
        const uint32_t vsb = 2u * (uint32_t)(suf ? vs_ts : vp_ts);
        kbase = uniform64((suf ? kb_s : kb_p) - kCopyBias);
        vbase = uniform64((suf ? vb_s : vb_p) - kCopyBias);
        nrec = ~0u;
        step_k = __builtin_amdgcn_readfirstlane(ksb * (uint32_t)kBN);
        step_v = __builtin_amdgcn_readfirstlane(vsb * (uint32_t)kBN);
        kblk = __builtin_amdgcn_readfirstlane(ksb * (uint32_t)kRowsPerOp - (uint32_t)kBlockBytes);
        vblk = __builtin_amdgcn_readfirstlane(vsb * (uint32_t)kRowsPerOp - (uint32_t)kBlockBytes);
        koff = __umul24(r_lane0, ksb) + kch;
        voff = __umul24(r_lane0, vsb) + vch;
    };
    // Job J of the copy of the current full tile: K of op J for J below
    // kOpsPerWave, then V of op J - kOpsPerWave.  Each tensor's first op
    // sets m0 to this wave's first block in the tile slot, the others reuse it.
    const uint32_t kdst0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(lds_k + wave * kOpsPerWave * kBlockElems));
    const uint32_t vdst0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(lds_v + wave * kOpsPerWave * kBlockElems));
    uint32_t m0_copy = 0;
    auto fast_job = [&](auto SLOT, auto J) __attribute__((always_inline)) {
        constexpr int j = decltype(J)::value;
        constexpr bool is_k = j < kOpsPerWave;
        constexpr int i = is_k ? j : j - kOpsPerWave;
        constexpr int slot_off = decltype(SLOT)::value * kTile * 2;
        const u32x4_t rs = make_rsrc(is_k ? kbase : vbase, nrec);
        const uint32_t soff = kCopyBias + (uint32_t)i * (is_k ? kblk : vblk);
        if constexpr (i == 0)
            m0_copy = lds_copy16_buf_m0<slot_off>(rs, is_k ? koff : voff, soff, is_k ? kdst0 : vdst0);
        else
            lds_copy16_buf_at<i * kBlockBytes>(rs, is_k ? koff : voff, soff, m0_copy);
    };
    // Whole-tile copy issued at once (before the loop).
    auto dma_tile_now = [&](int t, auto SLOT) __attribute__((always_inline)) {
        if (t < npart) {
#pragma unroll
            for (int i = 0; i < kOpsPerWave; ++i) dma_op(t, SLOT, i);
        } else {
            set_full_tile(t);
            static_for<2 * kOpsPerWave>([&](auto J) __attribute__((always_inline)) { fast_job(SLOT, J); });
        }
    };

    // ---- per-lane LDS fragment addresses (loop invariant; the tile slot and
    //      the unit enter as immediate offsets)
    //  K (A operand of S^T = K Q^T): lane (j, h) reads row perm_k(j), 16-byte
    //  chunk 2*ds + h of the [key][d] tile.
    //  V (A operand of O^T = V^T P^T) comes from the [key][d] tile through
    //  ds_read_b64_tr_b16: in each 16-lane group, source lane 4k+q points at
    //  key row (.. + k), features 4q..4q+3 of the group's 16-feature block, and
    //  result lane i receives feature i of those 4 keys.  Two such reads give
    //  a lane the 8 consecutive keys 16u + 8h .. +7 of one feature column.
    const int krow = perm_k(j);
    int k_lane[kDS];
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds)
        k_lane[ds] = row_elems<D>(krow) + k_pos<D>(2 * ds + h, krow) * 8;
    const int tr_k = (lane & 15) >> 2;       // key offset supplied by this lane
    const int tr_q = lane & 3;               // 4-feature group supplied by this lane
    const int tr_half = (lane >> 4) & 1;     // which 16 features of the 32-block
    int v_lane[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db)
        v_lane[db] = row_elems<D>(8 * h + tr_k) +
                     (2 * v_pos<D>(4 * db + 2 * tr_half + (tr_q >> 1), 8 * h + tr_k) + (tr_q & 1)) * 4;

    auto read_k = [&](auto SLOT, auto KB, int ds) __attribute__((always_inline)) {
        constexpr int off = row_elems<D>(decltype(KB)::value * 32);
        return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(kbuf(SLOT) + k_lane[ds] + off));
    };

    f32x16_t o[kQB][kDB];
    float m_ref[kQB], l_sum[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        m_ref[qb] = -INFINITY;
        l_sum[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.f;
            asm("" : "+a"(o[qb][db]));
        }
    }
    const float c = p.c;

    // Scores of the unused rows of tile 0 (at or past n0) -> -FLT_MAX.  A
    // finite value keeps a fully masked unit NaN-free: its weights are 0.
    auto mask_head = [&](f32x16_t (&s)[kQB], int kb) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const bool dead = kb * 32 + perm_k(8 * (r >> 2) + 4 * h + (r & 3)) >= n0;
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) s[qb][r] = dead ? -3.402823466e38f : s[qb][r];
        }
    };
    // Row max of one query block over one 32-key unit (both lane halves), in
    // log2 units, floored at -1e30 so that a fully masked unit stays finite.
    auto unit_max = [&](const f32x16_t& s) __attribute__((always_inline)) {
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
        return fmaxf(other_half_max(mx) * c, -1e30f);
    };
    // Weights 2^(S*c - m) of one query block in one unit, one accumulator
    // register per step so that they spread evenly over the MFMA slots: step
    // r forms weight r, adds weight r-1 to the lane's partial sum (fp32, of
    // the unrounded weights: LSE precision) and, every second step, packs two
    // weights to bf16 for the PV product.
    struct Weights {
        float e[16];
        float part;
        uint32_t pk[8];
    };
    auto w_step = [&](const f32x16_t& s, float m, Weights& w, auto R) __attribute__((always_inline)) {
        constexpr int r = decltype(R)::value;
        w.e[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -m));
        if constexpr (r == 1) w.part = w.e[0];
        if constexpr (r >= 2) w.part += w.e[r - 1];
        if constexpr (r >= 2 && (r & 1) == 0) w.pk[r / 2 - 1] = pack_bf16(w.e[r - 2], w.e[r - 1]);
    };
    auto w_tail = [&](Weights& w) __attribute__((always_inline)) {
        w.part += w.e[15];
        w.pk[7] = pack_bf16(w.e[14], w.e[15]);
    };
    auto w_all = [&](const f32x16_t& s, float m, Weights& w) __attribute__((always_inline)) {
        static_for<16>([&](auto R) __attribute__((always_inline)) { w_step(s, m, w, R); });
        w_tail(w);
    };
    auto pack_frags = [&](const uint32_t (&pk)[8], bf16x8_t (&pf)[2]) __attribute__((always_inline)) {
        pf[0] = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
        pf[1] = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[4], pk[5], pk[6], pk[7]});
    };
    // Lazy rescale.  Weights are formed against the running reference m_ref
    // without looking at the unit's max first; only when some lane's partial
    // sum exceeds 2^8 (a weight may then exceed 2^8, or be inf) does the wave
    // move the reference up to the unit's max, rescale that block's O and l,
    // and form the weights again.  So every weight that reaches the PV
    // product is <= 2^8, and m_ref stays within 8 (log2 units) of the running
    // max.  Then the lane sum is added to l.
    auto settle = [&](auto QB, const f32x16_t& s, Weights& w, bool valid) __attribute__((always_inline)) {
        constexpr int qb = decltype(QB)::value;
        // the common-path weights are formed before the branch, in the slots
        asm volatile("" : "+v"(w.part), "+v"(w.pk[0]), "+v"(w.pk[1]), "+v"(w.pk[2]), "+v"(w.pk[3]),
                     "+v"(w.pk[4]), "+v"(w.pk[5]), "+v"(w.pk[6]), "+v"(w.pk[7]));
        if (__builtin_amdgcn_ballot_w64(valid && w.part > kBound) != 0) {
            const float mn = fmaxf(m_ref[qb], unit_max(s));
            const float alpha = __builtin_amdgcn_exp2f(m_ref[qb] - mn);
            m_ref[qb] = mn;
            l_sum[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < kDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
            w_all(s, mn, w);
        }
        l_sum[qb] += valid ? w.part : 0.f;
    };

    // ---- One 32-key unit as a hand-placed instruction schedule.  Each slot
    //      holds one MFMA (32 cycles on the matrix core) and a few VALU or LDS
    //      instructions that issue while it runs; sched_barrier keeps the slots
    //      apart.
    //  X slots: QK^T MFMAs of the next unit (K tile KSN, half KBN) -> sn, with
    //           the weights of the current unit's second query block.
    //  Y slots: PV MFMAs of the current unit (V tile VS, half KBC), with the
    //           weights of the next unit's first query block, the K reads of
    //           the next X phase and, in the first unit of a tile, the copy of
    //           a later tile.
    // LDS fragments are read one phase ahead: the K fragments of an X phase
    // during the Y phase before it (kq), the V fragments of a Y phase during
    // the X phase before it (one transposed read per slot).  Each phase then
    // waits twice on lgkmcnt (LDS reads complete in order), each time for
    // reads issued at least half a phase earlier.
    bf16x8_t kq[kDS];
    auto lgkm_wait = [&](auto N) __attribute__((always_inline)) {
        constexpr int n = decltype(N)::value;
        static_assert(n >= 0 && n < 16, "lgkmcnt field is 4 bits");
        __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (n << 8) | (3 << 14));
    };
    auto read_v_half = [&](auto SLOT, auto KB, int f, int half) __attribute__((always_inline)) {
        const int db = f / 2, u = f % 2;
        // rows 8h + tr_k (in v_lane) plus 32 KB + 16 u + 4 half: the two
        // parts never carry across a copy block, so their offsets add
        const uint16_t* a = vbuf(SLOT) + v_lane[db] + row_elems<D>(decltype(KB)::value * 32 + 16 * u + 4 * half);
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(a));
    };
    // End of an MFMA slot: its instructions issue as the MFMA, then its LDS
    // read, then the VALU work (sched_group_barrier masks 0x8 MFMA, 0x100 LDS
    // read, 0x2 VALU), and nothing crosses into the next slot.  Measured
    // 0.5-1% faster than leaving the order within a slot to the scheduler,
    // and 3-4% faster than putting the LDS read first.
    auto slot_end = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto unit = [&](auto KSN, auto KBN, auto VS, auto KBC, auto KSNN, auto KBNN,
                    f32x16_t (&sc)[kQB], f32x16_t (&sn)[kQB], const bf16x8_t (&pc0)[2],
                    bf16x8_t (&pn0)[2], bool valid_next, auto MASK_NEXT, auto&& jobs) __attribute__((always_inline)) {
        constexpr int kVF = kDB * 2;                 // V fragments per unit (two reads each)
        static_assert(2 * kVF == kXSlots, "one transposed V read per X slot");
        static_assert(kYSlots == 2 * kDS, "one K read per two Y slots");
        s16x4_t vlo[kVF], vhi[kVF];
        Weights w1;
        // X phase
        static_for<kXSlots>([&](auto I) __attribute__((always_inline)) {
            constexpr int i = decltype(I)::value;
            constexpr int ds = i / kQB, qb = i % kQB;
            if constexpr (i == 0) lgkm_wait(ic<kDS / 2>{});            // kq[0, kDS/2)
            if constexpr (i == kXSlots / 2) lgkm_wait(ic<kXSlots / 2>{});  // rest of kq
            sn[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[ds], qf[qb][ds],
                                                             ds == 0 ? f32x16_t{} : sn[qb], 0, 0, 0);
            static_for<16>([&](auto R) __attribute__((always_inline)) {
                if constexpr (decltype(R)::value * kXSlots / 16 == i) w_step(sc[1], m_ref[1], w1, R);
            });
            if constexpr (i % 2 == 0) vlo[i / 2] = read_v_half(VS, KBC, i / 2, 0);
            else vhi[i / 2] = read_v_half(VS, KBC, i / 2, 1);
            slot_end();
        });
        w_tail(w1);
        settle(ic<1>{}, sc[1], w1, true);
        bf16x8_t p1[2];
        pack_frags(w1.pk, p1);
        // Y phase
        Weights w0;
        static_for<kYSlots>([&](auto I) __attribute__((always_inline)) {
            constexpr int i = decltype(I)::value;
            constexpr int step = i / kQB, qb = i % kQB;     // step = (db, u) = V fragment
            constexpr int db = step / 2, u = step % 2;
            if constexpr (i == 0) lgkm_wait(ic<kXSlots / 2>{});            // V fragments [0, kVF/2)
            if constexpr (i == kYSlots / 2) lgkm_wait(ic<kDS / 2>{});      // the rest of V
            const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, s16x8_t{
                vlo[step][0], vlo[step][1], vlo[step][2], vlo[step][3],
                vhi[step][0], vhi[step][1], vhi[step][2], vhi[step][3]});
            o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, qb == 0 ? pc0[u] : p1[u], o[qb][db], 0, 0, 0);
            if constexpr (i == 0 && decltype(MASK_NEXT)::value) {
                if (mask_first) mask_head(sn, decltype(KBN)::value);
            }
            static_for<16>([&](auto R) __attribute__((always_inline)) {
                if constexpr (decltype(R)::value * kYSlots / 16 == i) w_step(sn[0], m_ref[0], w0, R);
            });
            if constexpr (i % 2 == 0) kq[i / 2] = read_k(KSNN, KBNN, i / 2);
            else jobs(ic<i / 2>{});                  // next-tile copy (first unit of a tile)
            slot_end();
        });
        w_tail(w0);
        settle(ic<0>{}, sn[0], w0, valid_next);
        pack_frags(w0.pk, pn0);
    };

    // ---- prologue: the piece's tiles t0..t0+2 into LDS; scores, reference
    //      max and the first query block's weights of its first unit.
    f32x16_t sA[kQB], sB[kQB];
    bf16x8_t pA0[2], pB0[2];
    dma_tile_now(t0, ic<0>{});
    dma_tile_now(t0 + min(1, nt - 1), ic<1>{});
    dma_tile_now(t0 + min(2, nt - 1), ic<2>{});
    // Register classes: Q fragments and the O accumulators live in AGPRs (only
    // MFMAs touch them in the loop); the softmax VALU work uses VGPRs.  Pinned
    // only here, after the tile copies are issued: the pin waits for the Q
    // loads, and the copies then travel alongside them.
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int ds = 0; ds < kDS; ++ds) asm("" : "+a"(qf[qb][ds]));
    // tiles 0 and 1 must have landed; tile 2 may still be in flight
    tile_barrier();
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds) {
        const bf16x8_t kf = read_k(ic<0>{}, ic<0>{}, ds);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
            sA[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ds], ds == 0 ? f32x16_t{} : sA[qb], 0, 0, 0);
    }
    if (mask_first) mask_head(sA, 0);
    m_ref[0] = unit_max(sA[0]);
    m_ref[1] = unit_max(sA[1]);
    {
        Weights w0;
        w_all(sA[0], m_ref[0], w0);          // every weight <= 1 here
        pack_frags(w0.pk, pA0);
        l_sum[0] = w0.part;
    }
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds) kq[ds] = read_k(ic<0>{}, ic<1>{}, ds);

    // ---- one 64-key tile (the piece's r-th) in buffer S (of 4): units (r,0)
    //      and (r,1); tile r+3 is fetched into buffer S+3 meanwhile.  On the
    //      last tile the look-ahead of unit (r,1) reads a stale buffer; its
    //      reference update is suppressed and its weights are never used.
    auto body = [&](int r, auto S, auto FIRST) __attribute__((always_inline)) {
        constexpr int s = decltype(S)::value;
        constexpr int s1 = (s + 1) % 4, s3 = (s + 3) % 4;
        // Copy state for tile r+3 (never tile 0, so a full tile): advance 64
        // rows, or switch to the suffix, or an empty resource past the end.
        const int tt = t0 + r + 3;
        if (r + 3 >= nt) {
            nrec = 0u;
        } else if (tt == npart + Pf) {
            set_full_tile(tt);
        } else {
            kbase += step_k;
            vbase += step_v;
        }
        auto copy_jobs = [&](auto J) __attribute__((always_inline)) { fast_job(ic<s3>{}, J); };
        auto no_jobs = [&](auto J) __attribute__((always_inline)) {};
        unit(ic<s>{}, ic<1>{}, ic<s>{}, ic<0>{}, ic<s1>{}, ic<0>{}, sA, sB, pA0, pB0, true, FIRST,
             copy_jobs);
        unit(ic<s1>{}, ic<0>{}, ic<s>{}, ic<1>{}, ic<s1>{}, ic<1>{}, sB, sA, pB0, pA0,
             r + 1 < nt, std::false_type{}, no_jobs);
        // Tiles up to r+2 must have landed before the barrier (tile r+2 is
        // first read in the next tile); this tile's own prefetch (r+3, the
        // last kOpsPerWave*2 loads) may stay in flight.
        tile_barrier();
    };
    body(0, ic<0>{}, std::true_type{});
    int r = 1;
    for (; r + 4 <= nt; r += 4) {
        body(r, ic<1>{}, std::false_type{});
        body(r + 1, ic<2>{}, std::false_type{});
        body(r + 2, ic<3>{}, std::false_type{});
        body(r + 3, ic<0>{}, std::false_type{});
    }
    if (r < nt) body(r++, ic<1>{}, std::false_type{});
    if (r < nt) body(r++, ic<2>{}, std::false_type{});
    if (r < nt) body(r++, ic<3>{}, std::false_type{});
    // No tile copy may still be landing in LDS when the wave ends.
    __builtin_amdgcn_s_waitcnt(0);

    // ---- epilogue of a whole item: normalise, bf16 round-to-nearest-even,
    //      pad rows as zeros, rows written whole through LDS (every wave is
    //      done with the K/V tiles after the barrier; wave w uses K buffer w).
    if (whole) {
        __syncthreads();
        const int r0 = m0 + wave * (kQB * 32);
        float l_tot[kQB], inv[kQB];
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            l_tot[qb] = other_half_sum(l_sum[qb]);
            inv[qb] = 1.0f / l_tot[qb];
        }
        store_rows_bf16<D>(o, inv, (lds_u16*)(lds_k + wave * kTile), out_h + (int64_t)(q_start + r0) * p.o_ts,
                           p.o_ts, q_real - r0, q_slots - r0, lane);
        if (p.lse && h == 0) {
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) {
                const int qi = r0 + qb * 32 + j;
                if (qi < q_slots)
                    p.lse[(int64_t)hq * p.lse_ld + q_start + qi] =
                        qi < q_real ? (m_ref[qb] + __builtin_amdgcn_logf(l_tot[qb])) * 0.69314718055994531f
                                    : -INFINITY;
            }
        }
        continue;
    }

    // ---- a piece of a cut item: its O / l (fp32) and LSE (log2 units) go to
    //      the piece's workspace slot (slot 2w when it is the first piece of
    //      range w, else 2w + 1); jpa_merge_kernel combines them afterwards.
    //      O is kept in fragment order, float4 (qb, db, g) of lane l at
    //      ((qb * kDB + db) * 4 + g) * 64 + l of the wave's part: each store
    //      writes 1 KB contiguous.
    {
        const int64_t A = item_unit(item) - p.tail_unit0;       // first tail unit of the item
        const int slot = A <= rstart(w_me) ? 2 * w_me : 2 * w_me + 1;
        float* const so = p.ws_o + (size_t)slot * kBM * D + (size_t)wave * (kQB * 32) * D;
        float* const sl = p.ws_lse + (size_t)slot * kBM + wave * (kQB * 32);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            const float l_tot = other_half_sum(l_sum[qb]);
            const float inv = 1.0f / l_tot;
#pragma unroll
            for (int db = 0; db < kDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<float4*>(so + ((size_t)((qb * kDB + db) * 4 + g) * 64 + lane) * 4) =
                        make_float4(o[qb][db][4 * g] * inv, o[qb][db][4 * g + 1] * inv,
                                    o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv);
            if (h == 0) sl[qb * 32 + j] = m_ref[qb] + __builtin_amdgcn_logf(l_tot);
        }
    }
    }   // pieces
}

// Merge of the cut items: one workgroup per (item of the split part of the
// launch, items n_dp .., 64-row block of that item = one wave of
// jpa_fwd_kernel); its D/32 waves take one 32-feature block each, lanes
// holding the same rows and features as in jpa_fwd_kernel.  The pieces of an
// item are those of ranges w_first .. w_last (a piece is slot 2w when it is
// the first piece of range w, else 2w + 1; only range w_first's piece can be
// a second one); they are combined with the log-sum-exp merge of softmax
// partials:
//   lse = log2 sum_k 2^lse_k,  out = sum_k 2^(lse_k - lse) * O_k,
// kPieceBatch pieces at a time, so that their loads are in flight together
// (a wave walking the pieces one by one waited two memory round trips per
// piece).  Items that no range cut were written by jpa_fwd_kernel and are
// skipped.
constexpr int kPieceBatch = 4;

template <int D>
__global__ __launch_bounds__(2 * D)
void jpa_merge_kernel(const jpa_kernel_params p) {
    constexpr int kDB = D / 32;
    constexpr int kCH = D / 8;
    const int item = p.n_dp + (int)(blockIdx.x / kWaves);
    const int rblk = (int)(blockIdx.x % kWaves);           // 64-row block of the item
    const int hq = item / p.total_tiles;
    const int tile = item - hq * p.total_tiles;
    int b = 0;
    while (b + 1 < p.nrows && p.rows[b + 1].tile_start <= tile) ++b;
    const int m0 = (tile - p.rows[b].tile_start) * kBM;
    if (m0 >= p.rows[b].q_real) return;              // all-pad item: written directly
    // first tail unit of the item (units: jpa_kernel_params)
    int64_t A = (int64_t)hq * p.head_units;
    for (int rb = 0; rb < p.nrows; ++rb) {
        const int nt = (p.rows[rb].q_slots + kBM - 1) / kBM;
        const int nr = (p.rows[rb].q_real + kBM - 1) / kBM;
        const int nk = (p.rows[rb].keys + kBN - 1) / kBN;
        const int tr = tile - p.rows[rb].tile_start;
        if (tr < nt) {
            A += tr < nr ? (int64_t)tr * nk : (int64_t)nr * nk + (tr - nr);
            break;
        }
        A += (int64_t)nr * nk + (nt - nr);
    }
    A -= p.tail_unit0;
    const int64_t ntiles = (p.rows[b].keys + kBN - 1) / kBN;
    const int64_t skn = p.sk_wgs;
    const int w_first = (int)(((A + 1) * skn - 1) / p.tail_units);
    const int w_last = (int)(((A + ntiles) * skn - 1) / p.tail_units);
    if (w_first == w_last) return;                   // whole item: written directly
    const int s_first = A <= (int64_t)w_first * p.tail_units / skn ? 2 * w_first : 2 * w_first + 1;
    auto slot_of = [&](int w) { return w == w_first ? s_first : 2 * w; };

    __shared__ __attribute__((aligned(16))) uint16_t lds_o[64 * D];
    const int lane = threadIdx.x & 63;
    const int db = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // 32-feature block
    const int j = lane & 31, h = lane >> 5;
    const int rowb = rblk * (kQB * 32);                    // first row of the block within the item
    const int r0 = m0 + rowb;

    // LSE of each row over all pieces, accumulated online
    float mx[kQB], sm[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) { mx[qb] = -INFINITY; sm[qb] = 0.f; }
    for (int w0 = w_first; w0 <= w_last; w0 += kPieceBatch) {
        float l[kPieceBatch][kQB];
#pragma unroll
        for (int k = 0; k < kPieceBatch; ++k)
            if (w0 + k <= w_last) {
                const size_t base = (size_t)slot_of(w0 + k) * kBM + rowb + j;
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) l[k][qb] = p.ws_lse[base + qb * 32];
            }
#pragma unroll
        for (int k = 0; k < kPieceBatch; ++k)
            if (w0 + k <= w_last) {
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) {
                    const float mn = fmaxf(mx[qb], l[k][qb]);
                    sm[qb] = sm[qb] * __builtin_amdgcn_exp2f(mx[qb] - mn) + __builtin_amdgcn_exp2f(l[k][qb] - mn);
                    mx[qb] = mn;
                }
            }
    }
    float lse2[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) lse2[qb] = mx[qb] + __builtin_amdgcn_logf(sm[qb]);

    // weighted sum of the pieces' O for this wave's 32 features
    f32x16_t o[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) o[qb] = f32x16_t{};
    for (int w0 = w_first; w0 <= w_last; w0 += kPieceBatch) {
        float4 x[kPieceBatch][kQB][4];
        float a[kPieceBatch][kQB];
#pragma unroll
        for (int k = 0; k < kPieceBatch; ++k)
            if (w0 + k <= w_last) {
                const int sw = slot_of(w0 + k);
                const float* const so = p.ws_o + (size_t)sw * kBM * D + (size_t)rowb * D;
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) {
                    a[k][qb] = p.ws_lse[(size_t)sw * kBM + rowb + qb * 32 + j];
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        x[k][qb][g] = *reinterpret_cast<const float4*>(
                            so + ((size_t)((qb * kDB + db) * 4 + g) * 64 + lane) * 4);
                }
            }
#pragma unroll
        for (int k = 0; k < kPieceBatch; ++k)
            if (w0 + k <= w_last) {
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) {
                    const float wt = __builtin_amdgcn_exp2f(a[k][qb] - lse2[qb]);
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        o[qb][4 * g] += wt * x[k][qb][g].x;
                        o[qb][4 * g + 1] += wt * x[k][qb][g].y;
                        o[qb][4 * g + 2] += wt * x[k][qb][g].z;
                        o[qb][4 * g + 3] += wt * x[k][qb][g].w;
                    }
                }
            }
    }

    // bf16 rows through LDS (16-byte chunks XOR-swizzled by row, as in
    // store_rows_bf16), then whole 16-byte row chunks to out
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int row = 32 * qb + j;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int c = 4 * db + g;
            const u32x2_t v = {pack_bf16(o[qb][4 * g], o[qb][4 * g + 1]), pack_bf16(o[qb][4 * g + 2], o[qb][4 * g + 3])};
            *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>(
                (lds_u16*)lds_o + row * D + ((c ^ (row & (kCH - 1))) * 8) + 4 * h) = v;
        }
    }
    __syncthreads();
    const int q_start = p.rows[b].q_start, q_real = p.rows[b].q_real, q_slots = p.rows[b].q_slots;
    uint16_t* const out_row0 = p.out + (int64_t)hq * p.o_hs + (int64_t)(q_start + r0) * p.o_ts;
    constexpr int kThreadsM = 64 * kDB;
#pragma unroll
    for (int i = 0; i < 64 * kCH / kThreadsM; ++i) {
        const int id = i * kThreadsM + (int)threadIdx.x;
        const int row = id / kCH, c = id % kCH;
        u32x4_t v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
            (lds_u16*)lds_o + row * D + ((c ^ (row & (kCH - 1))) * 8));
        if (r0 + row < q_slots) {
            if (r0 + row >= q_real) v = u32x4_t{0u, 0u, 0u, 0u};        // pad row: +0.0
            *reinterpret_cast<u32x4_t*>(out_row0 + (int64_t)row * p.o_ts + 8 * c) = v;
        }
    }
    if (p.lse && db == 0 && lane < 32) {
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            const int qi = r0 + qb * 32 + j;
            if (qi < q_slots)
                p.lse[(int64_t)hq * p.lse_ld + q_start + qi] =
                    qi < q_real ? lse2[qb] * 0.69314718055994531f : -INFINITY;
        }
    }
}

}  // namespace

int jpa_launch_kernel(const jpa_kernel_params& p, int head_dim, void* stream) {
    const int blocks = p.n_dp + p.sk_wgs;
    if (blocks == 0) return (int)hipSuccess;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (head_dim == 128)
        hipLaunchKernelGGL(jpa_fwd_kernel<128>, dim3(blocks), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL(jpa_fwd_kernel<64>, dim3(blocks), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.sk_wgs == 0) return (int)e;
    // the items of the split part that ranges cut are merged by a second
    // kernel on the same stream (it sees the partials once the first ends)
    const int tail_items = p.total_tiles * p.hq - p.n_dp;
    if (head_dim == 128)
        hipLaunchKernelGGL(jpa_merge_kernel<128>, dim3(tail_items * kWaves), dim3(2 * 128), 0, s, p);
    else
        hipLaunchKernelGGL(jpa_merge_kernel<64>, dim3(tail_items * kWaves), dim3(2 * 64), 0, s, p);
    return (int)hipGetLastError();
}

// Compute units per device, queried once per device and kept for the life of
// the process (hipGetDevice reads the calling thread's current device).
int jpa_device_cus() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < kMaxDevices && cus > 0) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}
