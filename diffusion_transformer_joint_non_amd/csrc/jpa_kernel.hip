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
//   per lane, no staging registers) into natural [key][d] tiles; the V^T
//   operand is read with the gfx950 LDS transpose load ds_read_b64_tr_b16.
//   XOR swizzles of the 16-byte (K) and 8-byte (V) chunks keep the reads free
//   of bank conflicts.  K and V are triple-buffered; one barrier per tile.
// * Software pipeline inside each wave over 32-key units: the QK^T MFMAs of
//   unit u+1 are issued alongside the exponentials of unit u (second query
//   block), and the PV MFMAs of unit u alongside the row max and the first
//   query block's exponentials of unit u+1.
// * The key loop walks one index space [0, P_b + R_b): a key below P_b is
//   read from the prefix tensor, the rest from the suffix tensor, per row,
//   so the two tensors are never concatenated.  The tile grid is shifted so
//   it ends exactly at P_b + R_b: only the first tile is partial (its head
//   is masked) and no pad slot is ever loaded.
// * Online softmax in the log2 domain, fp32, with a lazy rescale: the running
//   reference max only moves when a tile's max exceeds it by more than 8
//   (so P <= 2^8 and fp32 accumulators are safe), which skips the O rescale
//   on almost every tile.
// * Work items are mapped so that the workgroups resident on one XCD (blocks
//   are dealt round-robin over the 8 XCDs) cover consecutive query tiles of
//   the same head, which then stream the same K/V through that XCD's L2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
constexpr float kTau = 8.0f;                 // lazy-rescale threshold (log2 units)

static_assert(kBM == JPA_BLOCK_M, "host and kernel tile height differ");

// MFMA row i of the score product reads K row pi(i): bits 2 and 3 swapped,
// so that accumulator registers 8t..8t+7 of lane half h hold keys
// 16t + 8h .. 16t + 8h + 7 -- exactly the B operand of the PV product.
__device__ __forceinline__ int perm_k(int i) {
    return (i & 0x13) | ((i & 4) << 1) | ((i & 8) >> 1);
}
// 16-byte chunk swizzle of K rows: the rows perm_k(0..15) read by lanes 0..15
// of a half get 0..15, distinct modulo 8 within each group of 8 lanes.
__device__ __forceinline__ int swz_k(int row) {
    return (row & 3) | (((row >> 3) & 1) << 2) | (((row >> 2) & 1) << 3);
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

__device__ __forceinline__ u32x4_t load16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
}

template <int D>
__global__ __launch_bounds__(kThreads, 1)
void jpa_fwd_kernel(const jpa_kernel_params p) {
    constexpr int kDS = D / 16;              // 16-wide k-steps of QK^T
    constexpr int kDB = D / 32;              // 32-row blocks of O^T
    constexpr int kCH = D / 8;               // 16-byte chunks per K/V row
    constexpr int kTile = kBN * D;           // elements of one K or V tile
    constexpr int kRowsPerOp = 512 / D;      // rows filled by one wave-wide 16 B/lane load
    constexpr int kOpsPerWave = kBN / kRowsPerOp / kWaves;

    // Three K tiles then three V tiles, all [key][d] (96 KB at D = 128).
    __shared__ __attribute__((aligned(16))) uint16_t lds[6 * kTile];

    // ---- work item: XCD-grouped order over (head, row, query tile)
    const int nblk = gridDim.x;
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int per = nblk >> 3, rem = nblk & 7;
    const int item = xcd * per + min(xcd, rem) + (bid >> 3);
    const int hq = item / p.total_tiles;
    const int tile = item - hq * p.total_tiles;
    int b = 0;
    while (b + 1 < p.nrows && p.rows[b + 1].tile_start <= tile) ++b;
    const int q_start = p.rows[b].q_start;
    const int q_slots = p.rows[b].q_slots;
    const int q_real = p.rows[b].q_real;
    const int m0 = (tile - p.rows[b].tile_start) * kBM;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane & 31;                 // query column inside a 32-block
    const int h = lane >> 5;                 // lane half

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
        return;
    }

    const int hk = hq / p.group;
    const int P = p.rows[b].p_len;
    const int Nk = p.rows[b].keys;
    const uint16_t* const kp = p.kp + (int64_t)hk * p.kp_hs;
    const uint16_t* const vp = p.vp + (int64_t)hk * p.vp_hs;
    const uint16_t* const ks = p.ks + (int64_t)hk * p.ks_hs;
    const uint16_t* const vs = p.vs + (int64_t)hk * p.vs_hs;
    // key k < P is prefix token p_row0 + k; key k >= P is suffix slot s_row0 + k
    const int64_t p_row0 = p.rows[b].p_start;
    const int64_t s_row0 = (int64_t)p.rows[b].s_start - P;
    // The key walk is shifted so that the tiles end exactly at Nk: only tile
    // 0 can be partial, and its missing keys are the negative indices.
    const int ntiles = (Nk + kBN - 1) / kBN;
    const int shift = ntiles * kBN - Nk;

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
    // Register classes: Q fragments and the O accumulators live in AGPRs (only
    // MFMAs touch them in the loop); scores live in VGPRs where the softmax
    // VALU work reads them.  Empty asm statements pin the classes.
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int ds = 0; ds < kDS; ++ds) asm("" : "+a"(qf[qb][ds]));

    // ---- global -> LDS tile loads, 16 bytes per lane straight into LDS
    //      (global_load_lds_dwordx4: lane l of a wave lands at base + 16*l).
    //      A wave instruction fills kRowsPerOp consecutive key rows; each lane
    //      fetches the global chunk that belongs at its physical LDS slot,
    //      which realises the XOR swizzles.  Negative keys (the head of tile 0)
    //      re-read key 0; their scores are masked.  No pad slot is touched.
    auto load_tile = [&](int t) {
        const int slot = t % 3;
        uint16_t* kdst = lds + slot * kTile;
        uint16_t* vdst = lds + (3 + slot) * kTile;
#pragma unroll
        for (int i = 0; i < kOpsPerWave; ++i) {
            const int row0 = (wave * kOpsPerWave + i) * kRowsPerOp;
            const int row = row0 + lane / kCH;
            const int pc = lane % kCH;
            const int key = max(t * kBN - shift + row, 0);
            const bool pre = key < P;
            const uint16_t* gk = (pre ? kp + (p_row0 + key) * p.kp_ts : ks + (s_row0 + key) * p.ks_ts) +
                                 ((pc ^ swz_k(row)) & (kCH - 1)) * 8;
            const uint16_t* gv = (pre ? vp + (p_row0 + key) * p.vp_ts : vs + (s_row0 + key) * p.vs_ts) +
                                 ((pc ^ (2 * (row & 3))) & (kCH - 1)) * 8;
            __builtin_amdgcn_global_load_lds(gk, (__attribute__((address_space(3))) void*)(kdst + row0 * D),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds(gv, (__attribute__((address_space(3))) void*)(vdst + row0 * D),
                                             16, 0, 0);
        }
    };

    // ---- per-lane LDS fragment addresses (loop invariant)
    //  K (A operand of S^T = K Q^T): lane (j, h) reads row perm_k(j), 16-byte
    //  chunk 2*ds + h of the [key][d] tile.
    //  V (A operand of O^T = V^T P^T) comes from the [key][d] tile through
    //  ds_read_b64_tr_b16: in each 16-lane group, source lane 4k+q points at
    //  key row (.. + k), features 4q..4q+3 of the group's 16-feature block, and
    //  result lane i receives feature i of those 4 keys.  Two such reads give
    //  a lane the 8 consecutive keys 16t + 8h .. +7 of one feature column.
    const int krow = perm_k(j);
    int k_off[kDS];
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds)
        k_off[ds] = krow * D + (((2 * ds + h) ^ swz_k(krow)) & (kCH - 1)) * 8;
    const int tr_k = (lane & 15) >> 2;       // key offset supplied by this lane
    const int tr_q = lane & 3;               // 4-feature group supplied by this lane
    const int tr_half = (lane >> 4) & 1;     // which 16 features of the 32-block
    const int v_row = (8 * h + tr_k) * D;
    int v_col[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db)
        v_col[db] = (((8 * db + 4 * tr_half + tr_q) ^ (4 * tr_k)) & (D / 4 - 1)) * 4;

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

    // One "unit" = 32 keys of a tile (kb = 0 or 1).
    // S^T = K Q^T for one unit, both query blocks (each K fragment feeds two MFMAs)
    auto qk = [&](f32x16_t (&s)[kQB], int t, int kb) {
        const uint16_t* base = lds + (t % 3) * kTile + kb * 32 * D;
#pragma unroll
        for (int ds = 0; ds < kDS; ++ds) {
            const bf16x8_t kf = __builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const u32x4_t*>(base + k_off[ds]));
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb)
                s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ds],
                                                                ds == 0 ? f32x16_t{} : s[qb], 0, 0, 0);
        }
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) asm("" : "+v"(s[qb]));
    };
    // O^T += V^T P^T for one unit (each V fragment feeds two MFMAs)
    auto pv = [&](int t, int kb, const bf16x8_t (&p0)[2], const bf16x8_t (&p1)[2]) {
        const uint16_t* base = lds + (3 + t % 3) * kTile + kb * 32 * D + v_row;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint16_t* a = base + 16 * u * D + v_col[db];
                const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4_t*)(a));
                const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4_t*)(a + 4 * D));
                const bf16x8_t vf = __builtin_bit_cast(
                    bf16x8_t, s16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
                o[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p0[u], o[0][db], 0, 0, 0);
                o[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p1[u], o[1][db], 0, 0, 0);
            }
    };
    // Scores of negative keys (head of tile 0) -> -FLT_MAX.  A finite value
    // keeps a fully masked unit NaN-free: its weights underflow to 0.
    auto mask_head = [&](f32x16_t (&s)[kQB], int kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const bool dead = kb * 32 + perm_k(8 * (r >> 2) + 4 * h + (r & 3)) < shift;
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) s[qb][r] = dead ? -3.402823466e38f : s[qb][r];
        }
    };
    // Move the reference max of each query block when the unit's max exceeds
    // it by more than kTau (log2 units); returns whether any lane moved.
    auto update_ref = [&](const f32x16_t (&s)[kQB], float (&alpha)[kQB]) {
        bool any = false;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            float mx = s[qb][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[qb][r]);
            const float mt = fmaxf(other_half_max(mx) * c, -1e30f);
            const bool need = mt > m_ref[qb] + kTau;
            const float mn = need ? mt : m_ref[qb];
            alpha[qb] = __builtin_amdgcn_exp2f(m_ref[qb] - mn);
            m_ref[qb] = mn;
            any |= need;
        }
        return __builtin_amdgcn_ballot_w64(any) != 0;
    };
    auto rescale = [&](const float (&alpha)[kQB]) {
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            l_sum[qb] *= alpha[qb];
#pragma unroll
            for (int db = 0; db < kDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha[qb];
        }
    };
    // P = 2^(S*c - m) for one query block of a unit, as two bf16 B-operand
    // fragments (keys 16u + 8h .. +7); returns the fp32 sum of the weights
    // (unrounded, so the LSE does not carry the bf16 rounding of P).
    auto exp_pack = [&](const f32x16_t& s, float m, bf16x8_t (&pf)[2]) {
        float lsum = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            uint32_t pk[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int r0 = 8 * u + 2 * w;
                const float e0 = __builtin_amdgcn_exp2f(fmaf(s[r0], c, -m));
                const float e1 = __builtin_amdgcn_exp2f(fmaf(s[r0 + 1], c, -m));
                pk[w] = pack_bf16(e0, e1);
                lsum += e0 + e1;
            }
            pf[u] = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
        }
        return lsum;
    };

    // ---- prologue: tiles 0 and 1 into LDS; scores, reference max and the
    //      first query block's weights of unit (0, 0).
    f32x16_t sA[kQB], sB[kQB];
    bf16x8_t pA0[2], pB0[2], p1[2];
    load_tile(0);
    if (ntiles > 1) load_tile(1);
    __syncthreads();
    qk(sA, 0, 0);
    mask_head(sA, 0);
    {
        float alpha[kQB];
        update_ref(sA, alpha);               // O and l are still zero
        l_sum[0] = exp_pack(sA[0], m_ref[0], pA0);
    }

    // ---- steady state, per tile t (two units):
    //   unit (t,0)  X: QK of unit (t,1)    || weights of (t,0), query block 1
    //               Y: PV of unit (t,0)    || max of (t,1), reference update,
    //                                          weights of (t,1), query block 0
    //   unit (t,1)  X: QK of unit (t+1,0)  || weights of (t,1), query block 1
    //               Y: PV of unit (t,1)    || max of (t+1,0), reference update,
    //                                          weights of (t+1,0), query block 0
    //   Tile t+2 is fetched at the start, one barrier at the end.  On the last
    //   tile the look-ahead re-reads unit (t,0) (already counted, so it can
    //   never move the reference) and its weights are dropped.
    auto body = [&](int t, auto first) {
        if (t + 2 < ntiles) load_tile(t + 2);
        float alpha[kQB];
        // unit (t,0)
        qk(sB, t, 1);
        l_sum[1] += exp_pack(sA[1], m_ref[1], p1);
        if constexpr (decltype(first)::value) mask_head(sB, 1);
        pv(t, 0, pA0, p1);
        {
            const bool any = update_ref(sB, alpha);
            float ts0 = exp_pack(sB[0], m_ref[0], pB0);
            asm volatile("" : "+v"(ts0), "+v"(pB0[0]), "+v"(pB0[1]));   // computed here, not after the branch
            if (any) rescale(alpha);
            l_sum[0] += ts0;
        }
        // unit (t,1)
        const bool last = t + 1 == ntiles;
        qk(sA, last ? t : t + 1, 0);
        l_sum[1] += exp_pack(sB[1], m_ref[1], p1);
        pv(t, 1, pB0, p1);
        {
            const bool any = update_ref(sA, alpha);
            float ts0 = exp_pack(sA[0], m_ref[0], pA0);
            asm volatile("" : "+v"(ts0), "+v"(pA0[0]), "+v"(pA0[1]));
            if (any) rescale(alpha);
            l_sum[0] += last ? 0.f : ts0;
        }
        __syncthreads();
    };
    body(0, std::true_type{});
    for (int t = 1; t < ntiles; ++t) body(t, std::false_type{});

    // ---- epilogue: normalise, bf16 round-to-nearest-even, pad rows as zeros.
    //      O^T accumulator register r of lane half h is feature
    //      32*db + 8*(r/4) + 4*h + r%4.
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int qi = m0 + wave * (kQB * 32) + qb * 32 + j;
        if (qi >= q_slots) continue;
        const bool real = qi < q_real;
        const float l_tot = other_half_sum(l_sum[qb]);
        const float inv = 1.0f / l_tot;
        uint16_t* dst = out_h + (int64_t)(q_start + qi) * p.o_ts + 4 * h;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2_t w = {pack_bf16(o[qb][db][4 * g] * inv, o[qb][db][4 * g + 1] * inv),
                             pack_bf16(o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv)};
                if (!real) w = u32x2_t{0u, 0u};             // pad row: +0.0
                *reinterpret_cast<u32x2_t*>(dst + 32 * db + 8 * g) = w;
            }
        if (p.lse && h == 0)
            p.lse[(int64_t)hq * p.lse_ld + q_start + qi] =
                real ? (m_ref[qb] + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
}

}  // namespace

int jpa_launch_kernel(const jpa_kernel_params& p, int head_dim, void* stream) {
    const int blocks = p.total_tiles * p.hq;
    if (blocks == 0) return (int)hipSuccess;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (head_dim == 128)
        hipLaunchKernelGGL(jpa_fwd_kernel<128>, dim3(blocks), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL(jpa_fwd_kernel<64>, dim3(blocks), dim3(kThreads), 0, s, p);
    return (int)hipGetLastError();
}
