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
//   no data movement.  The V^T rows feeding that product are permuted the
//   same way so that each lane's accumulator holds 16 consecutive feature
//   columns of one query, written with two 16-byte stores.
// * K tiles sit in LDS as [key][d]; V tiles are transposed on the way in
//   (register byte-permutes) to [d][key] so the PV operand is one 16-byte LDS
//   read per lane.  Both use an XOR swizzle of 16-byte chunks so the eight
//   lanes served together hit eight different bank groups.
// * The key loop walks one index space [0, P_b + R_b): a key below P_b is
//   read from the prefix tensor, the rest from the suffix tensor, per row,
//   so the two tensors are never concatenated and only the very last tile of
//   the walk is partial.  Pad slots are never loaded; out-of-range rows are
//   zero-filled in registers and their scores dropped.
// * Online softmax in the log2 domain, fp32, with a lazy rescale: the running
//   reference max only moves when a tile's max exceeds it by more than 8
//   (so P <= 2^8 and fp32 accumulators are safe), which skips the O rescale
//   on almost every tile.
// * Work items are mapped so that the workgroups resident on one XCD (blocks
//   are dealt round-robin over the 8 XCDs) cover consecutive query tiles of
//   the same head, which then stream the same K/V through that XCD's L2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jpa_params.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQB = 2;                       // 32-query blocks per wave
constexpr int kBM = kWaves * kQB * 32;       // query rows per workgroup
constexpr int kBN = 64;                      // keys per tile
constexpr int kKB = kBN / 32;                // 32-key blocks per tile
constexpr float kTau = 8.0f;                 // lazy-rescale threshold (log2 units)

static_assert(kBM == JPA_BLOCK_M, "host and kernel tile height differ");

// MFMA row i of the score product reads K row pi(i): bits 2 and 3 swapped.
__device__ __forceinline__ int perm_k(int i) {
    return (i & 0x13) | ((i & 4) << 1) | ((i & 8) >> 1);
}
// MFMA row i of the PV product reads V^T row sigma(i): i = b4 b3 b2 b1 b0 ->
// b2 b4 b3 b1 b0, so accumulator register r of lane half h is column 16h + r.
__device__ __forceinline__ int perm_v(int i) {
    return (((i >> 2) & 1) << 4) | (((i >> 3) & 3) << 2) | (i & 3);
}
// Chunk swizzles (16-byte chunks).  For K rows read by lanes 0..15 of a half
// (rows perm_k(0..15)) the swizzle is 0..15, distinct modulo 8 in each group
// of 8 lanes; likewise for V^T rows perm_v(0..7) and perm_v(8..15).
__device__ __forceinline__ int swz_k(int row) {
    return (row & 3) | (((row >> 3) & 1) << 2) | (((row >> 2) & 1) << 3);
}
__device__ __forceinline__ int swz_v(int row) {
    return (row & 3) | (((row >> 4) & 1) << 2);
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
    constexpr int kCH = D / 8;               // 16-byte chunks per K row
    constexpr int kRPP = kThreads / kCH;     // K rows loaded per pass
    constexpr int kNP = kBN / kRPP;          // K load passes per tile
    constexpr int kVCH = kBN / 8;            // 16-byte chunks per V^T row

    __shared__ __attribute__((aligned(16))) uint16_t k_lds[kBN * D];
    __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * kBN];

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

    // ---- Q fragments (B operand of S^T = K Q^T): lane (j, h) holds
    //      q[row j][16*ds + 8*h .. +7] for every k-step ds.
    bf16x8_t qf[kQB][kDS];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int qi = m0 + wave * (kQB * 32) + qb * 32 + j;
        const bool ok = qi < q_real;
        const uint16_t* src = p.q + (int64_t)(q_start + (ok ? qi : 0)) * p.q_ts + (int64_t)hq * p.q_hs + 8 * h;
#pragma unroll
        for (int ds = 0; ds < kDS; ++ds) {
            u32x4_t v = ok ? load16(src + 16 * ds) : u32x4_t{0u, 0u, 0u, 0u};
            qf[qb][ds] = __builtin_bit_cast(bf16x8_t, v);
        }
    }

    // ---- global -> register tile loads
    const int kc = tid % kCH, kr = tid / kCH;          // K: chunk, first row
    const int vq = tid & 15, vdc = tid >> 4;           // V: key quad, d chunk
    const bool v_active = vdc < kCH;
    u32x4_t kreg[kNP];
    u32x4_t vreg[4];

    auto load_tile = [&](int key0) {
#pragma unroll
        for (int i = 0; i < kNP; ++i) {
            const int key = key0 + kr + kRPP * i;
            const uint16_t* row = key < P ? kp + (p_row0 + key) * p.kp_ts : ks + (s_row0 + key) * p.ks_ts;
            kreg[i] = key < Nk ? load16(row + kc * 8) : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = key0 + 4 * vq + r;
            const uint16_t* row = key < P ? vp + (p_row0 + key) * p.vp_ts : vs + (s_row0 + key) * p.vs_ts;
            vreg[r] = (v_active && key < Nk) ? load16(row + vdc * 8) : u32x4_t{0u, 0u, 0u, 0u};
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < kNP; ++i) {
            const int row = kr + kRPP * i;
            const int chunk = (kc ^ swz_k(row)) & (kCH - 1);
            *reinterpret_cast<u32x4_t*>(k_lds + row * D + chunk * 8) = kreg[i];
        }
        if (v_active) {
            // 4 keys x 8 features -> 8 feature rows of 4 keys (transpose).
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int w = e >> 1;
                uint32_t lo, hi;
                if (e & 1) {
                    lo = (vreg[0][w] >> 16) | (vreg[1][w] & 0xFFFF0000u);
                    hi = (vreg[2][w] >> 16) | (vreg[3][w] & 0xFFFF0000u);
                } else {
                    lo = (vreg[0][w] & 0xFFFFu) | (vreg[1][w] << 16);
                    hi = (vreg[2][w] & 0xFFFFu) | (vreg[3][w] << 16);
                }
                const int row = vdc * 8 + e;
                const int chunk = (vq >> 1) ^ swz_v(row);
                *reinterpret_cast<u32x2_t*>(vt_lds + row * kBN + chunk * 8 + (vq & 1) * 4) =
                    u32x2_t{lo, hi};
            }
        }
    };

    // ---- per-lane LDS fragment addresses (loop invariant)
    const int krow = perm_k(j);
    const int vrow = perm_v(j);
    int k_off[kDS];
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds)
        k_off[ds] = krow * D + (((2 * ds + h) ^ swz_k(krow)) & (kCH - 1)) * 8;
    int v_off[kKB][2];
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
            v_off[kb][t] = vrow * kBN + (((4 * kb + 2 * t + h) ^ swz_v(vrow)) & (kVCH - 1)) * 8;
    // key offset (inside a 32-key block) of accumulator register r
    int key_of_reg[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) key_of_reg[r] = perm_k(8 * (r >> 2) + 4 * h + (r & 3));

    f32x16_t o[kQB][kDB];
    float m_ref[kQB], l_sum[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        m_ref[qb] = -INFINITY;
        l_sum[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.f;
    }

    const float c = p.c;
    const int ntiles = (Nk + kBN - 1) / kBN;
    load_tile(0);

    for (int kt = 0; kt < ntiles; ++kt) {
        const int key0 = kt * kBN;
        __syncthreads();                     // previous tile fully consumed
        store_tile();
        __syncthreads();
        if (kt + 1 < ntiles) load_tile(key0 + kBN);   // in flight during compute

        // S^T = K Q^T
        f32x16_t s[kQB][kKB];
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
#pragma unroll
            for (int ds = 0; ds < kDS; ++ds) {
                const bf16x8_t kf = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const u32x4_t*>(k_lds + kb * 32 * D + k_off[ds]));
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb)
                    s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ds], s[qb][kb], 0, 0, 0);
            }
        }

        const bool partial = key0 + kBN > Nk;
        bf16x8_t pf[kQB][kKB][2];
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            if (partial) {
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (key0 + kb * 32 + key_of_reg[r] >= Nk) s[qb][kb][r] = -INFINITY;
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
            mx = other_half_max(mx);
            const float mt = mx * c;
            const float mo = m_ref[qb];
            const bool need = mt > mo + kTau;
            const float mn = need ? mt : mo;
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float alpha = __builtin_amdgcn_exp2f(mo - mn);
                l_sum[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < kDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
            }
            m_ref[qb] = mn;
            float lsum = l_sum[qb];
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    uint32_t pk[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int r0 = 8 * t + 2 * u;
                        float e0 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][r0], c, -mn));
                        float e1 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][r0 + 1], c, -mn));
                        if (partial) {
                            if (key0 + kb * 32 + key_of_reg[r0] >= Nk) e0 = 0.f;
                            if (key0 + kb * 32 + key_of_reg[r0 + 1] >= Nk) e1 = 0.f;
                        }
                        pk[u] = pack_bf16(e0, e1);
                        // fp32 sum of the unrounded weights: the LSE must not
                        // carry the bf16 rounding of P (it would reach 2^-9
                        // relative on rows with few keys).
                        lsum += e0 + e1;
                    }
                    pf[qb][kb][t] = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
                }
            }
            l_sum[qb] = lsum;
        }

        // O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const bf16x8_t vf = __builtin_bit_cast(
                        bf16x8_t, *reinterpret_cast<const u32x4_t*>(vt_lds + db * 32 * kBN + v_off[kb][t]));
#pragma unroll
                    for (int qb = 0; qb < kQB; ++qb)
                        o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][kb][t], o[qb][db], 0, 0, 0);
                }
    }

    // ---- epilogue: normalise, bf16 round-to-nearest-even, pad rows as zeros
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int qi = m0 + wave * (kQB * 32) + qb * 32 + j;
        if (qi >= q_slots) continue;
        const bool real = qi < q_real;
        const float l_tot = other_half_sum(l_sum[qb]);
        const float inv = real ? 1.0f / l_tot : 0.f;
        uint16_t* dst = out_h + (int64_t)(q_start + qi) * p.o_ts + 16 * h;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
            u32x4_t w0, w1;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                w0[u] = pack_bf16(o[qb][db][2 * u] * inv, o[qb][db][2 * u + 1] * inv);
                w1[u] = pack_bf16(o[qb][db][8 + 2 * u] * inv, o[qb][db][9 + 2 * u] * inv);
            }
            if (!real) w0 = w1 = u32x4_t{0u, 0u, 0u, 0u};   // pad row: +0.0
            *reinterpret_cast<u32x4_t*>(dst + 32 * db) = w0;
            *reinterpret_cast<u32x4_t*>(dst + 32 * db + 8) = w1;
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
