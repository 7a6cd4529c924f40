// chunk_common.h - matrix-core and cross-lane helpers shared by the chunked
// prefill kernels (bf16 32x32x16 and fp32 16x16x4 MFMA fragments, LDS-only
// barriers, the in-register accumulator transpose, the wave prefix sum).
//
// Lane l of v_mfma_f32_32x32x16_bf16 holds A[l%32][8(l/32)+e] and
// B[8(l/32)+e][l%32] (e = 0..7); accumulator element r is
// C[8(r/4) + 4(l/32) + r%4][l%32]. Lane l of v_mfma_f32_16x16x4f32 supplies
// A[l%16][4s + l/16] and B[4s + l/16][l%16] for k-step s; accumulator element
// r is C[4(l/16) + r][l%16].
#pragma once

#include "common.h"

namespace gdn {

// Chain pass options: V read as zero; initial state the identity (the given
// start state ignored); outputs written (job tables only). With the first two
// and d_v = d_k the final state of a token range is the linear part A of its
// state map S_end = S_start A + B.
constexpr int CHAIN_ZERO_V = 1;
constexpr int CHAIN_INIT_IDENTITY = 2;
constexpr int CHAIN_OUTPUT = 4;

// One (sequence, head)-pair slot of a chain pass driven by a job table (the
// sequence-parallel prefill): walk the token range of segment `seg` of the
// packed axis from `init`, into `fin`, with the options in `flags`. init and
// fin point at [H][d_v][d_k] fp32 states (the head's block is added by the
// kernel) or are NULL (zero start state; final state not kept). seg < 0:
// nothing to do.
struct SegJob {
    int seg;
    int flags;
    const float *init;
    float *fin;
};

namespace chunk {

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 32 x 8 operand slice of a row-major bf16 LDS matrix: row r0 + lane%32,
// columns k0 + 8*(lane/32) .. +8
__device__ __forceinline__ bf16x8 frag32(const bf16 *m, int ld, int r0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8 *>(m + (r0 + (lane & 31)) * ld + k0 + 8 * (lane >> 5));
}
// The token-contiguous copies of K and V (sKt, sVt) are written as 8 x 8
// transposed blocks; to keep those writes free of LDS bank conflicts the
// 8-token column block of row d is stored at block (k/8) ^ ((d >> 4) & 7).
__device__ __forceinline__ bf16x8 frag32_sw(const bf16 *m, int ld, int r0, int k0, int lane) {
    const int row = r0 + (lane & 31);
    const int blk = ((k0 >> 3) + (lane >> 5)) ^ ((row >> 4) & 7);
    return *reinterpret_cast<const bf16x8 *>(m + row * ld + 8 * blk);
}
// acc += A[i0..i0+32, kb..kb+16*KS) B[kb..kb+16*KS, j0..j0+32]; A row-major
// (ld_a), B given as Bt[j][k] (ld_b), column-swizzled as above when SWB. All
// operand fragments are read before the first MFMA.
//
// The compiler's scheduler would otherwise interleave each fragment load
// with a wait right before its MFMA and expose the LDS latency once per
// k-step; sched_barrier keeps the whole batch of loads ahead of the MFMAs.
template <int KS, bool SWB = false>
__device__ __forceinline__ f32x16 mma32(f32x16 acc, const bf16 *a, int ld_a, int i0,
                                        const bf16 *bt, int ld_b, int j0, int lane, int kb = 0) {
    bf16x8 fa[KS], fb[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        fa[s] = frag32(a, ld_a, i0, kb + 16 * s, lane);
        fb[s] = SWB ? frag32_sw(bt, ld_b, j0, kb + 16 * s, lane) : frag32(bt, ld_b, j0, kb + 16 * s, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = mfma32(fa[s], fb[s], acc);
    return acc;
}
// Same product over k in [0, 32*KS2) as two independent accumulator chains
// (even / odd k-steps) interleaved, which halves the dependent MFMA latency;
// returns the sum.
template <int KS2, bool SWB = false>
__device__ __forceinline__ f32x16 mma32_2(f32x16 acc, const bf16 *a, int ld_a, int i0,
                                          const bf16 *bt, int ld_b, int j0, int lane) {
    bf16x8 fa[2 * KS2], fb[2 * KS2];
#pragma unroll
    for (int s = 0; s < 2 * KS2; ++s) {
        fa[s] = frag32(a, ld_a, i0, 16 * s, lane);
        fb[s] = SWB ? frag32_sw(bt, ld_b, j0, 16 * s, lane) : frag32(bt, ld_b, j0, 16 * s, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc1 = {};
#pragma unroll
    for (int s = 0; s < KS2; ++s) {
        acc = mfma32(fa[2 * s], fb[2 * s], acc);
        acc1 = mfma32(fa[2 * s + 1], fb[2 * s + 1], acc1);
    }
    return acc + acc1;
}
// row of accumulator element r of a 32x32 tile (the column is lane % 32)
__device__ __forceinline__ int acc_row(int r, int lane) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Workgroup barrier that orders LDS traffic only: global loads issued before
// it stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Keep the compiler from moving this wave's LDS accesses across the point
// (the hardware executes one wave's LDS instructions in order).
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// acc += X Y for 16 x 16 fp32 blocks in LDS (v_mfma_f32_16x16x4f32: lane l
// supplies X[l%16][4s + l/16] and Y[4s + l/16][l%16] for k-step s).
__device__ __forceinline__ f32x4 mm16(f32x4 acc, const float *X, int ldx, const float *Y, int ldy,
                                      int lane) {
    const int r = lane & 15, kq = lane >> 4;
    float xa[4], yb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        xa[s] = X[r * ldx + 4 * s + kq];
        yb[s] = Y[(4 * s + kq) * ldy + r];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[s], yb[s], acc, 0, 0, 0);
    return acc;
}
// Accumulator layout -> B-operand layout of v_mfma_f32_16x16x4f32 without
// LDS. Element r of lane (q, j) = 16q + j holds M[4q + r][j]; k-step s of a
// B operand needs M[4s + q][j] at lane (q, j). Viewing the four registers as
// a 4 x 4 grid of (register, 16-lane row) blocks, that is a block transpose:
// swap rows 2,3 of registers 0,1 with rows 0,1 of registers 2,3
// (v_permlane32_swap), then odd rows of registers 0,2 with even rows of
// registers 1,3 (v_permlane16_swap).
__device__ __forceinline__ f32x4 acc_to_bop(f32x4 c) {
    auto u = [](float x) { return __builtin_bit_cast(unsigned, x); };
    auto f = [](unsigned x) { return __builtin_bit_cast(float, x); };
    const auto p02 = __builtin_amdgcn_permlane32_swap(u(c[0]), u(c[2]), false, false);
    const auto p13 = __builtin_amdgcn_permlane32_swap(u(c[1]), u(c[3]), false, false);
    const auto q01 = __builtin_amdgcn_permlane16_swap(p02[0], p13[0], false, false);
    const auto q23 = __builtin_amdgcn_permlane16_swap(p02[1], p13[1], false, false);
    return f32x4{f(q01[0]), f(q01[1]), f(q23[0]), f(q23[1])};
}
// acc += X Y with X a 16 x 16 fp32 block in LDS and Y given in B-operand
// registers (acc_to_bop of a product computed by this wave)
__device__ __forceinline__ f32x4 mm16_rb(f32x4 acc, const float *X, int ldx, f32x4 yb, int lane) {
    const int r = lane & 15, kq = lane >> 4;
    float xa[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) xa[s] = X[r * ldx + 4 * s + kq];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[s], yb[s], acc, 0, 0, 0);
    return acc;
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8
// inside each 16-lane row, then the running totals of rows 0 and 0..1 are
// broadcast into the rows after them (DPP row_shr and row_bcast).
template <int CTRL, int ROWMASK, bool BOUND_ZERO>
__device__ __forceinline__ float dpp_or_zero(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), CTRL, ROWMASK, 0xF, BOUND_ZERO));
}
__device__ __forceinline__ float wave_inclusive_scan(float x) {
    x += dpp_or_zero<0x111, 0xF, true>(x);    // row_shr:1
    x += dpp_or_zero<0x112, 0xF, true>(x);    // row_shr:2
    x += dpp_or_zero<0x114, 0xF, true>(x);    // row_shr:4
    x += dpp_or_zero<0x118, 0xF, true>(x);    // row_shr:8
    x += dpp_or_zero<0x142, 0xA, false>(x);   // row_bcast:15 into rows 1, 3
    x += dpp_or_zero<0x143, 0xC, false>(x);   // row_bcast:31 into rows 2, 3
    return x;
}

// 8 x 8 bf16 transpose held as 8 rows of 8.
__device__ __forceinline__ void transpose8x8(const bf16x8 (&in)[8], bf16x8 (&out)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int r = 0; r < 8; ++r) out[e][r] = in[r][e];
}

// Work mapping of the sequential chunk kernels: one workgroup per (sequence,
// head) pair and 32-wide d_v tile, four tiles per pair. The dispatcher deals
// workgroups to the eight XCDs in turn (workgroup w on XCD w % 8); the k-th
// workgroup of an XCD takes tile k % 4 of pair 8 (k / 4) + w % 8. A pair's four
// tiles then run side by side on one XCD and share its L2, while consecutive
// pairs (the heads of one sequence, then the next sequence) go to different
// XCDs, so a long sequence does not pile up on one of them. The grid is rounded
// up to whole rounds of 32 workgroups; the surplus ones get false.
constexpr int PAIR_TILES = 4;
__host__ __device__ inline unsigned pair_grid(int npairs) { return (unsigned)((npairs + 7) / 8 * 8 * PAIR_TILES); }
__device__ __forceinline__ bool pair_tile(int wid, int npairs, int &pair, int &tile)
{
    const int kx = wid >> 3;
    pair = (kx / PAIR_TILES) * 8 + (wid & 7);
    tile = kx % PAIR_TILES;
    return pair < npairs;
}

// Longest-first dispatch of packed sequences. Workgroups start in index
// order, so when the pairs of the longest sequences take the lowest indices
// the short ones fill in behind them (list scheduling, longest processing
// time first) instead of a long chain starting last. seq_of_rank returns the
// sequence of rank r in the order by length, longest first, ties by index.
// Every thread of the workgroup calls it (it holds one barrier); lens is LDS
// scratch for RANK_MAX ints that no wave writes again before the caller's
// next barrier. Costs N * ceil(N / 64) LDS broadcast reads per wave; above
// RANK_MAX sequences the identity order is used instead.
constexpr int RANK_MAX = 256;
__device__ inline int seq_of_rank(const int32_t *cu, int N, int T, int r, int *lens)
{
    for (int n = (int)threadIdx.x; n < N; n += (int)blockDim.x) {
        long a = cu[n], b = cu[n + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        b = b < a ? a : (b > T ? T : b);
        lens[n] = (int)(b - a);
    }
    lds_barrier();
    const int lane = (int)threadIdx.x & 63;
    for (int j = 0; j < N; j += 64) {
        const int nn = j + lane;
        int rank = 0;
        if (nn < N) {
            const int ln = lens[nn];
            for (int m = 0; m < N; ++m) {
                const int lm = lens[m];
                rank += (lm > ln) | ((lm == ln) & (m < nn));
            }
        }
        const unsigned long long hit = __ballot(nn < N && rank == r);
        if (hit) return j + __ffsll((long long)hit) - 1;
    }
    return r;                                  // not reached: ranks are a permutation
}

}  // namespace chunk
}  // namespace gdn
