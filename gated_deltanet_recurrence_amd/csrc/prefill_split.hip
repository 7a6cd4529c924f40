// prefill_split.hip - chunkwise gated delta rule forward in two passes, for
// d_k = d_v = 128, bf16 q/k/v, chunks of 64 tokens, fp32 state.
//
// The chunk algebra is the one of "5. Linear Attention" (LinkQwen ch. 5),
// section "Chunk implementation of the Delta Rule", stages 1-3, and of
// "[LLM Algorithms-2] Gated DeltaNet: Teaching Linear Attention to Overwrite
// and Forget", section 7. Per chunk of C = 64 tokens, with the state stored
// S[d_v][d_k]:
//   gamma_i  = sum_{s<=i} g_s,  Gamma_ij = exp(gamma_i - gamma_j) (j <= i)
//   A        = -strict_lower(diag(beta) K K^T * Gamma),  T = (I - A)^-1
//   T_w      = T diag(beta e^gamma),  T_u = T diag(beta)
//   W        = T_w K,  U = T_u V,  Delta = U - W S^T
//   O        = scale (diag(e^gamma) Q S^T + lower_incl_diag(Q K^T * Gamma) Delta)
//   S       <- e^{gamma_63} S + Delta~^T K,  Delta~_j = e^{gamma_63 - gamma_j} Delta_j
//
// Everything up to T_u = T diag(beta) depends on one chunk of one head only,
// and is the same for every d_v column. The first pass (chunk_solve, one
// wave per (chunk, head)) computes it once per (chunk, head), fully in
// parallel over all chunks, from k, g and beta alone; the second pass
// (chunk_chain) walks the chunks of each sequence in order and carries the
// state. Without a workspace the chain kernel instead runs the same one-wave
// solver on two of its own waves, two chunks ahead (chunk_chain_kernel with
// FUSED). The chain folds the
// decay into the delta,
//   Delta = T_u (V - diag(e^gamma) K S^T)      (T_w K S^T = T_u diag(e^gamma) K S^T)
// so only T_u crosses between the passes, and it forms P = lower_incl_diag(
// Q K^T * Gamma) itself from the q and k tiles it stages anyway. Splitting
// takes the triangular solve off the sequential path and stops the d_v tiles
// of a head from each repeating it; the price is the 6 KiB bf16 T_u per
// (chunk, head) written to the caller's workspace and read back: 96 B of
// HBM traffic each way per token-head, on top of the 1032 B of q, k, v, o,
// g and beta (the solve pass also reads k, g and beta a second time, 264 B).
//
// q and k may have fewer heads (H_k) than v, g, beta, o and the state (H):
// value head h reads query/key head h / (H / H_k) (the repeat_interleave head
// expansion of the "Gated DeltaNet body" layer code, "5. Linear Attention").
// The workspace is per value head, since beta and g are.
//
// Workspace layout: for head h and chunk slot s, 3072 bf16 at
// ((h * nslots) + s) * 3072, as 384 pieces of 8 consecutive row elements of
// T_u (its non-zero lower 64 x 64 part: rows 0-31 span columns 0-31 only):
// pieces 0..255 are rows 32-63 (8 pieces per row), 256..383 rows 0-31 (4 per
// row). Chunk c of sequence n has slot (bos_n / 64) + n + c, where bos_n is
// its first token: slots of different sequences never collide and every slot
// is below nslots = total_tokens / 64 + N + 1. The per-channel item (below)
// starts with the same T_u pieces.
#include <atomic>
#include <type_traits>

#include "chunk_common.h"
#include "launch.h"

namespace gdn {

namespace split {

using namespace chunk;

constexpr int C = 64;
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int WS_T = 384;                     // 16-byte pieces of T_u per (chunk, head)
constexpr int WS_P = 384;                     // 16-byte pieces of P (per-channel items)
constexpr int ITEM_ELEMS = 8 * WS_T;          // 3072 bf16 per (chunk, head) in the workspace

// ---------------------------------------------------------------------------
// Pass 1 with a per-channel decay: chunk_prep_channel, workgroups of 4 waves
// looping over (chunk slot, head) items; the LDS layout of its triangular
// solve (solve_store). With a scalar gate the pass is chunk_solve (one wave
// per item, WaveSolver below).
// ---------------------------------------------------------------------------
constexpr int P_NT = 256;
constexpr int P_LD_K = DK + 8;                 // bf16 row stride of K
constexpr int P_LD_A = C + 4;                  // fp32 row stride of T
constexpr int P_LD_A2 = 52;                    // fp32 row stride of the off-diagonal part of A
constexpr int P_DB = 16 * 16 + 4;              // floats per diagonal 16 x 16 block of A (padded
                                               // so the four blocks' rows fall on different banks)
constexpr int P_SZ_R1 = C * P_LD_K * 2;        // 17408: K, then T
constexpr int P_SZ_A = 48 * P_LD_A2 * 4;       // 9984: rows 16-63, columns 0-47 of A
constexpr int P_SZ_Y = 4 * P_DB * 4;           // 4160: the diagonal blocks of A, row-major
static_assert(C * P_LD_A * 4 <= P_SZ_R1, "T fits where K was");

// ---------------------------------------------------------------------------
// Pass 2: chunk_chain. One workgroup of 8 waves per (32-wide d_v tile, head,
// sequence), one LDS barrier per chunk. LDS holds two staging buffers (the
// chunk being computed and the next one, written meanwhile) and two copies of
// every tile passed between waves. Row strides are chosen for the
// v_mfma_f32_16x16x32_bf16 operand reads (16 consecutive rows, four 16-byte
// column chunks), which then hit every LDS bank equally: 288 bytes for rows
// of 128, 160 for rows of 64 and 80 for rows of 32. The lower-triangular
// 64 x 64 tiles (T_u, and P with a per-channel decay) keep rows 0-31 (read in
// columns 0-31 only) and rows 32-63 as two tiles of different width.
// ---------------------------------------------------------------------------
constexpr int MAX_DEVICES = 64;               // per-device launch caches
constexpr int DVT = 32;
constexpr int NT = 512;
constexpr int LD_R = DK + 16;                  // 144: Q, K, S rows
constexpr int LD_L = C + 16;                   // 80: rows 32-63 of T_u, P; Delta^T rows
constexpr int LD_H = 32 + 8;                   // 40: rows 0-31 of T_u, P; V rows
constexpr int SZ_QK = C * LD_R * 2;            // 18432
constexpr int SZ_V = C * LD_H * 2;             // 5120
constexpr int SZ_TH = 32 * LD_H * 2;           // 2560: rows 0-31 of T_u
constexpr int SZ_TL = 32 * LD_L * 2;           // 5120: rows 32-63 of T_u
constexpr int SZ_SC = 3 * C * 4 + DK * 4;      // gamma log2(e), e^gamma, e^{gamma_63 - gamma},
                                               // then the key factors F of P (scalar gate)
                                               // or e^{gamma_63} per channel
constexpr int B_Q = 0;
constexpr int B_K = B_Q + SZ_QK;
constexpr int B_V = B_K + SZ_QK;
constexpr int B_TH = B_V + SZ_V;
constexpr int B_TL = B_TH + SZ_TH;
constexpr int B_SC = B_TL + SZ_TL;
constexpr int SZ_BUF = B_SC + SZ_SC;           // 50944
constexpr int SZ_PH = 32 * LD_H * 2;           // 2560: P rows 0-31
constexpr int SZ_P = SZ_PH + 32 * LD_L * 2;    // 7680: P rows 0-31, then 32-63
constexpr int SZ_S = DVT * LD_R * 2;           // 9216: bf16 S [32][144]
constexpr int SZ_DT = DVT * LD_L * 2;          // 5120: Delta^T [32][80]
constexpr int SZ_PB = 6 * 64 * 16;             // 6144: P^T of a chunk (scalar gate) as six
                                               // B-operand registers, 1 KiB each, lane-linear
constexpr int OFF_BUF = 0;                     // two of each from here on
// One wave's triangular solve (WaveSolver: the solve pass, and the in-chain
// solve with scalar gates and no workspace) keeps one chunk's 16 x 16 blocks
// (I, J), J <= I, of A and then T, fp32 row-major at row stride SV_LD
// (conflict-free operand reads), and the chunk's gamma log2(e) and beta. The
// four diagonal blocks come first, SV_DIAG floats apart, so that they start
// 64 bytes apart in the bank cycle: their forward substitutions read and
// write row i of all four at once. Then the six off-diagonal blocks.
constexpr int SV_LD = 20;
constexpr int SV_BLK = 16 * SV_LD;
constexpr int SV_DIAG = SV_BLK + 16;
constexpr int SV_OFF0 = 4 * SV_DIAG;
constexpr int SV_BYTES = (SV_OFF0 + 6 * SV_BLK + 2 * C) * 4;   // 13568: twelve per CU
constexpr int SV_WAVE0 = 6;                    // solver waves SV_WAVE0, + 1
constexpr int SV_LOAD0 = 4;                    // loading waves SV_LOAD0, + 1
constexpr int SV_PRIO = 1;                     // solver waves' issue priority
// The copies passed between waves follow the staging buffers: P copies (per
// channel: P from the workspace; scalar gate with the two-pass layout: P^T as
// formed by the staging waves), S, Delta^T, then the solver regions (in-chain
// solve only, which has no room for P copies: its output waves form P^T).
template <bool PERCH, bool FUSED> struct ChainLds {
    static constexpr bool PST = !PERCH && !FUSED;   // P^T formed by staging waves 6-7
    static constexpr int P = OFF_BUF + 2 * SZ_BUF;
    static constexpr int S = P + (PERCH ? 2 * SZ_P : PST ? 2 * SZ_PB : 0);
    static constexpr int DT = S + 2 * SZ_S;
    static constexpr int SV = DT + 2 * SZ_DT;
    static constexpr int BYTES = SV + (FUSED ? 2 * SV_BYTES : 0);
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(!(PERCH && FUSED), "the in-chain solve takes scalar gates");
};
static_assert(DV / DVT == PAIR_TILES, "one workgroup per d_v tile of a pair");
static_assert(SZ_BUF % 16 == 0 && SZ_P % 16 == 0, "16-byte aligned tiles");

// Accumulator tiles are written 8 bytes per lane (row lane%16, columns
// 4 (lane/16) ..); to spread those writes over the banks the 16-byte chunks
// of row r are swapped by ((r / 4) % 4) within aligned groups of four, which
// keeps the 16-row operand reads conflict-free and their addresses additive
// in the k-step. swz gives the element XOR for a lane whose row is
// (multiple of 16) + lane%16.
__device__ __forceinline__ int swz(int lane) { return ((lane & 15) >> 2) << 3; }
// The bf16 copies of S (row stride LD_R) and Delta^T (LD_L) that the recurrence
// waves pass to the output waves are read 16 rows at a time in the order
// 8 (i/4) + 4 u + i%4 (i = 0..15, u = 0 or 1), and both strides repeat the bank
// pattern every 8 rows; XOR-ing each row's 16-byte chunk index by these
// functions of its row bits 3 and 4 puts the 16 rows of a read on distinct
// banks (32 or 64 four-byte banks alike). Element XORs, by d_v row r < 32.
__device__ __forceinline__ int swS(int r) { return (((r >> 3) & 1) << 3) | (((r >> 4) & 1) << 6); }
__device__ __forceinline__ int swD(int r) { return ((r >> 3) & 3) << 3; }
// The staged Q and K tiles (row stride LD_R) swap the two 128-byte halves of
// rows 16-31 and 48-63 (element XOR by row bit 4). The recurrence reads K for
// X in the row order 8 (i/4) + 4 (t%2) + i%4 (+32 (t/2)); at 288 bytes per row
// its rows 16 apart then fall on the same banks, and measured on gfx950 these
// reads took 1.7x the cycles of conflict-free ones; with the swap they run at
// the conflict-free rate, and the 16-consecutive-row, transposing and staging
// accesses keep theirs. Element XOR by row r.
__device__ __forceinline__ int swK(int r) { return ((r >> 4) & 1) << 6; }
__device__ __forceinline__ bf16x8 lds8(const bf16 *base, int off) {
    return *reinterpret_cast<const bf16x8 *>(base + off);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// acc += L R for 16 x 16 fp32 blocks on the bf16 matrix cores, each operand
// split as x = hi + lo (hi = bf16(x), lo = bf16(x - hi)): the 32 k-slots of
// one v_mfma_f32_16x16x32_bf16 hold k = 4 q + e (e < 4) twice, so that
//   slots 8 q + e      L_hi[m][4 q + e] R_hi[4 q + e][n]
//   slots 8 q + 4 + e  L_hi[m][4 q + e] R_lo[4 q + e][n]
// and a second one adds L_lo R_hi: L R up to L_lo R_lo (relative 2^-17).
// Lane 16 q + m supplies lrow = L[m][4 q .. 4 q + 3] (a row piece) and
// rcol = R[4 q .. 4 q + 3][m] (a column piece: R's accumulator layout).
// The operands are split once each (lsplit, rsplit) and reused by every
// product they enter.
struct LSplit {
    bf16x8 a1, a2;                             // {hi, hi}, {lo, 0}
};
__device__ __forceinline__ LSplit lsplit(f32x4 lrow) {
    LSplit o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bf16 h = (bf16)lrow[e];
        o.a1[e] = h;
        o.a1[e + 4] = h;
        o.a2[e] = (bf16)(lrow[e] - (float)h);
        o.a2[e + 4] = (bf16)0.f;
    }
    return o;
}
__device__ __forceinline__ bf16x8 rsplit(f32x4 rcol) {             // {hi, lo}
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bf16 h = (bf16)rcol[e];
        b[e] = h;
        b[e + 4] = (bf16)(rcol[e] - (float)h);
    }
    return b;
}
__device__ __forceinline__ f32x4 mm16x(f32x4 acc, const LSplit &l, bf16x8 r) {
    acc = mfma16(l.a1, r, acc);
    return mfma16(l.a2, r, acc);
}
// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane L
// names 8 bytes at element offset off (its row k0 + L/4 and 4 columns of a
// row-major matrix M), and lane m receives four consecutive rows of one
// column: M[k0 .. k0 + 3][c(m)], where columns c(4g .. 4g + 3) are the four
// named by lanes with L % 4 = g. k0 may differ between groups.
__device__ __forceinline__ bf16x4 tr4(const bf16 *base, int off) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + off)));
}
__device__ __forceinline__ bf16x8 cat4(bf16x4 lo, bf16x4 hi) {
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// two 16x16 fp32 accumulators as one bf16 B operand (rows 4 (lane/16) + r of
// the first, then of the second)
__device__ __forceinline__ bf16x8 acc_pair_bf16(f32x4 a, f32x4 b) {
    return bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                  (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
}

// Bounds of sequence n: tokens [bos, eos) of the packed token axis.
__device__ __forceinline__ void seq_bounds(const int32_t *cu, int n, int T, long &bos, long &eos) {
    if (cu) {
        long a = cu[n], b = cu[n + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        b = b < a ? a : (b > T ? T : b);
        bos = a;
        eos = b;
    } else {
        bos = (long)n * T;
        eos = bos + T;
    }
}
__device__ __forceinline__ long first_slot(const int32_t *cu, int n, int T) {
    long bos, eos;
    seq_bounds(cu, n, T, bos, eos);
    return (bos >> 6) + n;
}

// acc += A B over k in [0, 16 KS) with A given row-major (a[i][k]) and B as
// bt[j][k]; SWA / SWB select the column-swizzled token-contiguous layout
// (frag32_sw) for either operand.
template <int KS, bool SWA, bool SWB>
__device__ __forceinline__ f32x16 mma32s(f32x16 acc, const bf16 *a, int ld_a, int i0,
                                         const bf16 *bt, int ld_b, int j0, int lane) {
    bf16x8 fa[KS], fb[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        fa[s] = SWA ? frag32_sw(a, ld_a, i0, 16 * s, lane) : frag32(a, ld_a, i0, 16 * s, lane);
        fb[s] = SWB ? frag32_sw(bt, ld_b, j0, 16 * s, lane) : frag32(bt, ld_b, j0, 16 * s, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = mfma32(fa[s], fb[s], acc);
    return acc;
}

}  // namespace split

using namespace split;

// The triangular solve and the stores of one (chunk, head) item, shared by the
// prep passes: with A = -strict_lower(...) given as its four diagonal 16 x 16
// blocks (sY, row-major, P_DB floats apart) and rows 16-63, columns 0-47
// (sA, row stride P_LD_A2), T = (I - A)^-1 is formed in sT (row stride
// P_LD_A) and T_u = T diag(colu) (colu = beta) is written to the workspace
// item dst as 16-byte bf16 pieces. All four waves of the workgroup call it.
__device__ __forceinline__ void solve_store(const float *sA, const float *sY, float *sT,
                                            const float *colu, bf16 *dst, int tid, int wave)
{
    const int lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4;
    auto blkA = [&](int I, int J) { return sA + (16 * (I - 1)) * P_LD_A2 + 16 * J; };
    auto blkT = [&](int I, int J) { return sT + (16 * I) * P_LD_A + 16 * J; };
    auto store_T = [&](int I, int J, f32x4 acc) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sT[(16 * I + 4 * lq + r) * P_LD_A + 16 * J + lr] = acc[r];
    };

    if (wave == 0) {
        // the other waves wait at the barrier below: this wave wins issue
        // arbitration against the co-resident workgroups' waves meanwhile
        __builtin_amdgcn_s_setprio(2);
        // ---- diagonal blocks, one per 16 lanes: lane 16 b + c computes
        //      column c of D_b = (I - A_bb)^-1 row by row,
        //      D[i][c] = [i == c] + sum_{m < i} A[i][m] D[m][c]
        //      (the block's row i read by all 16 lanes: an LDS broadcast);
        //      row i + 1 is loaded while row i is summed ----
        const int bb = lane >> 4, c = lane & 15;
        const float *Ab = sY + bb * P_DB;
        float D[16];
        f32x4 rowv[2][4];
        auto load_row = [&](int i, f32x4 (&dstv)[4]) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (4 * t < i) dstv[t] = *reinterpret_cast<const f32x4 *>(Ab + i * 16 + 4 * t);
        };
        load_row(1, rowv[1]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i + 1 < 16) load_row(i + 1, rowv[(i + 1) & 1]);
            float acc = i == c ? 1.f : 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * t + e < i) acc += rowv[i & 1][t][e] * D[4 * t + e];
            D[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[(16 * bb + i) * P_LD_A + 16 * bb + c] = D[i];
        __builtin_amdgcn_s_setprio(0);
    } else if (wave == 1) {
        // the 16 x 16 blocks (0,1) and (2,3) of T are zero; the output reads them
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int e = lane + 64 * u;   // 128 four-float pieces
            const int blk = e >> 6, row = (e >> 2) & 15, c4 = 4 * (e & 3);
            *reinterpret_cast<f32x4 *>(sT + (32 * blk + row) * P_LD_A + 32 * blk + 16 + c4) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    lds_barrier();

    // ---- off-diagonal blocks of T. With D_b the diagonal inverses:
    //   T10 = D1 A10 D0,  T32 = D3 A32 D2,  T21 = D2 A21 D1           (16-level)
    //   T20 = D2 (A20 D0 + A21 T10)
    //   T31 = T32 (A21 D1) + D3 (A31 D1)
    //   T30 = T32 (A20 D0 + A21 T10) + D3 (A30 D0 + A31 T10)          (32-level)
    {
        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
        f32x4 h0 = z4, h1 = z4;
        // the waves with the most products in a level go first in issue
        if (wave == 0 || wave == 2) __builtin_amdgcn_s_setprio(1);
        if (wave == 0) {
            const f32x4 c10 = mm16(z4, blkA(1, 0), P_LD_A2, blkT(0, 0), P_LD_A, lane);
            h0 = mm16(z4, blkA(2, 0), P_LD_A2, blkT(0, 0), P_LD_A, lane);              // A20 D0
            store_T(1, 0, mm16_rb(z4, blkT(1, 1), P_LD_A, acc_to_bop(c10), lane));
        } else if (wave == 1) {
            const f32x4 c32 = mm16(z4, blkA(3, 2), P_LD_A2, blkT(2, 2), P_LD_A, lane);
            store_T(3, 2, mm16_rb(z4, blkT(3, 3), P_LD_A, acc_to_bop(c32), lane));
        } else if (wave == 2) {
            h0 = mm16(z4, blkA(2, 1), P_LD_A2, blkT(1, 1), P_LD_A, lane);              // A21 D1
            h1 = mm16(z4, blkA(3, 1), P_LD_A2, blkT(1, 1), P_LD_A, lane);              // A31 D1
            store_T(2, 1, mm16_rb(z4, blkT(2, 2), P_LD_A, acc_to_bop(h0), lane));
        } else {
            h0 = mm16(z4, blkA(2, 0), P_LD_A2, blkT(0, 0), P_LD_A, lane);              // A20 D0
            h1 = mm16(z4, blkA(3, 0), P_LD_A2, blkT(0, 0), P_LD_A, lane);              // A30 D0
        }
        lds_barrier();
        __builtin_amdgcn_s_setprio(0);
        if (wave == 3) __builtin_amdgcn_s_setprio(2);
        if (wave == 0) {
            const f32x4 y00 = mm16(h0, blkA(2, 1), P_LD_A2, blkT(1, 0), P_LD_A, lane);
            store_T(2, 0, mm16_rb(z4, blkT(2, 2), P_LD_A, acc_to_bop(y00), lane));
        } else if (wave == 2) {
            const f32x4 t = mm16_rb(z4, blkT(3, 2), P_LD_A, acc_to_bop(h0), lane);
            store_T(3, 1, mm16_rb(t, blkT(3, 3), P_LD_A, acc_to_bop(h1), lane));
        } else if (wave == 3) {
            const f32x4 y00 = mm16(h0, blkA(2, 1), P_LD_A2, blkT(1, 0), P_LD_A, lane);
            const f32x4 y10 = mm16(h1, blkA(3, 1), P_LD_A2, blkT(1, 0), P_LD_A, lane);
            const f32x4 t = mm16_rb(z4, blkT(3, 2), P_LD_A, acc_to_bop(y00), lane);
            store_T(3, 0, mm16_rb(t, blkT(3, 3), P_LD_A, acc_to_bop(y10), lane));
        }
        lds_barrier();
    }

    __builtin_amdgcn_s_setprio(0);
    // ---- T diag(beta) -> workspace as 16-byte pieces (bf16). Piece order:
    //        0..255     rows 32-63 (8 per row)
    //        256..383   rows 0-31, columns 0-31 (4 per row) ----
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int e = tid + P_NT * u;
        if (e >= WS_T) break;                  // uniform per wave
        int i, j0;
        if (e < 256) {
            i = 32 + (e >> 3);
            j0 = 8 * (e & 7);
        } else {
            i = (e - 256) >> 2;
            j0 = 8 * (e & 3);
        }
        const f32x4 t0 = *reinterpret_cast<const f32x4 *>(sT + i * P_LD_A + j0);
        const f32x4 t1 = *reinterpret_cast<const f32x4 *>(sT + i * P_LD_A + j0 + 4);
        const f32x4 s0 = *reinterpret_cast<const f32x4 *>(colu + j0);
        const f32x4 s1 = *reinterpret_cast<const f32x4 *>(colu + j0 + 4);
        bf16x8 out;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            out[e2] = (bf16)(t0[e2] * s0[e2]);
            out[e2 + 4] = (bf16)(t1[e2] * s1[e2]);
        }
        *reinterpret_cast<bf16x8 *>(dst + 8 * e) = out;
    }
}

// ---------------------------------------------------------------------------
// chunk_prep: the parts of a chunk that do not depend on the state, for
// (chunk, head) items (prep_locate: which slot and head an item is); a workgroup takes
// items blockIdx.x, + gridDim.x, ... and loads the next item's K, g and beta
// into registers while it works on the current one, so that the HBM latency
// is paid once per workgroup.
//
//   stage  K (64 x 128) into LDS; gamma = prefix sum of g (wave 0)
//   gram   waves 0-2, one 32 x 32 tile each of A = -strict_lower(diag(beta)
//          K K^T * Gamma) (v_mfma_f32_32x32x16_bf16): wave 0 tile (0,0),
//          wave 1 (1,1), wave 2 (1,0). On the diagonal tiles one exponential
//          per element; across the halves Gamma_ij = E_i E_j with
//          E_t = e^{gamma_t - gamma_32} (t >= 32) or e^{gamma_32 - gamma_t}
//          (t < 32), two factors no larger than 1 for gates in (0, 1]
//   solve  wave 0 inverts the four 16 x 16 diagonal blocks of I - A by
//          forward substitution, 16 lanes per block and one column per lane
//   L1/L2  the off-diagonal blocks of T by two levels of 2 x 2 block
//          inversion, (L^-1)_21 = L22^-1 A21 L11^-1 (fp32 16x16x4 MFMA)
//   store  T diag(beta), bf16, to the workspace
// ---------------------------------------------------------------------------
struct PrepItem {
    int slot, h, nvalid;                       // nvalid = 0: nothing to do
    long row0;                                 // first token of the chunk
};
// Items and their order. Workgroup b runs on XCD b % 8, and every grid of the
// prep passes is a multiple of 8 workgroups, so item i always runs on XCD
// i % 8. Item i takes slot 8 (j / H) + i % 8 and head j % H, with j = i / 8:
// the H heads of a chunk slot run on one XCD, one after the other in
// workgroup order, and read the chunk's g and beta through one L2. Each
// 128-byte line of g or beta holds two tokens of every head; dealt head-minor
// over all XCDs, every XCD fetched it. The count is rounded up to whole
// groups of 8 slots; slots past the last sequence's chunks are unused items.
__host__ __device__ inline long prep_nitems(long nslots, int H) { return (nslots + 7) / 8 * 8 * H; }
__device__ __forceinline__ PrepItem prep_locate(const int32_t *cu, int item, int nitems, int T,
                                                int H, int N) {
    PrepItem it{0, 0, 0, 0};
    if (item >= nitems) return it;
    const int j = item >> 3;
    it.slot = 8 * (j / H) + (item & 7);
    it.h = j % H;
    // sequence of the slot: the last n whose first slot is <= slot
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (first_slot(cu, mid, T) <= it.slot) lo = mid;
        else hi = mid - 1;
    }
    long bos, eos;
    seq_bounds(cu, lo, T, bos, eos);
    const long c = it.slot - ((bos >> 6) + lo);
    const long len = eos - bos;
    if (c < 0 || c * C >= len) return it;      // unused slot
    it.row0 = bos + c * C;
    it.nvalid = (int)(len - c * C < C ? len - c * C : C);
    return it;
}

// ---------------------------------------------------------------------------
// chunk_prep_channel: the prep pass for a per-channel decay ("6.6 Gated
// DeltaNet", section 6.6.7: alpha_t in R^{d_k}, g = log alpha of shape
// [T][H][d_k]). With gamma_t[c] the chunk's running sum of g[c] (t inclusive)
// the chunk algebra keeps its shape once the keys and queries carry the decay
// channel by channel:
//   K+ = K e^gamma, Q+ = Q e^gamma, K^ = K e^{gamma_63 - gamma}  (factors <= 1)
//   M[i][j] = sum_c k_i[c] k_j[c] e^{gamma_i[c] - gamma_j[c]},  A = -strict_lower(diag(beta) M)
//   T = (I - A)^-1,  T_u = T diag(beta),  P = lower_incl(sum_c q_i k_j e^{gamma_i - gamma_j})
//   Delta = T_u (V - K+ S^T),  O = Q+ S^T + P Delta,  S <- S diag(e^{gamma_63}) + Delta^T K^
// M and P are products only after the exponent is split at a reference per
// 16-token row block I, rho_I = gamma at the token before the block:
// e^{gamma_i - gamma_j} = e^{gamma_i - rho_I} e^{rho_I - gamma_j}. The first
// factor is <= 1; the second is <= 1 below the block diagonal and at most the
// block's own decay on it (e^{rho_I - gamma_j}, j in block I); these bounds hold
// for gates in (0, 1] (g <= 0, gamma non-increasing), as the pages define the
// decay. While every channel decays by less than e^-80 inside every 16-token
// block of the item
// (both factors then fit bf16 and fp32), the diagonal blocks come from the same
// products; otherwise the item's diagonal blocks are summed element by element
// with exact exponentials.
//
// One item per loop step per workgroup of 4 waves; thread (c8, tg) = (tid %
// 16, tid / 16) owns tokens 4 tg .. 4 tg + 3 and channels 8 c8 .. 8 c8 + 7
// (wave I owns row block I), loads them (the next item's loads are issued
// while the current item computes), scans gamma (its four tokens in
// registers, the wave's four token groups by lane shifts, the earlier waves'
// totals through LDS), and writes every scaled copy of its elements: LDS
// operand tiles (KR = K e^{gamma - rho_I}, QR likewise, KC_I = K e^{rho_I -
// gamma} over tokens 0 .. 16 I + 15 for each I), and K+, K^, Q+ to the
// workspace. Wave I then forms row block I of M and of P^T on the matrix cores
// (16x16x32 bf16, operand tiles with 256-byte rows and 16-byte chunks
// XOR-swizzled by the row): the diagonal block from its own rows before the
// workgroup barrier (P's with bf16 hi + lo operand splits), the blocks left
// of it after. The triangular solve and the T stores are those of the scalar
// prep pass.
// Workspace item (CH_ITEM_ELEMS bf16): the pieces of T_u as in the scalar
// item, then P (rows 0-31 by keys 0-31, rows 32-63 by keys 0-63,
// row-major); then K+ and K^ ([64][128] row-major); Q+ in the output waves'
// operand order (fragment f = 4 (t / 16) + c / 32 of 1 KiB, lane 16 ((c / 8)
// % 4) + t % 16, 8 channels); then e^{gamma_63} (128 fp32).
// ---------------------------------------------------------------------------
constexpr int CH_P = ITEM_ELEMS;               // element offsets inside the item
constexpr int CH_KP = CH_P + 8 * WS_P;
constexpr int CH_KH = CH_KP + C * DK;
constexpr int CH_QP = CH_KH + C * DK;
constexpr int CH_EC = CH_QP + C * DK;          // 128 fp32 = 256 bf16 slots
constexpr int CH_ITEM_ELEMS = CH_EC + 2 * DK;
static_assert((CH_ITEM_ELEMS * 2) % 256 == 0, "items stay 256-byte aligned");
// LDS (bytes)
constexpr int CP_ROW = DK * 2;                 // 256-byte operand rows (swizzled)
constexpr int CP_KR = 0;
constexpr int CP_QR = CP_KR + C * CP_ROW;
constexpr int CP_KC = CP_QR + C * CP_ROW;      // KC_0 .. KC_3: 16, 32, 48, 64 rows
constexpr int CP_RHO = CP_KC + 160 * CP_ROW;   // rho_1 .. rho_4 [4][128] fp32
constexpr int CP_BETA = CP_RHO + 4 * DK * 4;   // beta [64], -beta [64]
constexpr int CP_FLAG = CP_BETA + 2 * C * 4;
constexpr int CP_TAB = CP_FLAG + 16;           // e^rho_1..4, F21 F31 F32, G1 G2 G3: [10][128]
constexpr int CP_LDS_BYTES = CP_TAB + 10 * DK * 4;
static_assert(CP_LDS_BYTES <= 160 * 1024 / 2, "two workgroups per CU");
static_assert(C * P_LD_A * 4 <= CP_KC, "T fits in the KR, QR tiles");
static_assert(P_SZ_A + P_SZ_Y <= 160 * CP_ROW, "A fits in the KC tiles");
static_assert(16 * DK * 4 <= 160 * CP_ROW, "the block totals fit in the KC tiles");
constexpr float CH_EXP_MAX = 80.f;             // largest exponent the products take
// KC_I starts at row kc_row0(I) of the KC area
__device__ __forceinline__ int kc_row0(int I) { return 8 * I * (I + 1); }
// byte offset of the 16-byte chunk holding channels 8 g .. 8 g + 7 of row r of
// a swizzled operand tile
__device__ __forceinline__ int cp_off(int r, int g) { return r * CP_ROW + 16 * (g ^ (r & 15)); }

__global__ void __launch_bounds__(P_NT, 2)
chunk_prep_channel_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                          const float *__restrict__ g, const float *__restrict__ beta,
                          const int32_t *__restrict__ cu_seqlens, bf16 *__restrict__ ws, int T,
                          int H, int Hk, int N, int nslots)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    float *sRho = reinterpret_cast<float *>(smem + CP_RHO);
    float *sBeta = reinterpret_cast<float *>(smem + CP_BETA);
    float *sNegBeta = sBeta + C;
    int *sFlag = reinterpret_cast<int *>(smem + CP_FLAG);
    float *sTab = reinterpret_cast<float *>(smem + CP_TAB);
    float *sTot = reinterpret_cast<float *>(smem + CP_KC);       // [16][128], before KC
    float *sT = reinterpret_cast<float *>(smem);                 // solve: T over KR, QR
    float *sA = reinterpret_cast<float *>(smem + CP_KC);         // and A over KC
    float *sY = sA + P_SZ_A / 4;

    const int tid0 = (int)threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    const int nitems = (int)prep_nitems(nslots, H);
    const int stride = (int)gridDim.x;
    const int tstride = Hk * DK;

    struct Pre {
        bf16x8 kr[4], qr[4];
        f32x4 gr[8];
        float bv;
    };
    auto fetch = [&](const PrepItem &it, Pre &p) {
        const size_t tok0 = (size_t)it.row0;
        const int c8 = tid0 & 15, tg = tid0 >> 4;
        const unsigned nb = (unsigned)it.nvalid * tstride * 2;
        const size_t hoff = tok0 * tstride + (size_t)(it.h / (H / Hk)) * DK;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)(k + hoff), 0, nb, 0x00020000);
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void *)(q + hoff), 0, nb, 0x00020000);
        const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(g + (tok0 * H + it.h) * DK), 0, (unsigned)it.nvalid * H * DK * 4, 0x00020000);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = 4 * tg + j;
            const unsigned o = (unsigned)((t * tstride + 8 * c8) * 2);
            p.kr[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0));
            p.qr[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, o, 0, 0));
            const unsigned og = (unsigned)(((size_t)t * H * DK + 8 * c8) * 4);
            p.gr[2 * j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, og, 0, 0));
            p.gr[2 * j + 1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, og + 16, 0, 0));
        }
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(beta + tok0 * H + it.h), 0, (unsigned)it.nvalid * H * 4, 0x00020000);
        p.bv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, 4 * H * (tid0 & 63), 0, 0));
    };

    auto item_step = [&](const PrepItem &it, const Pre &p, const PrepItem &nit, Pre &pn,
                         int after, PrepItem &ait) {
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, c8 = tid & 15, tg = tid >> 4;
        const int m = lane & 15, kq = lane >> 4;
        const int I = wave;                    // row block of this wave's tokens and products
        bf16 *dst = ws + ((size_t)it.h * nslots + it.slot) * CH_ITEM_ELEMS;

        // ---- gamma: running sums over the thread's 4 tokens, then the
        //      totals of the earlier token groups ----
        if (it.nvalid == 0) {                  // uniform over the workgroup
            fetch(nit, pn);
            ait = prep_locate(cu_seqlens, after, nitems, T, H, N);
            return;
        }
        float gm[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = e < 4 ? p.gr[2 * j][e] : p.gr[2 * j + 1][e - 4];
                gm[j][e] = j ? gm[j - 1][e] + x : x;
            }
        // the wave's four token groups of the same channels sit 16 lanes
        // apart: an inclusive scan over them by two lane shifts, then the
        // wave totals (row 3) through LDS for the later waves
        float inc[8];
        {
            const int row = (tid & 63) >> 4;
            auto from = [&](int dl, float v) {
                return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                    4 * (((tid & 63) - dl) & 63), __builtin_bit_cast(int, v)));
            };
#pragma unroll
            for (int e = 0; e < 8; ++e) inc[e] = gm[3][e];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float t = from(16, inc[e]);
                if (row >= 1) inc[e] += t;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float t = from(32, inc[e]);
                if (row >= 2) inc[e] += t;
            }
            if (row == 3) {
                *reinterpret_cast<f32x4 *>(sTot + wave * DK + 8 * c8) = f32x4{inc[0], inc[1], inc[2], inc[3]};
                *reinterpret_cast<f32x4 *>(sTot + wave * DK + 8 * c8 + 4) = f32x4{inc[4], inc[5], inc[6], inc[7]};
            }
        }
        if (tid < C) {
            sBeta[tid] = p.bv;
            sNegBeta[tid] = -p.bv;
        }
        if (tid == 0) *sFlag = 0;
        lds_barrier();
        {
            // the group's offset: the earlier groups of its wave, then the
            // totals of the earlier waves
            float off[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) off[e] = inc[e] - gm[3][e];
            for (int w = 0; w < wave; ++w) {   // uniform
                const f32x4 a = *reinterpret_cast<const f32x4 *>(sTot + w * DK + 8 * c8);
                const f32x4 b = *reinterpret_cast<const f32x4 *>(sTot + w * DK + 8 * c8 + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) { off[e] += a[e]; off[4 + e] += b[e]; }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) gm[j][e] += off[e];
            if ((tg & 3) == 3) {               // token 16 (I + 1) - 1: rho_{I+1}
                *reinterpret_cast<f32x4 *>(sRho + I * DK + 8 * c8) = f32x4{gm[3][0], gm[3][1], gm[3][2], gm[3][3]};
                *reinterpret_cast<f32x4 *>(sRho + I * DK + 8 * c8 + 4) = f32x4{gm[3][4], gm[3][5], gm[3][6], gm[3][7]};
            }
        }
        lds_barrier();
        // ---- per-channel tables (rho_0 = 0, rho_4 = gamma_63):
        //      0-2  e^{rho_1}, e^{rho_2}, e^{rho_3}
        //      3-5  e^{rho_2 - rho_1}, e^{rho_3 - rho_2}, e^{rho_4 - rho_3}
        //      6-9  e^{rho_I - rho_{I+1}}, I = 0..3: the inverse of block I's decay,
        //           clamped at e^80; beyond it the item takes the exact
        //           diagonal blocks ----
        //      (all exponents read before any table entry or the flag is
        //      written, so that the five entries of a thread are independent)
        {
            static_assert(10 * DK == 5 * P_NT, "five table entries per thread");
            float ex[5];
            bool big = false;
#pragma unroll
            for (int u = 0; u < 5; ++u) {
                const int x = tid + P_NT * u, id = x / DK, c = x - id * DK;
                const float *r = sRho + c;     // r[(I - 1) * DK] = rho_I
                if (id < 3) ex[u] = r[id * DK];
                else if (id < 6) ex[u] = r[(id - 2) * DK] - r[(id - 3) * DK];
                else {
                    const int I2 = id - 6;
                    const float e2 = (I2 ? r[(I2 - 1) * DK] : 0.f) - r[I2 * DK];
                    big = big || e2 > CH_EXP_MAX;
                    ex[u] = e2 > CH_EXP_MAX ? CH_EXP_MAX : e2;
                }
            }
#pragma unroll
            for (int u = 0; u < 5; ++u) sTab[tid + P_NT * u] = __expf(ex[u]);
            if (big) *sFlag = 1;
        }
        if (tg == 0) {                         // e^{gamma_63} of the thread's channels
            float *ec = reinterpret_cast<float *>(dst + CH_EC) + 8 * c8;
            const float *r4 = sRho + 3 * DK + 8 * c8;
            *reinterpret_cast<f32x4 *>(ec) = f32x4{__expf(r4[0]), __expf(r4[1]), __expf(r4[2]), __expf(r4[3])};
            *reinterpret_cast<f32x4 *>(ec + 4) = f32x4{__expf(r4[4]), __expf(r4[5]), __expf(r4[6]), __expf(r4[7])};
        }
        lds_barrier();
        // ---- the scaled copies of the thread's elements (wave I: tokens of
        //      row block I; specialised per block so that only its copies are
        //      formed). The operands of the diagonal block (I, I) of P are also
        //      split into bf16 hi + lo parts; the lo parts stay in registers ----
        bf16x8 qlo[4], dlo[4];
        auto scaled_copies = [&](auto IC) {
            constexpr int BI = decltype(IC)::value;
            auto tab = [&](int id, int e) { return sTab[id * DK + 8 * c8 + e]; };
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 4 * tg + j;
                // per channel: rho_I, rho_{I+1}, e^{rho_I}, e^{rho_4 - rho_{I+1}} (K^),
                // e^{rho_I - rho_{I+1}}, e^{rho_{I+2} - rho_{I+1}}, e^{rho_3 - rho_1};
                // read again for each token (the clobber keeps them from being
                // held in registers over the four)
                asm volatile("" ::: "memory");
                float rho0[8], rho1[8], eI[8], gI[8], dI[8], fI2[8], f31[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    rho0[e] = BI ? sRho[(BI - 1) * DK + 8 * c8 + e] : 0.f;
                    rho1[e] = sRho[BI * DK + 8 * c8 + e];
                    eI[e] = BI ? tab(BI - 1, e) : 1.f;
                    const float f21 = tab(3, e), f32 = tab(4, e), g3 = tab(5, e);
                    gI[e] = BI == 3 ? 1.f : BI == 2 ? g3 : BI == 1 ? g3 * f32 : g3 * f32 * f21;
                    dI[e] = tab(6 + BI, e);
                    fI2[e] = BI == 0 ? f21 : f32;
                    f31[e] = f21 * f32;
                }
                bf16x8 kr, qr, kd, kp, kh, qp, kc1, kc2, kc3;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float rf = __expf(gm[j][e] - rho0[e]);
                    const float nf = __expf(rho1[e] - gm[j][e]);
                    const float E = eI[e] * rf;
                    const float kk = (float)p.kr[j][e], qq2 = (float)p.qr[j][e];
                    const float vq = qq2 * rf, vd = kk * nf * dI[e];   // e^{rho_I - gamma}
                    kr[e] = (bf16)(kk * rf);
                    qr[e] = (bf16)vq;
                    kd[e] = (bf16)vd;
                    qlo[j][e] = (bf16)(vq - (float)qr[e]);
                    dlo[j][e] = (bf16)(vd - (float)kd[e]);
                    kp[e] = (bf16)(kk * E);
                    qp[e] = (bf16)(qq2 * E);
                    kh[e] = (bf16)(kk * nf * gI[e]);
                    if constexpr (BI <= 2) kc1[e] = (bf16)(kk * nf);            // KC_{I+1}
                    if constexpr (BI <= 1) kc2[e] = (bf16)(kk * nf * fI2[e]);   // KC_{I+2}
                    if constexpr (BI == 0) kc3[e] = (bf16)(kk * nf * f31[e]);   // KC_3
                }
                *reinterpret_cast<bf16x8 *>(smem + CP_KR + cp_off(t, c8)) = kr;
                *reinterpret_cast<bf16x8 *>(smem + CP_QR + cp_off(t, c8)) = qr;
                *reinterpret_cast<bf16x8 *>(smem + CP_KC + cp_off(kc_row0(BI) + t, c8)) = kd;
                if constexpr (BI <= 2) *reinterpret_cast<bf16x8 *>(smem + CP_KC + cp_off(kc_row0(BI + 1) + t, c8)) = kc1;
                if constexpr (BI <= 1) *reinterpret_cast<bf16x8 *>(smem + CP_KC + cp_off(kc_row0(BI + 2) + t, c8)) = kc2;
                if constexpr (BI == 0) *reinterpret_cast<bf16x8 *>(smem + CP_KC + cp_off(kc_row0(3) + t, c8)) = kc3;
                *reinterpret_cast<bf16x8 *>(dst + CH_KP + t * DK + 8 * c8) = kp;
                *reinterpret_cast<bf16x8 *>(dst + CH_KH + t * DK + 8 * c8) = kh;
                const int f = 4 * (t >> 4) + (c8 >> 2), ln = 16 * (c8 & 3) + (t & 15);
                *reinterpret_cast<bf16x8 *>(dst + CH_QP + 512 * f + 8 * ln) = qp;
            }
        };
        // wave 0 writes the most copies (KC_1 .. KC_3 besides its own): it
        // goes first in issue arbitration
        if (I == 0) __builtin_amdgcn_s_setprio(1);
        switch (I) {
        case 0: scaled_copies(std::integral_constant<int, 0>{}); break;
        case 1: scaled_copies(std::integral_constant<int, 1>{}); break;
        case 2: scaled_copies(std::integral_constant<int, 2>{}); break;
        default: scaled_copies(std::integral_constant<int, 3>{}); break;
        }
        __builtin_amdgcn_s_setprio(0);
        // ---- wave I, diagonal block (I, I) of M (dM) and of P^T (dP). Its
        //      operands are rows this wave wrote and only it reads, so it is
        //      summed before the workgroup barrier. P's block is summed as
        //      hi hi + hi lo + lo hi, which keeps fp32-level products: with
        //      bf16 operands alone an entry loses its relative precision where
        //      q_i k_j nearly cancels, and P weights the outputs directly (a
        //      one-token sequence's output is P_00 Delta_0). M's block enters
        //      the outputs only through T, against v, and keeps bf16 operands.
        //      ak, aq (rows 16 I + m of KR, QR) stay in registers for the
        //      off-diagonal blocks; the lo parts are written over the QR and
        //      KC rows once these are read ----
        unsigned char *kcI = smem + CP_KC + kc_row0(I) * CP_ROW;
        bf16x8 ak[4], aq[4];
        f32x4 dM = f32x4{0.f, 0.f, 0.f, 0.f}, dP = dM;
        {
            bf16x8 bd[4];
            wave_lds_order();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int gr = 4 * s + kq;
                ak[s] = *reinterpret_cast<const bf16x8 *>(smem + CP_KR + cp_off(16 * I + m, gr));
                aq[s] = *reinterpret_cast<const bf16x8 *>(smem + CP_QR + cp_off(16 * I + m, gr));
                bd[s] = *reinterpret_cast<const bf16x8 *>(kcI + cp_off(16 * I + m, gr));
                dM = mfma16(ak[s], bd[s], dM);
                dP = mfma16(bd[s], aq[s], dP);
            }
            wave_lds_order();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 4 * tg + j;
                *reinterpret_cast<bf16x8 *>(smem + CP_QR + cp_off(t, c8)) = qlo[j];
                *reinterpret_cast<bf16x8 *>(kcI + cp_off(t, c8)) = dlo[j];
            }
            wave_lds_order();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int gr = 4 * s + kq;
                const bf16x8 ql = *reinterpret_cast<const bf16x8 *>(smem + CP_QR + cp_off(16 * I + m, gr));
                const bf16x8 dl = *reinterpret_cast<const bf16x8 *>(kcI + cp_off(16 * I + m, gr));
                dP = mfma16(dl, aq[s], mfma16(bd[s], ql, dP));
            }
        }
        // the item's loads are consumed: the next item's are issued now and
        // overlap the products, the solve and the stores
        fetch(nit, pn);
        ait = prep_locate(cu_seqlens, after, nitems, T, H, N);
        lds_barrier();
        // waves with more column blocks ahead of the next barrier go first
        if (I == 3) __builtin_amdgcn_s_setprio(2);
        else if (I == 2) __builtin_amdgcn_s_setprio(1);
        // ---- wave I: off-diagonal blocks J < I of row block I of M (accM[J])
        //      and of P^T (accP[J], rows = keys 16 J + .., columns = queries
        //      16 I + ..) ----
        f32x4 accM[3], accP[3];
#pragma unroll
        for (int J = 0; J < 3; ++J) { accM[J] = f32x4{0.f, 0.f, 0.f, 0.f}; accP[J] = accM[J]; }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int gr = 4 * s + kq;
#pragma unroll
            for (int J = 0; J < 3; ++J) {
                if (J >= I) break;             // uniform
                const bf16x8 b = *reinterpret_cast<const bf16x8 *>(kcI + cp_off(16 * J + m, gr));
                accM[J] = mfma16(ak[s], b, accM[J]);
                accP[J] = mfma16(b, aq[s], accP[J]);
            }
        }
        lds_barrier();                         // operand tiles read
        if (*sFlag) {
            // ---- exact diagonal blocks (rare: a channel decays by more than
            //      e^-80 inside a 16-token block). k, q and g of the item are
            //      read again from memory (the registers hold the next item's),
            //      gamma is summed per channel into LDS, then lane (n, qq) of
            //      wave I sums entries (4 qq + r, n) of block (I, I) with one
            //      exponential per channel ----
            float *sG = reinterpret_cast<float *>(smem);              // [64][128] fp32
            bf16 *sKr = reinterpret_cast<bf16 *>(smem + C * DK * 4);  // [64][128]
            bf16 *sQr = sKr + C * DK;
            const size_t kqh = (size_t)it.row0 * tstride + (size_t)(it.h / (H / Hk)) * DK;
            for (int x = tid; x < C * DK / 8; x += P_NT) {
                const int t = x >> 4, cg = x & 15;
                const bool ok = t < it.nvalid;
                *reinterpret_cast<bf16x8 *>(sKr + t * DK + 8 * cg) =
                    ok ? *reinterpret_cast<const bf16x8 *>(k + kqh + (size_t)t * tstride + 8 * cg) : bf16x8{};
                *reinterpret_cast<bf16x8 *>(sQr + t * DK + 8 * cg) =
                    ok ? *reinterpret_cast<const bf16x8 *>(q + kqh + (size_t)t * tstride + 8 * cg) : bf16x8{};
            }
            if (tid < DK) {
                const float *gp = g + ((size_t)it.row0 * H + it.h) * DK + tid;
                float run = 0.f;
                for (int t = 0; t < C; ++t) {
                    run += t < it.nvalid ? gp[(size_t)t * H * DK] : 0.f;
                    sG[t * DK + tid] = run;
                }
            }
            lds_barrier();
            const int jn = 16 * I + m;         // key (column of M, row of P^T)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int iq = 16 * I + 4 * kq + r;   // query/key row of M
                float sm = 0.f, sp = 0.f;
                if (jn < iq) {                 // M[iq][jn]
                    for (int c = 0; c < DK; ++c)
                        sm += (float)sKr[iq * DK + c] * (float)sKr[jn * DK + c] *
                              __expf(sG[iq * DK + c] - sG[jn * DK + c]);
                }
                // P^T[key 16 I + 4 kq + r][query 16 I + m] = P[query][key]
                const int qi = 16 * I + m, kj = 16 * I + 4 * kq + r;
                if (kj <= qi) {
                    for (int c = 0; c < DK; ++c)
                        sp += (float)sQr[qi * DK + c] * (float)sKr[kj * DK + c] *
                              __expf(sG[qi * DK + c] - sG[kj * DK + c]);
                }
                dM[r] = sm;
                dP[r] = sp;
            }
            lds_barrier();                     // scratch read before A is written over it
        }
        // ---- A = -strict_lower(diag(beta) M) into sY (diagonal blocks) and
        //      sA (rows 16-63, columns 0-47); P (queries x keys, lower incl.)
        //      straight to the workspace ----
        float nbeta[4];                        // -beta of rows 16 I + 4 kq + r, read once
#pragma unroll
        for (int r = 0; r < 4; ++r) nbeta[r] = sNegBeta[16 * I + 4 * kq + r];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            if (J > I) break;
            const f32x4 aM = J == I ? dM : accM[J < 3 ? J : 0], aP = J == I ? dP : accP[J < 3 ? J : 0];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * I + 4 * kq + r, j = 16 * J + m;
                const float a = j < i ? nbeta[r] * aM[r] : 0.f;
                if (J == I) sY[I * P_DB + (4 * kq + r) * 16 + m] = a;
                else if (j < 48) sA[(i - 16) * P_LD_A2 + j] = a;
            }
            // P^T accumulator r: key 16 J + 4 kq + r, query 16 I + m
            const int qi = 16 * I + m;
            bf16x4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = (bf16)(16 * J + 4 * kq + r <= qi ? aP[r] : 0.f);
            bf16 *prow = dst + CH_P + (qi < 32 ? 32 * qi : 1024 + 64 * (qi - 32));
            *reinterpret_cast<bf16x4 *>(prow + 16 * J + 4 * kq) = x;
        }
        if (I == 0 || I == 2) {                // keys 16 I + 16 .. 16 I + 31 of these rows are stored: zero
            const int qi = 16 * I + m;
            bf16 *prow = dst + CH_P + (qi < 32 ? 32 * qi : 1024 + 64 * (qi - 32));
            *reinterpret_cast<bf16x4 *>(prow + 16 * (I + 1) + 4 * kq) = bf16x4{};
        }
        __builtin_amdgcn_s_setprio(0);
        lds_barrier();                         // A complete
        solve_store(sA, sY, sT, sBeta, dst, tid, wave);
        lds_barrier();                         // T and the scalars read before the next item
    };

    const int first = (int)blockIdx.x;
    PrepItem it = prep_locate(cu_seqlens, first, nitems, T, H, N);
    PrepItem nit = prep_locate(cu_seqlens, first + stride, nitems, T, H, N);
    Pre pre;
    fetch(it, pre);
    for (int item = first; item < nitems; item += stride) {
        PrepItem ait;
        item_step(it, pre, nit, pre, item + 2 * stride, ait);
        it = nit;
        nit = ait;
    }
}

// ---------------------------------------------------------------------------
// One wave's solve of one (chunk, head): T_u = (I - A)^-1 diag(beta) with
// A = -strict_lower(diag(beta) K K^T * Gamma), Gamma_ij = e^{gamma_i - gamma_j}
// ("5. Linear Attention", chunked delta rule, stage 1), in SV_BYTES of LDS
// that no other wave touches and no workgroup barrier:
//   phase1  gamma = prefix sum of g; the ten Gram blocks (I, J), J <= I, of
//           K K^T on the bf16 matrix cores (K given in operand order); A
//           row-major into the blocks; the diagonal blocks D_b = (I - A_bb)^-1
//           by forward substitution, in place
//   phase2  the off-diagonal blocks of T by two levels of 2 x 2 block
//           inversion on split bf16 products (mm16x), in place
//   emit    T diag(beta) as 384 bf16 pieces of 8 row elements: pieces
//           0..255 rows 32-63 (8 per row), 256..383 rows 0-31, columns 0-31
//           (4 per row), handed to sink(piece, value)
// Rows past the chunk's valid tokens have k = 0, g = 0, beta = 0 and come
// out as identity rows of T and zero columns of T_u.
// ---------------------------------------------------------------------------
struct WaveSolver {
    float *sv;
    __device__ float *blk(int I, int J) const {
        return I == J ? sv + I * SV_DIAG : sv + SV_OFF0 + (I * (I - 1) / 2 + J) * SV_BLK;
    }
    __device__ float *gl() const { return sv + SV_OFF0 + 6 * SV_BLK; }          // gamma log2(e)
    __device__ float *be() const { return gl() + C; }                           // beta

    // K rows 16 I + lane % 16, columns 32 s + 8 (lane / 16) .. of a chunk whose
    // first row is `krow` (rows tstride elements apart), and g, beta of token
    // `lane` (H floats apart); rows past `nrow` read as zero
    __device__ static void fetch(const bf16 *krow, int tstride, const float *grow,
                                 const float *brow, int H, int nrow, int lane,
                                 bf16x8 (&kr)[4][4], float &gv, float &bv) {
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void *)krow, 0, (unsigned)nrow * tstride * 2, 0x00020000);
        const unsigned off = (unsigned)(((lane & 15) * tstride + 8 * (lane >> 4)) * 2);
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
                kr[I][s2] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                rk, off, (unsigned)((16 * I * tstride + 32 * s2) * 2), 0));
        const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
            (void *)grow, 0, (unsigned)nrow * H * 4, 0x00020000);
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            (void *)brow, 0, (unsigned)nrow * H * 4, 0x00020000);
        gv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, 4 * H * lane, 0, 0));
        bv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, 4 * H * lane, 0, 0));
    }
    // accumulator layout (lane (q, m) holds rows 4 q + r of column m) -> row-major block
    __device__ static void store_blk(float *p, f32x4 acc, int lane) {
        const int m = lane & 15, qq = lane >> 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) p[(4 * qq + r) * SV_LD + m] = acc[r];
    }
    __device__ void phase1(const bf16x8 (&kr)[4][4], float gv, float bv, int lane) const {
        float *sgl = gl(), *sbe = be();
        const int m = lane & 15, qq = lane >> 4;
        const float gam = wave_inclusive_scan(gv);
        sgl[lane] = gam * 1.4426950408889634f;
        sbe[lane] = bv;
        // Gram blocks (I, J), J <= I: G[16 I + 4 q + r][16 J + m]
        f32x4 G[10];
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int J = 0; J <= I; ++J) {
                f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) a = mfma16(kr[I][s2], kr[J][s2], a);
                G[I * (I + 1) / 2 + J] = a;
            }
        wave_lds_order();
        // A_ij = -beta_i G_ij e^{gamma_i - gamma_j} for j < i (each
        // exponent <= 0), zero elsewhere; row-major into the blocks
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const f32x4 gli = *reinterpret_cast<const f32x4 *>(sgl + 16 * I + 4 * qq);
            const f32x4 bi = *reinterpret_cast<const f32x4 *>(sbe + 16 * I + 4 * qq);
#pragma unroll
            for (int J = 0; J <= I; ++J) {
                const float glj = sgl[16 * J + m];
                f32x4 a = G[I * (I + 1) / 2 + J];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = __builtin_amdgcn_exp2f(gli[r] - glj);
                    a[r] = (J < I || m < 4 * qq + r) ? -(bi[r] * a[r]) * e : 0.f;
                }
                store_blk(blk(I, J), a, lane);
            }
        }
        wave_lds_order();
        // diagonal blocks, one per 16 lanes: lane 16 b + c computes
        // column c of D_b = (I - A_bb)^-1 row by row,
        // D[i][c] = [i == c] + sum_{j < i} A[i][j] D[j][c]
        // (row i + 1 read while row i is summed)
        const int bb = lane >> 4, c = lane & 15;
        const float *Ab = blk(bb, bb);
        float D[16];
        f32x4 rowv[2][4];
        auto load_row = [&](int i, f32x4 (&dstv)[4]) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (4 * t < i) dstv[t] = *reinterpret_cast<const f32x4 *>(Ab + i * SV_LD + 4 * t);
        };
        load_row(1, rowv[1]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i + 1 < 16) load_row(i + 1, rowv[(i + 1) & 1]);
            float acc = i == c ? 1.f : 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * t + e < i) acc += rowv[i & 1][t][e] * D[4 * t + e];
            D[i] = acc;
        }
        wave_lds_order();
        // D_b row-major in place (its columns, right-hand operands below,
        // are read as four single elements per lane)
        float *Db = blk(bb, bb);
#pragma unroll
        for (int i = 0; i < 16; ++i) Db[i * SV_LD + c] = D[i];
        wave_lds_order();
    }
    __device__ void phase2(int lane) const {
        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
        const int m = lane & 15, qq = lane >> 4;
        // With D_b the diagonal inverses:
        //   T10 = D1 A10 D0,  T32 = D3 A32 D2,  T21 = D2 A21 D1
        //   T20 = D2 (A20 D0 + A21 T10)
        //   T31 = T32 (A21 D1) + D3 (A31 D1)
        //   T30 = T32 (A20 D0 + A21 T10) + D3 (A30 D0 + A31 T10)
        // Left factors are row pieces of row-major blocks, right
        // factors column pieces of the row-major D_b or accumulators.
        auto piece = [&](const float *p, int ld) {
            return *reinterpret_cast<const f32x4 *>(p + m * ld + 4 * qq);
        };
        auto colpiece = [&](const float *p) {
            return f32x4{p[(4 * qq) * SV_LD + m], p[(4 * qq + 1) * SV_LD + m],
                         p[(4 * qq + 2) * SV_LD + m], p[(4 * qq + 3) * SV_LD + m]};
        };
        const LSplit lA10 = lsplit(piece(blk(1, 0), SV_LD)), lA32 = lsplit(piece(blk(3, 2), SV_LD));
        const LSplit lA21 = lsplit(piece(blk(2, 1), SV_LD)), lA20 = lsplit(piece(blk(2, 0), SV_LD));
        const LSplit lA31 = lsplit(piece(blk(3, 1), SV_LD)), lA30 = lsplit(piece(blk(3, 0), SV_LD));
        const LSplit lD1 = lsplit(piece(blk(1, 1), SV_LD)), lD2 = lsplit(piece(blk(2, 2), SV_LD));
        const LSplit lD3 = lsplit(piece(blk(3, 3), SV_LD));
        const bf16x8 rD0 = rsplit(colpiece(blk(0, 0))), rD1 = rsplit(colpiece(blk(1, 1)));
        const bf16x8 rD2 = rsplit(colpiece(blk(2, 2)));
        const f32x4 u10 = mm16x(z4, lA10, rD0);
        const f32x4 u32 = mm16x(z4, lA32, rD2);
        const bf16x8 X = rsplit(mm16x(z4, lA21, rD1));         // A21 D1
        const f32x4 W0 = mm16x(z4, lA20, rD0);                 // A20 D0
        const bf16x8 Z = rsplit(mm16x(z4, lA31, rD1));         // A31 D1
        const f32x4 V0 = mm16x(z4, lA30, rD0);                 // A30 D0
        const f32x4 t10 = mm16x(z4, lD1, rsplit(u10));
        const f32x4 t32 = mm16x(z4, lD3, rsplit(u32));
        const f32x4 t21 = mm16x(z4, lD2, X);
        const bf16x8 rT10 = rsplit(t10);
        const bf16x8 W = rsplit(mm16x(W0, lA21, rT10));        // + A21 T10
        const bf16x8 V = rsplit(mm16x(V0, lA31, rT10));        // + A31 T10
        const f32x4 t20 = mm16x(z4, lD2, W);
        // T32 is a left factor next: through its block (A32 is read)
        store_blk(blk(3, 2), t32, lane);
        wave_lds_order();
        const LSplit lT32 = lsplit(piece(blk(3, 2), SV_LD));
        const f32x4 t31 = mm16x(mm16x(z4, lT32, X), lD3, Z);
        const f32x4 t30 = mm16x(mm16x(z4, lT32, W), lD3, V);
        store_blk(blk(1, 0), t10, lane);
        store_blk(blk(2, 1), t21, lane);
        store_blk(blk(2, 0), t20, lane);
        store_blk(blk(3, 1), t31, lane);
        store_blk(blk(3, 0), t30, lane);
        wave_lds_order();
    }
    template <typename Sink> __device__ void emit(int lane, Sink &&sink) const {
        const float *sbe = be();
        // T diag(beta) as bf16 pieces of 8 row elements: pieces
        // 0..255 rows 32-63 (8 per row), 256..383 rows 0-31, columns
        // 0-31 (4 per row); blocks above the diagonal are zero
#pragma unroll
        for (int u6 = 0; u6 < 6; ++u6) {
            const int e = lane + 64 * u6;
            const int i = u6 < 4 ? 32 + (e >> 3) : (e - 256) >> 2;
            const int gc = u6 < 4 ? e & 7 : e & 3;
            const int I = i >> 4, J = gc >> 1;
            const float *tp = blk(I, J < I ? J : I) + (i & 15) * SV_LD + 8 * (gc & 1);
            const f32x4 t0 = *reinterpret_cast<const f32x4 *>(tp);
            const f32x4 t1 = *reinterpret_cast<const f32x4 *>(tp + 4);
            const f32x4 b0 = *reinterpret_cast<const f32x4 *>(sbe + 8 * gc);
            const f32x4 b1 = *reinterpret_cast<const f32x4 *>(sbe + 8 * gc + 4);
            bf16x8 outp;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                outp[e2] = (bf16)(J <= I ? t0[e2] * b0[e2] : 0.f);
                outp[e2 + 4] = (bf16)(J <= I ? t1[e2] * b1[e2] : 0.f);
            }
            sink(e, outp);
        }
    }
};

// ---------------------------------------------------------------------------
// chunk_solve: the first pass of the two-pass path with a scalar gate. One
// wave per workgroup and (chunk, head) item at a time (items blockIdx.x,
// + gridDim.x, ...), each wave with its own SV_BYTES of LDS, so that up to
// twelve items are in flight per compute unit (three waves per SIMD, which
// its register count is held to) and none waits at a workgroup barrier.
// Writes T_u = T diag(beta) of the item into the workspace. With PREFETCH
// each item's keys are requested while the item before it is solved (more
// registers: eight waves per CU), which pays once the plain kernel's grid
// would need a second round of items.
// ---------------------------------------------------------------------------
constexpr int SOLVE_NT = 64;
template <bool PREFETCH>
__global__ void __launch_bounds__(SOLVE_NT) __attribute__((amdgpu_waves_per_eu(PREFETCH ? 2 : 3)))
chunk_solve_kernel(const bf16 *__restrict__ k, const float *__restrict__ g,
                   const float *__restrict__ beta, const int32_t *__restrict__ cu_seqlens,
                   bf16 *__restrict__ ws, int T, int H, int Hk, int N, int nslots)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const WaveSolver sol{reinterpret_cast<float *>(smem)};
    const int lane = (int)threadIdx.x;
    const int nitems = (int)prep_nitems(nslots, H);
    const int tstride = Hk * DK;
    const int stride = (int)gridDim.x;
    auto fetch_item = [&](const PrepItem &it, bf16x8 (&kr)[4][4], float &gv, float &bv) {
        const size_t tok0 = (size_t)it.row0;
        WaveSolver::fetch(k + tok0 * tstride + (size_t)(it.h / (H / Hk)) * DK, tstride,
                          g + tok0 * H + it.h, beta + tok0 * H + it.h, H, it.nvalid, lane, kr,
                          gv, bv);
    };
    auto solve_item = [&](const PrepItem &it, const bf16x8 (&kr)[4][4], float gv, float bv) {
        sol.phase1(kr, gv, bv, lane);
        sol.phase2(lane);
        bf16 *dst = ws + ((size_t)it.h * nslots + it.slot) * ITEM_ELEMS;
        sol.emit(lane, [&](int e, bf16x8 p) { *reinterpret_cast<bf16x8 *>(dst + 8 * e) = p; });
        wave_lds_order();                      // the blocks read before the next item writes them
    };
    if constexpr (!PREFETCH) {
        for (int item = (int)blockIdx.x; item < nitems; item += stride) {
            const PrepItem it = prep_locate(cu_seqlens, item, nitems, T, H, N);
            if (it.nvalid == 0) continue;      // uniform
            bf16x8 kr[4][4];
            float gv, bv;
            fetch_item(it, kr, gv, bv);
            solve_item(it, kr, gv, bv);
        }
    } else {
        // the next item with work at or after `from` (unused slots skipped)
        auto next_item = [&](int from, PrepItem &it) {
            int item = from;
            while (item < nitems) {
                it = prep_locate(cu_seqlens, item, nitems, T, H, N);
                if (it.nvalid != 0) break;     // uniform
                item += stride;
            }
            return item;
        };
        PrepItem it;
        int item = next_item((int)blockIdx.x, it);
        if (item >= nitems) return;
        bf16x8 kr[4][4];
        float gv, bv;
        fetch_item(it, kr, gv, bv);
        while (true) {
            PrepItem itn;
            const int nxt = next_item(item + stride, itn);
            bf16x8 krn[4][4];
            float gvn = 0.f, bvn = 0.f;
            if (nxt < nitems) fetch_item(itn, krn, gvn, bvn);
            solve_item(it, kr, gv, bv);
            if (nxt >= nitems) break;
            item = nxt;
            it = itn;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) kr[i][j] = krn[i][j];
            gv = gvn;
            bv = bvn;
        }
    }
}

// ---------------------------------------------------------------------------
// chunk_chain: the sequential pass. One workgroup of 8 waves per (32-wide d_v
// tile, head, sequence), one LDS barrier per chunk.
//
// Waves 0 and 1 carry the recurrence, each for 16 of the tile's d_v columns:
// the wave keeps its slice of S^T (128 x 16, fp32) in eight 16x16 MFMA
// accumulators for the whole sequence, and per chunk computes
//   X     = K S^T                       (B operand: the state accumulators)
//   R     = V - diag(e^gamma) X         (vector ALU, on X's accumulators)
//   Delta = T_u R                       (B operand: R from X's accumulators)
//   S^T  <- e^{gamma_63} S^T + K^T Delta~,  Delta~_j = e^{gamma_63 - gamma_j} Delta_j
//                                       (B operand: Delta~'s accumulators)
// entirely in registers: an accumulator pair holds rows 4 (lane/16) + r of
// two 16-row tiles, which is a B operand over that row order, and the A
// operands are read in the matching order (K rows for X chosen per lane,
// K^T for the update transposed on read). T_u (V - diag(e^gamma) K S^T) is
// "5. Linear Attention"'s U - W S^T with W = T diag(beta e^gamma) K: neither
// W nor U is formed.
// Waves 2 and 3 form the output, each for two of the chunk's four 16-token
// tiles (wave 2 tiles 0 and 3, wave 3 tiles 1 and 2: equal work) over all 32
// columns of the tile: O^T = (S Q^T) diag(e^gamma) + Delta^T P^T, the second
// term one chunk later. P^T = upper_incl(K Q^T * Gamma^T) is formed from the
// staged K and Q tiles by staging waves 6 and 7 (the two that share SIMDs
// with waves 2 and 3 and have the least to stage), for the token tiles of
// wave 2 and wave 3 respectively, and passed to them as their B-operand
// registers through a P copy; the in-chain solve (no room for the copies)
// leaves P^T to the output waves, which then take its Q operand from S Q^T's
// and hold it in registers until Delta arrives. The rows of S and Delta^T are
// taken in an order that leaves 8 consecutive d_v of one token in each lane,
// stored as 16 bytes. With a per-channel decay P comes from the workspace
// instead (its decay is per channel) and waves 2 and 3 take tokens 0-31 and
// 32-63. Waves 4-7 stage the next chunk.
//
// Iteration c (buffers b = c % 2):
//   waves 0-1  recurrence step of chunk c: reads staging b, writes Delta^T
//              into copy b and the new bf16 S into copy (c + 1) % 2
//   waves 2-3  S Q^T of chunk c (S copy b, staging b); finish chunk c - 1
//              (Delta^T and P copies (c - 1) % 2) and store its output rows
//   waves 4-7  store chunk c + 1 (in registers since iteration c - 2) into
//              staging (c + 1) % 2, load chunk c + 3 into the registers
//   waves 6-7  (scalar gate) then P^T of chunk c from staging b into P copy b
//   waves 4-5  (per-channel decay) P of chunk c, loaded in iteration c - 2,
//              into copy b
//   barrier
// Tokens past the end of a sequence are identity steps (q = k = v = 0,
// g = 0, and T_u vanishes on them) and their outputs are not stored.
// ---------------------------------------------------------------------------
template <bool PERCH, bool FUSED>
__global__ void __launch_bounds__(NT, 1)
chunk_chain_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                   const bf16 *__restrict__ v, const float *__restrict__ g,
                   const float *__restrict__ beta,
                   const bf16 *__restrict__ ws, const float *s_init, float *s_final,
                   bf16 *__restrict__ o, const int32_t *__restrict__ cu_seqlens,
                   const SegJob *__restrict__ jobs, int T, int H, int Hk, int npairs, int nslots,
                   float scale, int flags)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    bf16 *lds = reinterpret_cast<bf16 *>(smem);
    // tiles of staging buffer b, and copies b of the tiles passed between waves
    auto stQ = [&](int b) { return lds + (OFF_BUF + b * SZ_BUF + B_Q) / 2; };
    auto stK = [&](int b) { return lds + (OFF_BUF + b * SZ_BUF + B_K) / 2; };
    auto stV = [&](int b) { return lds + (OFF_BUF + b * SZ_BUF + B_V) / 2; };
    auto stTH = [&](int b) { return lds + (OFF_BUF + b * SZ_BUF + B_TH) / 2; };   // [32][LD_H]
    auto stTL = [&](int b) { return lds + (OFF_BUF + b * SZ_BUF + B_TL) / 2; };   // [32][LD_L]
    auto stSc = [&](int b) { return reinterpret_cast<float *>(smem + OFF_BUF + b * SZ_BUF + B_SC); };
    using L = ChainLds<PERCH, FUSED>;
    auto cpP = [&](int b) { return lds + (L::P + b * SZ_P) / 2; };
    auto cpS = [&](int b) { return lds + (L::S + b * SZ_S) / 2; };
    auto cpDt = [&](int b) { return lds + (L::DT + b * SZ_DT) / 2; };
    constexpr bool PST = L::PST;
    // P^T register pb[x][s] of the output wave for token tiles {t, 3 - t}
    // (x = 0: tile t, x = 1: tile 3 - t; s: key block) in P copy b: one
    // lane-linear 1 KiB slab each, three per output wave
    auto cpPB = [&](int b, int t, int x, int s) {
        return lds + (L::P + b * SZ_PB) / 2 + 512 * (3 * t + (x ? 1 + s : 0));
    };

    const int tid0 = (int)threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    int pair, tile;                          // (sequence, head) pair and d_v tile
    if (!pair_tile((int)blockIdx.x, npairs, pair, tile)) return;   // uniform
    // packed sequences are dealt longest first (staging buffer 0 is free
    // until the loaders' first store, two barriers into the loop)
    const int h = pair % H, nsq = npairs / H;
    const size_t hstate = (size_t)h * DV * DK;
    int n;
    const float *sin = nullptr;              // this head's start state, or NULL (zero)
    float *sfin = nullptr;                   // ... end state, or NULL
    bf16 *out = o;                           // NULL: no outputs
    if (jobs) {                              // job table: one entry per pair / H
        const SegJob jb = jobs[pair / H];
        if (jb.seg < 0) return;              // uniform
        n = jb.seg;
        flags = jb.flags;
        sin = jb.init ? jb.init + hstate : nullptr;
        sfin = jb.fin ? jb.fin + hstate : nullptr;
        if (!(flags & CHAIN_OUTPUT)) out = nullptr;
    } else {
        n = (cu_seqlens && nsq <= RANK_MAX)
            ? seq_of_rank(cu_seqlens, nsq, T, pair / H, reinterpret_cast<int *>(smem + OFF_BUF))
            : pair / H;
        const size_t sbase = (size_t)n * H * DV * DK + hstate;
        sin = s_init ? s_init + sbase : nullptr;
        sfin = s_final ? s_final + sbase : nullptr;
    }
    const int cbase = tile * DVT;

    long bos, eos;
    seq_bounds(cu_seqlens, n, T, bos, eos);
    const int len = (int)(eos - bos);
    const int nchunks = (len + C - 1) / C;
    // workspace item stride: the per-channel item also holds P, K+, K^, Q+ and
    // the chunk's per-channel decay
    constexpr int IST = PERCH ? CH_ITEM_ELEMS : ITEM_ELEMS;
    const bf16 *wsh = ws + ((size_t)h * nslots + (size_t)((bos >> 6) + n)) * IST;
    const int lane0 = tid0 & 63;

    // ---- state: wave hv < 2 holds Sacc[d][r] = S[cbase + 16 hv + lane%16][dk(d, lane/16, r)]
    //      with dk(d, q, r) = 32 (d/2) + 8 q + 4 (d%2) + r: accumulator pair (2s, 2s+1)
    //      then covers d_k 32 s + 8 q + 0..7 contiguously (see the state update)
    f32x4 Sacc[8];
    bf16x8 Sb[4];                           // the same as four bf16 B operands (32 d_k each)
#pragma unroll
    for (int d = 0; d < 8; ++d) Sacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (wave < 2) {
        const int m = lane0 & 15, qq = lane0 >> 4;
        const int col = cbase + 16 * wave + m;
        if (flags & CHAIN_INIT_IDENTITY) {
            // S = I: this lane's entries S[col][32 (d/2) + 8 qq + 4 (d%2) + r]
#pragma unroll
            for (int d = 0; d < 8; ++d)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Sacc[d][r] = (32 * (d >> 1) + 8 * qq + 4 * (d & 1) + r == col) ? 1.f : 0.f;
        } else if (sin) {
#pragma unroll
            for (int d = 0; d < 8; ++d)
                Sacc[d] = *reinterpret_cast<const f32x4 *>(sin + (size_t)col * DK + 32 * (d >> 1) + 8 * qq + 4 * (d & 1));
        }
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) Sb[s2] = acc_pair_bf16(Sacc[2 * s2], Sacc[2 * s2 + 1]);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            bf16x4 x = {(bf16)Sacc[d][0], (bf16)Sacc[d][1], (bf16)Sacc[d][2], (bf16)Sacc[d][3]};
            *reinterpret_cast<bf16x4 *>(cpS(0) + (16 * wave + m) * LD_R + ((32 * (d >> 1) + 8 * qq + 4 * (d & 1)) ^ swS(16 * wave + m))) = x;
        }
    }

    // ---- loads of one chunk into registers, by waves 4-7 (wi = wave - 4), as
    //      16-byte buffer loads per lane:
    //        b[0..7]  Q (wi 0, 1) or K (wi 2, 3) rows 32 (wi % 2) + lane/16 + 4 r,
    //                 columns 8 (lane % 16) ..
    //        t[0..2]  (wi 0, 1) workspace pieces 192 wi + 64 r + lane of T_u
    //        v[0..1]  (wi 2, 3) V rows lane/4 + 16 (2 (wi - 2) + r), 8 columns of
    //                 this tile
    //        g        (wi 3) g of token lane
    //      A buffer resource per chunk spans the chunk's tokens inside the
    //      sequence only: loads past its end read as zero, which turns tokens
    //      past the end into identity steps with no clamping or masking.
    //      Workspace piece order (8 bf16 each): 0..255 rows 32-63 of T_u (8
    //      per row), 256..383 rows 0-31 (4 per row: columns 0-31). ----
    // elements between tokens of the staged Q and K tiles (per channel: the
    // workspace's K^ and K+ rows)
    const int tstride = PERCH ? DK : Hk * DK;
    const int tsv = H * DV;                    // ... and of v
    // With the in-chain solve only waves 4 and 5 load: wave 4 all of Q and V
    // row groups 0-1, wave 5 all of K, V row groups 2-3 and g.
    const int wi = FUSED ? wave - SV_LOAD0 : wave - 4;
    constexpr int NQK = FUSED ? 16 : 8;        // Q or K rows (of 4) per loading wave
    const int qkmat = FUSED ? wi : wi >> 1;    // 0 Q, 1 K
    const int qkrow0 = FUSED ? 0 : 32 * (wi & 1);
    const int qkrow = qkrow0 + (lane0 >> 4), qkcol = 8 * (lane0 & 15);
    const int goffQK = 2 * (qkrow * tstride + qkcol);
    const int goffV = 2 * ((lane0 >> 2) * tsv + 8 * (lane0 & 3));
    const int vr0 = FUSED ? 2 * wi : 2 * (wi - 2);   // first V row group
    // LDS element offset of workspace piece e within a staging buffer (uniform
    // per 64-piece group)
    auto tpiece_loff = [&](int e) {
        return e < 256 ? B_TL / 2 + (e >> 3) * LD_L + 8 * (e & 7)
                       : B_TH / 2 + ((e - 256) >> 2) * LD_H + 8 * (e & 3);
    };
    const bf16 *qk_head = (qkmat ? k : q) + (size_t)bos * (Hk * DK) + (size_t)(h / (H / Hk)) * DK;
    const bf16 *v_head = v + (size_t)bos * tsv + (size_t)h * DV + cbase;
    const float *g_head = g + (size_t)bos * H + h;
    // Two register sets: chunk c is loaded into set c % 2 three iterations
    // before its use and stored to LDS one iteration before.
    struct Pref {
        bf16x8 b[NQK], t[3], v[2];
        float g;
        f32x2 ec;                              // per channel: e^{gamma_63}, channels 2 lane ..
    };
    Pref pA, pB;
    // WT: whether this wave loads T_u pieces, WG: whether it loads and scans
    // g, WV: whether it loads V (compile-time flags, so that no loop holds a
    // load it may not need)
    auto fetch = [&](int ch, Pref &rs, auto WT, auto WG, auto WV) {
        const int base = ch * C;
        const int nrow = len - base < C ? len - base : C;      // tokens of the chunk in the sequence
        const unsigned nb = (unsigned)nrow * tstride * 2;
        // per channel the Q tile is K^ and the K tile K+, both from the workspace
        const bf16 *qk_src = PERCH ? wsh + (size_t)ch * IST + (qkmat ? CH_KP : CH_KH)
                                   : qk_head + (size_t)base * tstride;
        const __amdgpu_buffer_rsrc_t rqk = __builtin_amdgcn_make_buffer_rsrc(
            (void *)qk_src, 0, nb, 0x00020000);
#pragma unroll
        for (int r = 0; r < NQK; ++r)
            rs.b[r] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                          rqk, goffQK, r * 4 * tstride * 2, 0));
        if constexpr (decltype(WT)::value) {
            const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(wsh + (size_t)ch * IST), 0, WS_T * 16, 0x00020000);
#pragma unroll
            for (int r = 0; r < 3; ++r)
                rs.t[r] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                              rw, 16 * lane0, 16 * (192 * wi + 64 * r), 0));
        }
        if constexpr (decltype(WV)::value) {
            // with CHAIN_ZERO_V the resource spans nothing and every load reads zero
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(v_head + (size_t)base * tsv), 0,
                (flags & CHAIN_ZERO_V) ? 0u : (unsigned)nrow * tsv * 2, 0x00020000);
#pragma unroll
            for (int r = 0; r < 2; ++r)
                rs.v[r] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                              rv, goffV, (vr0 + r) * 16 * tsv * 2, 0));
        }
        if constexpr (decltype(WG)::value) {
            if constexpr (PERCH) {
                // no per-token gate (the decay is in K+, K^, Q+); the state's
                // per-channel decay of the chunk instead
                rs.g = 0.f;
                rs.ec = *reinterpret_cast<const f32x2 *>(
                    reinterpret_cast<const float *>(wsh + (size_t)ch * IST + CH_EC) + 2 * lane0);
            } else {
                const __amdgpu_buffer_rsrc_t rgs = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(g_head + (size_t)base * H), 0, (unsigned)nrow * H * 4, 0x00020000);
                rs.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rgs, 4 * H * lane0, 0, 0));
            }
        }
    };
    auto store = [&](const Pref &rs, int b, auto WT, auto WG, auto WV, int lane) {
        bf16 *buf = lds + (OFF_BUF + b * SZ_BUF) / 2;
        // row qkrow0 + lane/16 + 4 r: qkrow0 is 0 or 32, so its bit 4 is bit 2 of r
        const int lrow = (qkmat ? B_K : B_Q) / 2 + (qkrow0 + (lane >> 4)) * LD_R, lcol = 8 * (lane & 15);
#pragma unroll
        for (int r = 0; r < NQK; ++r) *reinterpret_cast<bf16x8 *>(buf + lrow + 4 * r * LD_R + (lcol ^ swK(4 * r))) = rs.b[r];
        if constexpr (decltype(WT)::value) {
#pragma unroll
            for (int r = 0; r < 3; ++r)
                *reinterpret_cast<bf16x8 *>(buf + tpiece_loff(192 * wi + 64 * r + lane)) = rs.t[r];
        }
        if constexpr (decltype(WV)::value) {
#pragma unroll
            for (int r = 0; r < 2; ++r)
                *reinterpret_cast<bf16x8 *>(buf + B_V / 2 + ((lane >> 2) + 16 * (vr0 + r)) * LD_H + 8 * (lane & 3)) = rs.v[r];
        }
        if constexpr (decltype(WG)::value) {
            float *sc = stSc(b);
            const float gam = wave_inclusive_scan(rs.g);
            const float glast = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gam), 63));
            sc[C + lane] = __expf(gam);
            sc[2 * C + lane] = __expf(glast - gam);
            if constexpr (PERCH) {
                *reinterpret_cast<f32x2 *>(sc + 3 * C + 2 * lane) = rs.ec;
            } else {
                // gamma log2(e), and F_j = e^{gamma_r - gamma_j} <= 1 with r the
                // last token of j's 16-token tile (the key factor of P's
                // off-diagonal tiles)
                const float gl = gam * 1.4426950408889634f;
                const float glr = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                    4 * (lane | 15), __builtin_bit_cast(int, gl)));
                sc[lane] = gl;
                sc[3 * C + lane] = __builtin_amdgcn_exp2f(glr - gl);
            }
        }
    };
    const std::true_type with_t{}, with_g{}, with_v{}, with_p{};
    const std::false_type no_t{}, no_g{}, no_v{}, no_p{};

    // P^T of the chunk in staging buffer b (scalar gate) for token tiles
    // TA < TB, from the B operands fq of those tiles' Q rows: P^T tile (key
    // tile kt, token tile TX) = K_kt Q_TX^T, masked to keys j <= token i and
    // scaled by e^{gamma_i - gamma_j} <= 1 elementwise (directly on the
    // diagonal tile, as e^{gamma_i - gamma_r} F_j below it, r the last token
    // of key tile kt; both factors <= 1). pb[x][s] is the accumulator pair of
    // key tiles 2 s, 2 s + 1 as bf16: the B operand of Delta^T P^T over keys
    // 32 s + 4 q + 0..3, 32 s + 16 + 4 q + 0..3, the order the recurrence
    // writes Delta^T in. The k-steps run outermost so that the independent
    // accumulator chains interleave.
    auto ptiles = [&](auto TAc, auto TBc, const bf16x8 (&fq)[2][4], int b, int m, int qq,
                      bf16x8 (&pb)[2][2]) {
        constexpr int TA = decltype(TAc)::value, TB = decltype(TBc)::value;
        constexpr int TX[2] = {TA, TB};
        constexpr int NKB[2] = {TA / 2 + 1, TB / 2 + 1};
        const bf16 *sK = stK(b);
        const float *sG = stSc(b), *sF = stSc(b) + 3 * C;
        f32x4 pacc[2][4];
        {
            bf16x8 fk[TB + 1][4];
#pragma unroll
            for (int kt = 0; kt <= TB; ++kt)
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2)
                    fk[kt][s2] = lds8(sK, (16 * kt + m) * LD_R + ((32 * s2 + 8 * qq) ^ swK(16 * kt)));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int kt = 0; kt <= TX[x]; ++kt) pacc[x][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int kt = 0; kt <= TX[x]; ++kt)
                        pacc[x][kt] = mfma16(fk[kt][s2], fq[x][s2], pacc[x][kt]);
        }
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int ti = 16 * TX[x] + m;
            const float gs = sG[ti];
#pragma unroll
            for (int kt = 0; kt <= TX[x]; ++kt) {
                if (kt < TX[x]) {
                    const float ek = __builtin_amdgcn_exp2f(gs - sG[16 * kt + 15]);
                    const f32x4 fj = *reinterpret_cast<const f32x4 *>(sF + 16 * kt + 4 * qq);
#pragma unroll
                    for (int r = 0; r < 4; ++r) pacc[x][kt][r] = pacc[x][kt][r] * (ek * fj[r]);
                } else {
                    const f32x4 gj = *reinterpret_cast<const f32x4 *>(sG + 16 * kt + 4 * qq);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float e = __builtin_amdgcn_exp2f(gs - gj[r]);
                        pacc[x][kt][r] = 4 * qq + r <= m ? pacc[x][kt][r] * e : 0.f;
                    }
                }
            }
#pragma unroll
            for (int s = 0; s < NKB[x]; ++s)
                pb[x][s] = acc_pair_bf16(pacc[x][2 * s],
                                         2 * s + 1 <= TX[x] ? pacc[x][2 * s + 1] : f32x4{0.f, 0.f, 0.f, 0.f});
        }
    };
    // Each wave role runs its own loop, unrolled by two from the odd chunk -3
    // so that every buffer and register-set index is a compile-time constant:
    // in iteration c = ch0 + hf, c % 2 = 1 - hf and (c + 1) % 2 = hf. Every
    // role runs the same iterations (-3 .. nchunks or nchunks + 1) and one
    // barrier per iteration; iterations -3 and -2 only load, -1 also stores
    // chunk 0, and nchunks finishes the last output. The loaders' prefetch is
    // one straight-line site per role (every iteration loads, clamped to the
    // last chunk), so the compiler never waits for it at a join or the loop
    // back-edge.
    if (nchunks == 0) {
        // nothing to do but the state copy below
    } else if (wave < 2) {
        // ============ waves 0-1: the recurrence ============
        // the sequential path: these waves win instruction arbitration on their SIMDs
        __builtin_amdgcn_s_setprio(3);
        const int hv = wave;
        for (int ch0 = -3; ch0 <= nchunks; ch0 += 2)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int ch = ch0 + hf;
            const int b = 1 - hf;              // ch % 2
            const int lane = lane0, m = lane & 15, qq = lane >> 4;
            if (ch >= 0 && ch < nchunks) {
                const bf16 *sK = stK(b), *sV = stV(b), *sTH = stTH(b), *sTL = stTL(b);
                // rows 16 t + m of T_u, columns 32 s + 8 q ..
                auto tfrag = [&](int t, int s2) {
                    return t < 2 ? lds8(sTH, (16 * t + m) * LD_H + 8 * qq)
                                 : lds8(sTL, (16 * (t - 2) + m) * LD_L + 32 * s2 + 8 * qq);
                };
                const float *sEg = stSc(b) + C, *sDend = stSc(b) + 2 * C;
                // Every LDS operand of the chunk is read before it is needed, so
                // that no LDS round trip sits between two dependent products:
                // the gates, K, V and T_u first; K^T once X's products have
                // been issued (into K's registers).
                f32x4 dend[4], eg[2][2];
#pragma unroll
                for (int t = 0; t < 4; ++t) dend[t] = *reinterpret_cast<const f32x4 *>(sDend + 16 * t + 4 * qq);
                // e^gamma of tokens 32 s + 8 q + 0..7 (R's rows)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        eg[s2][u] = *reinterpret_cast<const f32x4 *>(sEg + 32 * s2 + 8 * qq + 4 * u);
                const float eend = sEg[C - 1];
                f32x4 dacc[4], xacc[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) { dacc[t] = f32x4{0.f, 0.f, 0.f, 0.f}; xacc[t] = dacc[t]; }
                bf16x8 fv[2], fu[4][2];
                {
                    // X tile t takes K rows 32 (t/2) + 8 (m/4) + 4 (t%2) + m%4, so that its
                    // accumulator pairs run over tokens 32 s + 8 q + 0..7 contiguously
                    bf16x8 fk[4][4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int row = 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3);
#pragma unroll
                        // (32 s + 8 q) ^ swK(row) as two per-lane bases with
                        // immediate offsets
                        for (int s2 = 0; s2 < 4; ++s2) fk[t][s2] = lds8(sK, row * LD_R + 8 * qq + (s2 < 2 ? swK(row) + 32 * s2 : 32 * s2 - swK(row)));
                    }
                    // V in X's accumulator-pair layout: tokens 32 s + 8 q + 0..7 of
                    // column 16 hv + m
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        const int off = (32 * s2 + 8 * qq + (m >> 2)) * LD_H + 16 * hv + 4 * (m & 3);
                        fv[s2] = cat4(tr4(sV, off), tr4(sV, off + 4 * LD_H));
                    }
#pragma unroll
                    for (int t = 0; t < 4; ++t)
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2)
                            if (s2 <= (t >> 1)) fu[t][s2] = tfrag(t, s2);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
                        for (int t = 0; t < 4; ++t) xacc[t] = mfma16(fk[t][s2], Sb[s2], xacc[t]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                // K^T as the A operand of the state update: tile d, lane m takes d_k
                // column 32 (d/2) + 8 (m/4) + 4 (d%2) + m%4 (the state's row order)
                // and tokens 32 s + 4 q + 0..3, 32 s + 16 + 4 q + 0..3 (Delta~'s row
                // order), transposed on read
                // (the wait retires the reads above, so that Delta's products
                // wait for none of these)
                __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
                bf16x8 fkt[8][2];
#pragma unroll
                for (int d = 0; d < 8; ++d)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        const int c0 = 32 * (d >> 1) + 4 * (d & 1) + 8 * (m & 3);
                        const int r0 = 32 * s2 + 4 * qq + (m >> 2);
                        // per channel the update's keys are K^ (in the Q tile)
                        const bf16 *sKu = PERCH ? stQ(b) : sK;
                        fkt[d][s2] = cat4(tr4(sKu, r0 * LD_R + (c0 ^ swK(r0))), tr4(sKu, (r0 + 16) * LD_R + (c0 ^ swK(r0 + 16))));
                    }
                __builtin_amdgcn_sched_barrier(0);
                // R = V - diag(e^gamma) X (per channel e^gamma = 1: the decay is
                // in K+), then Delta = T_u R
                {
                    bf16x8 rb[2];
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float x = e < 4 ? xacc[2 * s2][e] : xacc[2 * s2 + 1][e - 4];
                            rb[s2][e] = (bf16)((float)fv[s2][e] - eg[s2][e >> 2][e & 3] * x);
                        }
#pragma unroll
                    for (int t = 0; t < 4; ++t)
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2)
                            if (s2 <= (t >> 1)) dacc[t] = mfma16(fu[t][s2], rb[s2], dacc[t]);
                }
                // Delta^T -> LDS (output term); Delta~ as the B operand of the update
                bf16x8 db[2];
                {
                    bf16 *sDt = cpDt(b);
                    const int row = 16 * hv + m;
                    if constexpr (PERCH) {
                        // keys in order: the per-channel P from the workspace is
                        // read with consecutive keys
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            bf16x4 x = {(bf16)dacc[t][0], (bf16)dacc[t][1], (bf16)dacc[t][2], (bf16)dacc[t][3]};
                            *reinterpret_cast<bf16x4 *>(sDt + row * LD_L + ((16 * t + 4 * qq) ^ swD(row))) = x;
                        }
                    } else {
                        // key position 32 s + 8 q + e holds key 32 s + 4 q + e (e < 4)
                        // or 32 s + 16 + 4 q + e - 4: the order of the output waves'
                        // P^T accumulator pairs
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2)
                            *reinterpret_cast<bf16x8 *>(sDt + row * LD_L + ((32 * s2 + 8 * qq) ^ swD(row))) =
                                acc_pair_bf16(dacc[2 * s2], dacc[2 * s2 + 1]);
                    }
                    db[0] = acc_pair_bf16(dacc[0] * dend[0], dacc[1] * dend[1]);
                    db[1] = acc_pair_bf16(dacc[2] * dend[2], dacc[3] * dend[3]);
                }
                // S^T <- e^{gamma_63} S^T + K^T Delta~ (the decay while Delta is formed)
#pragma unroll
                for (int d = 0; d < 8; ++d) Sacc[d] = Sacc[d] * eend;
                if constexpr (PERCH) {
                    // S <- S diag(e^{gamma_63}): row dk(d, q, r) of S^T by its channel's factor
                    const float *ec = stSc(b) + 3 * C;
#pragma unroll
                    for (int d = 0; d < 8; ++d)
                        Sacc[d] = Sacc[d] * *reinterpret_cast<const f32x4 *>(ec + 32 * (d >> 1) + 8 * qq + 4 * (d & 1));
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int d = 0; d < 8; ++d) {
                    Sacc[d] = mfma16(fkt[d][0], db[0], Sacc[d]);
                    Sacc[d] = mfma16(fkt[d][1], db[1], Sacc[d]);
                }
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) Sb[s2] = acc_pair_bf16(Sacc[2 * s2], Sacc[2 * s2 + 1]);
                // the bf16 S copy for the output waves: Sb[s] is d_k 32 s + 8 q .. + 7
                // of row 16 hv + m (the swizzle leaves the 16-byte piece whole)
                bf16 *sSn = cpS(hf);           // (ch + 1) % 2
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2)
                    *reinterpret_cast<bf16x8 *>(sSn + (16 * hv + m) * LD_R + ((32 * s2 + 8 * qq) ^ swS(16 * hv + m))) = Sb[s2];
            }
            lds_barrier();
        }
    } else if (wave < 4) {
        // ============ waves 2-3: the output ============
        // Per 16-token tile two O^T accumulators, over the d_v rows 8 (i/4) +
        // 4 u + i%4 of tile row i (u = 0, 1): a lane's accumulators then hold
        // d_v 8 q .. 8 q + 7 of one token, stored as 16 contiguous bytes (64 per
        // token row and instruction), and the wave reads Q only for its own
        // tokens.
        auto store_rows = [&](const f32x4 (&acc)[2], int cp, int tt, int m, int qq, float sc) {
            const int tok = cp * C + 16 * tt + m;
            if (tok < len) {
                const f32x4 a = acc[0], c = acc[1];
                const bf16x8 x = {(bf16)(sc * a[0]), (bf16)(sc * a[1]), (bf16)(sc * a[2]), (bf16)(sc * a[3]),
                                  (bf16)(sc * c[0]), (bf16)(sc * c[1]), (bf16)(sc * c[2]), (bf16)(sc * c[3])};
                *reinterpret_cast<bf16x8 *>(out + ((size_t)bos + tok) * H * DV + (size_t)h * DV + cbase + 8 * qq) = x;
            }
        };
        // scalar gate: token tiles TA < TB = 3 - TA of every chunk. P^T comes
        // from staging wave 6 + TA through P copy (ch - 1) % 2 when the chunk
        // is finished; with the in-chain solve this wave forms it (ptiles,
        // its Q operand the one S Q^T reads) and holds it for one iteration.
        auto oloop_scalar = [&](auto TAc, auto TBc) {
            constexpr int TA = decltype(TAc)::value, TB = decltype(TBc)::value;
            constexpr int TX[2] = {TA, TB};
            constexpr int NKB[2] = {TA / 2 + 1, TB / 2 + 1};    // 32-key blocks per tile
            f32x4 oacc[2][2][2];               // [chunk parity][tile][u]
            bf16x8 pb[2][2][2];                // [chunk parity][tile][key block]
            for (int ch0 = -3; ch0 <= nchunks; ch0 += 2)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int ch = ch0 + hf;
                const int b = 1 - hf;          // ch % 2; (ch + 1) % 2 = (ch - 1) % 2 = hf
                int tidl = tid0;
                asm volatile("" : "+v"(tidl));
                const int lane = tidl & 63, m = lane & 15, qq = lane >> 4;
                const int r0 = 8 * (m >> 2) + (m & 3);     // d_v row of tile row m, u = 0
                if (out && ch >= 0 && ch < nchunks) {   // o == NULL: the states only
                    const bf16 *sSc = cpS(b), *sQ = stQ(b);
                    const float *sEg = stSc(b) + C;
                    bf16x8 fs[2][4], fq[2][4];
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
                        for (int u = 0; u < 2; ++u)
                            fs[u][s2] = lds8(sSc, (r0 + 4 * u) * LD_R + ((32 * s2 + 8 * qq) ^ swS(r0 + 4 * u)));
#pragma unroll
                        for (int x = 0; x < 2; ++x)
                            fq[x][s2] = lds8(sQ, (16 * TX[x] + m) * LD_R + ((32 * s2 + 8 * qq) ^ swK(16 * TX[x])));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    // (Q S^T)^T = S Q^T for the wave's tokens (the k-steps outermost, so
                    // that the four accumulator chains interleave), then scale e^gamma
                    // per token
#pragma unroll
                    for (int x = 0; x < 2; ++x)
#pragma unroll
                        for (int u = 0; u < 2; ++u) oacc[b][x][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
                        for (int x = 0; x < 2; ++x)
#pragma unroll
                            for (int u = 0; u < 2; ++u)
                                oacc[b][x][u] = mfma16(fs[u][s2], fq[x][s2], oacc[b][x][u]);
                    if constexpr (!PST) ptiles(TAc, TBc, fq, b, m, qq, pb[b]);
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        const float e_i = sEg[16 * TX[x] + m];
#pragma unroll
                        for (int u = 0; u < 2; ++u) oacc[b][x][u] = oacc[b][x][u] * e_i;
                    }
                }
                if (out && ch >= 1 && ch <= nchunks) {
                    // finish chunk ch - 1: O^T += Delta^T P^T, then its rows to HBM
                    const int cp = ch - 1;
                    const bf16 *sDt = cpDt(hf);
                    bf16x8 fd[2][2];
#pragma unroll
                    for (int s = 0; s < NKB[1]; ++s)
#pragma unroll
                        for (int u = 0; u < 2; ++u)
                            fd[u][s] = lds8(sDt, (r0 + 4 * u) * LD_L + ((32 * s + 8 * qq) ^ swD(r0 + 4 * u)));
                    if constexpr (PST) {
#pragma unroll
                        for (int x = 0; x < 2; ++x)
#pragma unroll
                            for (int s = 0; s < NKB[x]; ++s) pb[hf][x][s] = lds8(cpPB(hf, TA, x, s), 8 * lane);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
#pragma unroll
                        for (int s = 0; s < NKB[x]; ++s)
#pragma unroll
                            for (int u = 0; u < 2; ++u)
                                oacc[hf][x][u] = mfma16(fd[u][s], pb[hf][x][s], oacc[hf][x][u]);
                        // oacc[x][u][r] = O[token 16 TX + m][d_v 8 qq + 4 u + r]
                        store_rows(oacc[hf][x], cp, TX[x], m, qq, scale);
                    }
                }
                lds_barrier();
            }
        };
        // per-channel decay: tokens 32 hw .. 32 hw + 31, P from the workspace
        // (staged into the P copies by waves 4-5), Q+ from the workspace in
        // operand order: chunk c into register set c % 2, two iterations ahead,
        // by one load site per iteration that runs unconditionally (clamped to
        // the last chunk; with no outputs its resource spans nothing), like the
        // staging waves' prefetch: a load site under a condition let the
        // compiler wait at the join for the loads just issued
        auto oloop_channel = [&](auto HW) {
            constexpr int hw = decltype(HW)::value;
            constexpr int NS = hw + 1;         // key blocks of 32 that tokens 32 hw .. need
            f32x4 oacc[2][2][2];               // [chunk parity][token tile 2 hw + tt][u]
            bf16x8 fqg[2][2][4];
            auto qfetch = [&](int c, bf16x8 (&dst)[2][4], int lane) {
                const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(wsh + (size_t)c * IST + CH_QP), 0, out ? (unsigned)(C * DK * 2) : 0u,
                    0x00020000);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2)
                        dst[tt][s2] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                            rq, 16 * lane, 1024 * (4 * (2 * hw + tt) + s2), 0));
            };
            for (int ch0 = -3; ch0 <= nchunks; ch0 += 2)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int ch = ch0 + hf;
                const int b = 1 - hf;
                int tidl = tid0;
                asm volatile("" : "+v"(tidl));
                const int lane = tidl & 63, m = lane & 15, qq = lane >> 4;
                const int r0 = 8 * (m >> 2) + (m & 3);
                if (out && ch >= 0 && ch < nchunks) {
                    const bf16 *sSc = cpS(b);
                    bf16x8 fs[2][4];
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
                        for (int u = 0; u < 2; ++u)
                            fs[u][s2] = lds8(sSc, (r0 + 4 * u) * LD_R + ((32 * s2 + 8 * qq) ^ swS(r0 + 4 * u)));
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int s2 = 0; s2 < 4; ++s2) a = mfma16(fs[u][s2], fqg[b][tt][s2], a);
                            oacc[b][tt][u] = a;
                        }
                }
                // chunk ch + 2 into the set chunk ch has just been read from
                qfetch(ch + 2 < 0 ? 0 : ch + 2 < nchunks ? ch + 2 : nchunks - 1, fqg[b], lane);
                if (out && ch >= 1 && ch <= nchunks) {
                    const int cp = ch - 1;
                    const bf16 *sDt = cpDt(hf), *sP = cpP(hf);
                    bf16x8 fd[2][NS], fp[2][NS];
#pragma unroll
                    for (int s2 = 0; s2 < NS; ++s2) {
#pragma unroll
                        for (int u = 0; u < 2; ++u)
                            fd[u][s2] = lds8(sDt, (r0 + 4 * u) * LD_L + ((32 * s2 + 8 * qq) ^ swD(r0 + 4 * u)));
#pragma unroll
                        for (int tt = 0; tt < 2; ++tt) {
                            const int t = 2 * hw + tt;
                            fp[tt][s2] = t < 2 ? lds8(sP, (16 * t + m) * LD_H + ((8 * qq) ^ swz(lane)))
                                               : lds8(sP + SZ_PH / 2, (16 * (t - 2) + m) * LD_L + ((32 * s2 + 8 * qq) ^ swz(lane)));
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                        for (int s2 = 0; s2 < NS; ++s2)
#pragma unroll
                            for (int u = 0; u < 2; ++u)
                                oacc[hf][tt][u] = mfma16(fd[u][s2], fp[tt][s2], oacc[hf][tt][u]);
                        store_rows(oacc[hf][tt], cp, 2 * hw + tt, m, qq, scale);
                    }
                }
                lds_barrier();
            }
        };
        if constexpr (PERCH) {
            if (wave == 2) oloop_channel(std::integral_constant<int, 0>{});
            else oloop_channel(std::integral_constant<int, 1>{});
        } else {
            if (wave == 2) oloop_scalar(std::integral_constant<int, 0>{}, std::integral_constant<int, 3>{});
            else oloop_scalar(std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{});
        }
    } else {
        // ============ waves 4-7: staging; waves 4-5 also stage P (per channel),
        //              waves 6-7 form P^T (scalar gate) ============
        // below the recurrence and above the output waves in issue arbitration:
        // the next chunk's tiles must be in LDS by the barrier (per channel the
        // output waves also load Q+ from memory and keep the default)
        if constexpr (!PERCH) __builtin_amdgcn_s_setprio(1);
        // P pieces 192 (wave - 4) + 64 r + lane (r < 3) of the workspace item,
        // held in one of two register sets by chunk parity: chunk c's pieces
        // are loaded in iteration c - 2 and written into P copy c % 2 in
        // iteration c (the output waves read that copy in iteration c + 1).
        // P copy layout: rows 0-31 (columns 0-31) at row stride LD_H, rows
        // 32-63 at LD_L, 16-byte column groups swapped as for the other
        // accumulator-order tiles.
        const int pe0 = 192 * (wave - 4);
        auto pfetch = [&](int ch, bf16x8 (&pr)[3]) {
            const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(wsh + (size_t)ch * IST + CH_P), 0, WS_P * 16, 0x00020000);
#pragma unroll
            for (int r = 0; r < 3; ++r)
                pr[r] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                            rp, 16 * (pe0 + lane0), 1024 * r, 0));
        };
        auto pstore = [&](const bf16x8 (&pr)[3], bf16 *sP, int lane) {
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                const int e = pe0 + 64 * r + lane;
                const int row = e < 128 ? e >> 2 : (e - 128) >> 3;
                const int grp = e < 128 ? e & 3 : (e - 128) & 7;
                const int off = e < 128 ? row * LD_H : SZ_PH / 2 + row * LD_L;
                *reinterpret_cast<bf16x8 *>(sP + off + 8 * (grp ^ ((row & 15) >> 2))) = pr[r];
            }
        };
        // WPT: the token tiles {R, 3 - R} whose P^T this wave forms (scalar
        // gate, two-pass layout: waves 6 and 7 for output waves 2 and 3), or
        // R < 0 for none. It runs after the wave's stores and loads, which
        // the next iteration waits for: formed before them it made the step
        // ~10% slower.
        auto lloop = [&](auto WT, auto WG, auto WV, auto WP, auto WPT) {
            constexpr int R = decltype(WPT)::value;
            auto pstage = [&](int b, int lane) {
                if constexpr (R >= 0) {
                    const int m = lane & 15, qq = lane >> 4;
                    constexpr int TX[2] = {R, 3 - R};
                    constexpr int NKB[2] = {R / 2 + 1, (3 - R) / 2 + 1};
                    const bf16 *sQ = stQ(b);
                    bf16x8 fq[2][4], pbv[2][2];
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
                        for (int x = 0; x < 2; ++x)
                            fq[x][s2] = lds8(sQ, (16 * TX[x] + m) * LD_R + ((32 * s2 + 8 * qq) ^ swK(16 * TX[x])));
                    ptiles(std::integral_constant<int, R>{}, std::integral_constant<int, 3 - R>{}, fq, b, m, qq, pbv);
#pragma unroll
                    for (int x = 0; x < 2; ++x)
#pragma unroll
                        for (int s = 0; s < NKB[x]; ++s)
                            *reinterpret_cast<bf16x8 *>(cpPB(b, R, x, s) + 8 * lane) = pbv[x][s];
                }
            };
            bf16x8 pp[2][3];
            for (int ch0 = -3; ch0 <= nchunks; ch0 += 2)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int ch = ch0 + hf;
                const int b = 1 - hf;          // ch % 2
                Pref &ps = hf ? pB : pA;
                int tidl = tid0;
                asm volatile("" : "+v"(tidl));
                const int lane = tidl & 63;
                if constexpr (decltype(WP)::value) {
                    if (ch >= 0 && ch < nchunks) pstore(pp[b], cpP(b), lane);
                    const int cf = ch + 2 < 0 ? 0 : ch + 2 < nchunks ? ch + 2 : nchunks - 1;
                    pfetch(cf, pp[b]);
                }
                if (ch + 1 >= 0 && ch + 1 < nchunks) store(ps, hf, WT, WG, WV, lane);   // chunk ch + 1
                fetch(ch + 3 < nchunks ? ch + 3 : nchunks - 1, ps, WT, WG, WV);
                if (out && ch >= 0 && ch < nchunks) pstage(b, lane);
                lds_barrier();
            }
        };
        // ---- in-chain solve: waves 6 and 7 form T_u = (I - A)^-1 diag(beta)
        //      of chunk c (wave 6 + c % 2) into staging buffer c % 2 over two
        //      iterations, each phase bounded by the iteration's barrier:
        //        iteration c - 3  load K (operand order), g, beta of chunk c
        //        iteration c - 2  gamma; Gram tiles K K^T (bf16 MFMA); A =
        //                         -strict_lower(diag(beta) K K^T * Gamma);
        //                         diagonal blocks D_b = (I - A_bb)^-1 by
        //                         forward substitution
        //        iteration c - 1  off-diagonal blocks of T by two levels of
        //                         2 x 2 block inversion (fp32 MFMA), T diag(beta)
        //                         as bf16 pieces into the staging buffer (which
        //                         the loaders fill with chunk c's tiles in the
        //                         same iteration)
        //      ("5. Linear Attention", chunked delta rule, stage 1; the same
        //      arithmetic as the prep pass, by one wave per chunk) ----
        auto sloop = [&](auto SID) {
            constexpr int sid = decltype(SID)::value;      // chunks c with c % 2 == sid
            __builtin_amdgcn_s_setprio(SV_PRIO);
            const WaveSolver sol{reinterpret_cast<float *>(smem + L::SV + sid * SV_BYTES)};
            const bf16 *k_head = k + (size_t)bos * (Hk * DK) + (size_t)(h / (H / Hk)) * DK;
            const float *b_head = beta + (size_t)bos * H + h;
            bf16x8 kr[4][4];
            float gv = 0.f, bv = 0.f;
            for (int ch0 = -3; ch0 <= nchunks; ch0 += 2)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int ch = ch0 + hf;
                int tidl = tid0;
                asm volatile("" : "+v"(tidl));
                const int lane = tidl & 63;
                if (hf == sid) {
                    // (ch + 1) % 2 == sid: finish chunk ch + 1 into staging hf,
                    // then load chunk ch + 3
                    if (ch + 1 >= 0 && ch + 1 < nchunks) {
                        sol.phase2(lane);
                        bf16 *sb = lds + (OFF_BUF + hf * SZ_BUF) / 2;
                        sol.emit(lane, [&](int e, bf16x8 p) {
                            *reinterpret_cast<bf16x8 *>(sb + tpiece_loff(e)) = p;
                        });
                    }
                    const int cf = ch + 3 < 0 ? 0 : ch + 3 < nchunks ? ch + 3 : nchunks - 1;
                    const int nrow = len - cf * C < C ? len - cf * C : C;
                    WaveSolver::fetch(k_head + (size_t)cf * C * tstride, tstride,
                                      g_head + (size_t)cf * C * H, b_head + (size_t)cf * C * H, H,
                                      nrow, lane, kr, gv, bv);
                } else if (ch + 2 >= 0 && ch + 2 < nchunks) {
                    sol.phase1(kr, gv, bv, lane);  // chunk ch + 2
                }
                lds_barrier();
            }
        };
        if constexpr (FUSED) {
            if (wave == SV_LOAD0 + 1) lloop(no_t, with_g, with_v, no_p, std::integral_constant<int, -1>{});
            else if (wave == SV_LOAD0) lloop(no_t, no_g, with_v, no_p, std::integral_constant<int, -1>{});
            else if (wave == SV_WAVE0) sloop(std::integral_constant<int, 0>{});
            else sloop(std::integral_constant<int, 1>{});
        } else {
            // wave 6 forms P^T for output wave 2 (token tiles 0, 3), wave 7
            // for output wave 3 (tiles 1, 2)
            using PT0 = std::integral_constant<int, PST ? 0 : -1>;
            using PT1 = std::integral_constant<int, PST ? 1 : -1>;
            using PTN = std::integral_constant<int, -1>;
            if (wave == 7) lloop(no_t, with_g, with_v, no_p, PT1{});
            else if (wave == 6) lloop(no_t, no_g, with_v, no_p, PT0{});
            else if constexpr (PERCH) lloop(with_t, no_g, no_v, with_p, PTN{});
            else lloop(with_t, no_g, no_v, no_p, PTN{});
        }
    }
    if (sfin && wave < 2) {
        const int m = lane0 & 15, qq = lane0 >> 4;
        float *dst = sfin + (size_t)(cbase + 16 * wave + m) * DK + 8 * qq;
#pragma unroll
        for (int d = 0; d < 8; ++d) *reinterpret_cast<f32x4 *>(dst + 32 * (d >> 1) + 4 * (d & 1)) = Sacc[d];
    }
}

// Workspace bytes of the two-pass path for `tokens` packed tokens in N
// sequences of H heads (per_channel: the larger per-channel item).
size_t prefill_split_workspace_bytes(long tokens, int H, int N, bool per_channel) {
    const long nslots = tokens / C + N + 1;
    return (size_t)nslots * H * (per_channel ? CH_ITEM_ELEMS : ITEM_ELEMS) * sizeof(bf16);
}

// Raise a kernel's dynamic LDS limit on the current device, once per device
// (the attribute belongs to the device's copy of the kernel; concurrent first
// calls set the same value).
static hipError_t raise_lds_limit(const void *kern, int bytes, std::atomic<int> *done)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < MAX_DEVICES && done[dev].load(std::memory_order_relaxed)) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && dev < MAX_DEVICES) done[dev].store(1, std::memory_order_relaxed);
    return e;
}

// Workgroups that fill every CU of the current device at the occupancy a
// persistent prep kernel reaches (cached per device; concurrent first calls
// compute the same value).
static hipError_t prep_fill(const void *kern, int nt, int lds, std::atomic<long> *cache, long &fill)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    fill = dev < MAX_DEVICES ? cache[dev].load(std::memory_order_relaxed) : 0;
    if (fill == 0) {
        int cus = 0, per_cu = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, nt, lds);
        if (e != hipSuccess) return e;
        fill = (long)(per_cu < 1 ? 1 : per_cu) * (cus < 1 ? 1 : cus);
        if (fill >= 8) fill = fill / 8 * 8;      // whole rounds of the 8 XCDs (prep_nitems)
        if (dev < MAX_DEVICES) cache[dev].store(fill, std::memory_order_relaxed);
    }
    return hipSuccess;
}

hipError_t launch_prefill_prepare(const void *q, const void *k, const float *g, const float *beta,
                                  const int32_t *cu, int T, int H, int Hk, int N, void *ws,
                                  hipStream_t stream, bool per_channel)
{
    const long tokens = cu ? (long)T : (long)N * T;
    const long nslots = tokens / C + N + 1;
    if (tokens == 0) return hipSuccess;        // no chunk: nothing to prepare
    const long nitems = prep_nitems(nslots, H);
    static std::atomic<long> fill_scalar[MAX_DEVICES], fill_prefetch[MAX_DEVICES];
    static std::atomic<long> fill_channel[MAX_DEVICES];
    static std::atomic<int> lds_scalar[MAX_DEVICES], lds_prefetch[MAX_DEVICES];
    static std::atomic<int> lds_channel[MAX_DEVICES];
    long fill = 0;
    if (per_channel) {
        const hipError_t attr = raise_lds_limit((const void *)chunk_prep_channel_kernel,
                                                CP_LDS_BYTES, lds_channel);
        if (attr != hipSuccess) return attr;
        hipError_t e = prep_fill((const void *)chunk_prep_channel_kernel, P_NT, CP_LDS_BYTES,
                                 fill_channel, fill);
        if (e != hipSuccess) return e;
        dim3 grid((unsigned)(nitems < fill ? nitems : fill)), block(P_NT);
        hipLaunchKernelGGL(chunk_prep_channel_kernel, grid, block, CP_LDS_BYTES, stream,
                           (const bf16 *)q, (const bf16 *)k, g, beta, cu, (bf16 *)ws, T, H, Hk, N,
                           (int)nslots);
        return hipGetLastError();
    }
    // more items than the plain kernel's grid has waves: the kernel that
    // fetches each item's keys during the previous item's solve (its second
    // items' keys then arrive while the first ones are solved, where the plain
    // kernel's second round waits for them; with the keys coming from HBM, as
    // after the chain pass of the previous call, that is 1.7 us of the 4096
    // items of B=4 T=4096 H=16)
    const void *plain = (const void *)chunk_solve_kernel<false>;
    const void *pref = (const void *)chunk_solve_kernel<true>;
    hipError_t e = raise_lds_limit(plain, SV_BYTES, lds_scalar);
    if (e == hipSuccess) e = raise_lds_limit(pref, SV_BYTES, lds_prefetch);
    if (e != hipSuccess) return e;
    e = prep_fill(plain, SOLVE_NT, SV_BYTES, fill_scalar, fill);
    if (e != hipSuccess) return e;
    const bool prefetch = nitems > fill;
    if (prefetch) {
        e = prep_fill(pref, SOLVE_NT, SV_BYTES, fill_prefetch, fill);
        if (e != hipSuccess) return e;
    }
    dim3 grid((unsigned)(nitems < fill ? nitems : fill)), block(SOLVE_NT);
    if (prefetch)
        hipLaunchKernelGGL(chunk_solve_kernel<true>, grid, block, SV_BYTES, stream,
                           (const bf16 *)k, g, beta, cu, (bf16 *)ws, T, H, Hk, N, (int)nslots);
    else
        hipLaunchKernelGGL(chunk_solve_kernel<false>, grid, block, SV_BYTES, stream,
                           (const bf16 *)k, g, beta, cu, (bf16 *)ws, T, H, Hk, N, (int)nslots);
    return hipGetLastError();
}

// jobs: NULL, or a device table of njobs entries (one per pair / H) that
// replaces the one pair per (sequence, head); N is then the number of
// segments in cu.
template <bool PERCH, bool FUSED = false>
static hipError_t launch_chain(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *s_init, float *s_final, void *o,
                               const int32_t *cu, int T, int H, int Hk, int N, float scale,
                               const void *ws, hipStream_t stream, int flags, const SegJob *jobs,
                               int njobs)
{
    constexpr int LDS_BYTES = ChainLds<PERCH, FUSED>::BYTES;
    // the dynamic LDS limit, raised once per device (one flag set per instantiation)
    static std::atomic<int> lds_done[MAX_DEVICES];
    const hipError_t attr = raise_lds_limit((const void *)chunk_chain_kernel<PERCH, FUSED>,
                                            LDS_BYTES, lds_done);
    if (attr != hipSuccess) return attr;
    const long tokens = cu ? (long)T : (long)N * T;
    const long nslots = tokens / C + N + 1;
    const int npairs = H * (jobs ? njobs : N);
    if (npairs == 0) return hipSuccess;
    dim3 grid(pair_grid(npairs)), block(NT);
    auto *kern = chunk_chain_kernel<PERCH, FUSED>;
    hipLaunchKernelGGL(kern, grid, block, LDS_BYTES, stream,
                       (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, g, beta,
                       (const bf16 *)ws, s_init, s_final, (bf16 *)o, cu, jobs, T, H, Hk, npairs,
                       (int)nslots, scale, flags);
    return hipGetLastError();
}

hipError_t launch_prefill_apply(const void *q, const void *k, const void *v, const float *g,
                                const float *s_init, float *s_final, void *o, const int32_t *cu,
                                int T, int H, int Hk, int N, float scale, const void *ws,
                                hipStream_t stream, int flags, bool per_channel,
                                const SegJob *jobs, int njobs)
{
    return per_channel ? launch_chain<true>(q, k, v, g, nullptr, s_init, s_final, o, cu, T, H, Hk,
                                            N, scale, ws, stream, flags, jobs, njobs)
                       : launch_chain<false>(q, k, v, g, nullptr, s_init, s_final, o, cu, T, H, Hk,
                                             N, scale, ws, stream, flags, jobs, njobs);
}

hipError_t launch_prefill_fused(const void *q, const void *k, const void *v, const float *g,
                                const float *beta, const float *s_init, float *s_final, void *o,
                                const int32_t *cu, int T, int H, int Hk, int N, float scale,
                                hipStream_t stream, int flags, const SegJob *jobs, int njobs)
{
    return launch_chain<false, true>(q, k, v, g, beta, s_init, s_final, o, cu, T, H, Hk, N, scale,
                                     nullptr, stream, flags, jobs, njobs);
}

}  // namespace gdn
