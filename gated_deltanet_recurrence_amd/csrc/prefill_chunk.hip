// prefill_chunk.hip - chunkwise-parallel gated delta rule forward on bf16
// matrix cores (MFMA), d_k = d_v = 128, chunks of 64 tokens, fp32 state.
//
// Algorithm: "5. Linear Attention" (LinkQwen ch. 5), section "Chunk
// implementation of the Delta Rule", stages 1-3, and "[LLM Algorithms-2]
// Gated DeltaNet: Teaching Linear Attention to Overwrite and Forget",
// section 7 (a chunk of tokens composes into one state update). With the
// state stored S[d_v][d_k] and, per chunk of C = 64 tokens,
//   gamma_i  = sum_{s<=i} g_s                       (log decay up to token i)
//   Gamma_ij = exp(gamma_i - gamma_j), j <= i        (always <= 1: never overflows)
//   A        = -strict_lower(diag(beta) K K^T * Gamma)
//   T        = (I - A)^-1                            (unit lower triangular)
//   W        = T diag(beta e^gamma) K,   U = T diag(beta) V
//   Delta    = U - W S^T                             (per chunk, needs the state)
//   O        = scale (diag(e^gamma) Q S^T + lower_incl_diag(Q K^T * Gamma) Delta)
//   S       <- e^{gamma_63} S + Delta~^T K,  Delta~_j = e^{gamma_63 - gamma_j} Delta_j
// the chunk reproduces the token-by-token recurrence exactly (A is
// nilpotent, so the inverse is a finite series).
//
// Work mapping: one workgroup of 8 waves (two per SIMD) per (32-wide d_v
// tile, head, sequence); the columns of S (rows of our d_v x d_k state) evolve
// independently, so the four d_v tiles of a head never communicate. The
// state tile (32 x 128 fp32) stays in MFMA accumulator registers for the
// whole sequence; a bf16 copy in LDS is the operand of the next chunk.
// The next chunk's q, k, v are loaded into registers while the current one
// is computed. Inside a chunk:
//   load   Q, K row-major and K^T, V^T (token-contiguous) into LDS
//   gamma  inclusive prefix sum of g over the chunk (wave 0, DPP row shifts and
//          row broadcasts)
//   gram   K K^T lower tiles on MFMA, masked -> A (fp32)
//   solve  T = (I - A)^-1 in fp32. Waves 0-3 invert the four 16 x 16 diagonal
//          blocks by forward substitution while waves 4-7 form
//          P = lower(Q K^T * Gamma) on MFMA; the off-diagonal blocks follow
//          from two levels of 2 x 2 block inversion, (L^-1)_21 =
//          L22^-1 A21 L11^-1, as 16 x 16 fp32 MFMA products. Every finished
//          block is also written as bf16 T diag(beta e^gamma) and T diag(beta).
//   W, U   bf16 MFMA
//   chain  Delta = U - W S^T, O = e^gamma Q S^T + P Delta, S update (MFMA)
// Tokens past the end of a sequence are identity steps (q = k = v = 0,
// beta = 0, g = 0) and their outputs are not stored.
//
// Launch: a 1-D grid ordered so that the four d_v tiles of one (sequence,
// head) run on the same XCD (workgroups are dealt to the 8 XCDs round-robin),
// where the XCD's L2 serves their shared q/k reads and merges their partial
// output rows.
//
// Barriers wait for LDS traffic only (lgkmcnt), never for the global loads of
// the next chunk that are in flight.
//
// MFMA used: v_mfma_f32_16x16x32_bf16 and, for the solve, v_mfma_f32_16x16x4f32. Lane l holds A[l%16][8(l/16)+e] and
// B[8(l/16)+e][l%16] (e = 0..7), and accumulator element r is
// C[4(l/16)+r][l%16]; so both operands are read as 16-byte rows of a
// k-contiguous LDS matrix.
#include "common.h"

namespace gdn {

namespace chunk {

constexpr int C = 64;          // tokens per chunk
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int DVT = 32;        // d_v columns per workgroup
constexpr int NW = 8;          // waves per workgroup
constexpr int NT = 64 * NW;    // threads per workgroup

// LDS leading dimensions (elements); +8 bf16 / +4 fp32 of padding per row
constexpr int LD_QK = DK + 8;  // sQ, sK, sWn rows (bf16)
constexpr int LD_T = C + 8;    // token-contiguous bf16 rows: sKt, sVt, sP, sTw, sTu, sDt, sDtw
constexpr int LD_S = DK + 8;   // sS rows (bf16)
constexpr int LD_A = C + 4;    // fp32 rows: sA, sT
constexpr int LD_Y = 16 + 4;   // fp32 16x16 scratch blocks
constexpr int LD_O = DVT + 8;  // output staging (bf16)

// LDS regions (bytes)
constexpr int SZ_Q = C * LD_QK * 2;       // 17408
constexpr int SZ_KT = DK * LD_T * 2;      // 18432
constexpr int SZ_VT = DVT * LD_T * 2;     // 4608
constexpr int SZ_A = C * LD_A * 4;        // 17408 (also holds -W as bf16 [64][LD_QK])
constexpr int SZ_T = C * LD_A * 4;        // 17408
constexpr int SZ_Y = 2 * C * LD_T * 2;    // 18432: solve scratch, then sDt|sDtw|sO
constexpr int SZ_TWU = 2 * C * LD_T * 2;  // 18432: sTw | sTu (bf16)
constexpr int SZ_P = C * LD_T * 2;        // 9216
constexpr int SZ_S = DVT * LD_S * 2;      // 8704
constexpr int SZ_SC = 8 * C * 4;          // 2048: per-token scalars

constexpr int OFF_Q = 0;
constexpr int OFF_K = OFF_Q + SZ_Q;
constexpr int OFF_KT = OFF_K + SZ_Q;
constexpr int OFF_VT = OFF_KT + SZ_KT;
constexpr int OFF_A = OFF_VT + SZ_VT;
constexpr int OFF_T = OFF_A + SZ_A;
constexpr int OFF_Y = OFF_T + SZ_T;
constexpr int OFF_TWU = OFF_Y + SZ_Y;
constexpr int OFF_P = OFF_TWU + SZ_TWU;
constexpr int OFF_S = OFF_P + SZ_P;
constexpr int OFF_SC = OFF_S + SZ_S;
constexpr int LDS_BYTES = OFF_SC + SZ_SC;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
static_assert(C * LD_QK * 2 <= SZ_A, "-W fits in the A region");
static_assert(9 * 16 * LD_Y * 4 <= SZ_Y, "solve scratch fits");
static_assert(2 * DVT * LD_T * 2 + C * LD_O * 2 <= SZ_Y, "chain buffers fit");

// per-token scalar slots in the SC region
enum { SC_GAM = 0, SC_BETA, SC_BEG, SC_EG, SC_DEND };

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16 x 8 operand slice: row r0 + lane%16, columns k0 + 8*(lane/16) .. +8
__device__ __forceinline__ bf16x8 frag(const bf16 *m, int ld, int r0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8 *>(m + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}

// acc += A[i0.., 0..32*KS) B[0..32*KS, j0..]; A row-major (ld_a), B given as
// Bt[j][k] (ld_b). All operand fragments are read before the first MFMA.
template <int KS>
__device__ __forceinline__ f32x4 mma(f32x4 acc, const bf16 *a, int ld_a, int i0, const bf16 *bt,
                                     int ld_b, int j0, int lane) {
    bf16x8 fa[KS], fb[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        fa[s] = frag(a, ld_a, i0, 32 * s, lane);
        fb[s] = frag(bt, ld_b, j0, 32 * s, lane);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = mfma16(fa[s], fb[s], acc);
    return acc;
}
// products with a lower-triangular 64 x 64 left factor, row tile ti: the
// k range is [0, 32) for ti < 2 and [0, 64) otherwise
__device__ __forceinline__ f32x4 mma_tri(f32x4 acc, int ti, const bf16 *a, int ld_a,
                                         const bf16 *bt, int ld_b, int j0, int lane) {
    return ti < 2 ? mma<1>(acc, a, ld_a, 16 * ti, bt, ld_b, j0, lane)
                  : mma<2>(acc, a, ld_a, 16 * ti, bt, ld_b, j0, lane);
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
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[s], yb[s], acc, 0, 0, 0);
    return acc;
}
// 16 x 16 fp32 block <-> accumulator layout (element r of lane l is row
// 4(l/16) + r, column l%16)
__device__ __forceinline__ void st16(float *Z, int ldz, f32x4 acc, int lane) {
#pragma unroll
    for (int r = 0; r < 4; ++r) Z[(4 * (lane >> 4) + r) * ldz + (lane & 15)] = acc[r];
}
__device__ __forceinline__ f32x4 ld16(const float *Z, int ldz, int lane) {
    f32x4 a;
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = Z[(4 * (lane >> 4) + r) * ldz + (lane & 15)];
    return a;
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

// lower 16x16 tiles (ti, tj), tj <= ti, enumerated 0..9
constexpr int TI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
constexpr int TJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

}  // namespace chunk

using namespace chunk;

__global__ void __launch_bounds__(NT, 1)
prefill_chunk_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                     const bf16 *__restrict__ v, const float *__restrict__ g,
                     const float *__restrict__ beta, const float *s_init, float *s_final,
                     bf16 *__restrict__ o, const int32_t *__restrict__ cu_seqlens, int T, int H,
                     float scale)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    bf16 *sQ = reinterpret_cast<bf16 *>(smem + OFF_Q);
    bf16 *sK = reinterpret_cast<bf16 *>(smem + OFF_K);
    bf16 *sKt = reinterpret_cast<bf16 *>(smem + OFF_KT);
    bf16 *sVt = reinterpret_cast<bf16 *>(smem + OFF_VT);
    float *sA = reinterpret_cast<float *>(smem + OFF_A);
    bf16 *sWn = reinterpret_cast<bf16 *>(smem + OFF_A);        // -W, after the solve
    float *sT = reinterpret_cast<float *>(smem + OFF_T);
    float *sY = reinterpret_cast<float *>(smem + OFF_Y);       // solve scratch
    bf16 *sTw = reinterpret_cast<bf16 *>(smem + OFF_TWU);      // T diag(beta e^gamma)
    bf16 *sTu = sTw + C * LD_T;                                // T diag(beta)
    bf16 *sDt = reinterpret_cast<bf16 *>(smem + OFF_Y);        // chain phase
    bf16 *sDtw = sDt + DVT * LD_T;
    bf16 *sO = sDtw + DVT * LD_T;
    bf16 *sP = reinterpret_cast<bf16 *>(smem + OFF_P);
    bf16 *sS = reinterpret_cast<bf16 *>(smem + OFF_S);
    float *sSc = reinterpret_cast<float *>(smem + OFF_SC);
    const float *sGam = sSc + SC_GAM * C;
    const float *sBeta = sSc + SC_BETA * C;
    const float *sBeg = sSc + SC_BEG * C;
    const float *sEg = sSc + SC_EG * C;
    const float *sDend = sSc + SC_DEND * C;

    const int tid0 = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);   // uniform: scalar branches
    // work item of this workgroup: (sequence n, head h, d_v tile). Workgroup w
    // runs on XCD w % 8; give each XCD a contiguous range of work items so the
    // four tiles of a head share an L2.
    int work = (int)blockIdx.x;
    const int total = (int)gridDim.x;
    if (total % (8 * (DV / DVT)) == 0) work = (work % 8) * (total / 8) + work / 8;
    const int tile = work % (DV / DVT);
    const int h = (work / (DV / DVT)) % H;
    const int n = work / ((DV / DVT) * H);
    const int cbase = tile * DVT;              // first d_v column of this tile

    long bos, eos;
    if (cu_seqlens) {
        long a = cu_seqlens[n], b = cu_seqlens[n + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        b = b < a ? a : (b > T ? T : b);
        bos = a;
        eos = b;
    } else {
        bos = (long)n * T;
        eos = bos + T;
    }
    const int len = (int)(eos - bos);
    const int nchunks = (len + C - 1) / C;

    // ---- state tile in accumulators: wave w owns state rows (d_v) cs0..cs0+15
    //      and d_k tiles dt0, dt0 + 1 ---------------------------------------------
    const int tid = tid0, lane = tid0 & 63, lr = lane & 15, lq = lane >> 4;
    const int cs0 = 16 * (wave & 1);
    const int dt0 = 2 * (wave >> 1);
    f32x4 accS[2];
    const size_t sbase = ((size_t)n * H + h) * DV * DK;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = cs0 + 4 * lq + r, d = 16 * (dt0 + t2) + lr;
            accS[t2][r] = s_init ? s_init[sbase + (size_t)(cbase + c) * DK + d] : 0.0f;
        }

    // ---- one-time LDS initialisation: the blocks above the diagonal of P, T_w
    //      and T_u are never written again; the bf16 copy of the state ---------
    for (int e = tid; e < C * LD_T; e += NT) {
        sP[e] = (bf16)0.0f;
        sTw[e] = (bf16)0.0f;
        sTu[e] = (bf16)0.0f;
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            sS[(cs0 + 4 * lq + r) * LD_S + 16 * (dt0 + t2) + lr] = (bf16)accS[t2][r];

    // ---- register prefetch of one chunk ---------------------------------------
    // Q: 2 x 16 B per thread (token row id/16, 8 columns). One 8 x 8 block (8
    // tokens x 8 channels) per thread of threads 0..159: K for 0..127 (token
    // block jb, d_k block cb), V for 128..159 (token block jb, d_v block cb of
    // this tile). g, beta: wave 0, one token per lane.
    const size_t tstride = (size_t)H * DK;     // elements between tokens (q, k, v)
    const bool blk_k = tid < 128, blk_v = tid >= 128 && tid < 160;
    const int blk_jb = blk_k ? (tid >> 4) : ((tid - 128) >> 2);
    const int blk_cb = blk_k ? (tid & 15) : ((tid - 128) & 3);
    const bf16 *qb0 = q + (size_t)bos * tstride + (size_t)h * DK + 8 * (tid & 15);
    const int qrow0 = tid >> 4;                // rows qrow0 and qrow0 + 32
    const bf16 *bb0 = (blk_k ? k + (size_t)h * DK : v + (size_t)h * DV + cbase) + 8 * blk_cb
                      + ((size_t)bos + 8 * blk_jb) * tstride;
    bf16x8 rq[2], rb[8];
    float rg = 0.f, rbeta = 0.f;
    auto fetch = [&](int ch) {
        const bf16x8 z8 = {};
        const size_t coff = (size_t)ch * C * tstride;
        const int base = ch * C;
        const bool full = base + C <= len;     // uniform
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int row = qrow0 + 32 * u;
            rq[u] = z8;
            if (full || base + row < len)
                rq[u] = *reinterpret_cast<const bf16x8 *>(qb0 + coff + (size_t)row * tstride);
        }
        if (blk_k || blk_v) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                rb[r] = z8;
                if (full || base + 8 * blk_jb + r < len)
                    rb[r] = *reinterpret_cast<const bf16x8 *>(bb0 + coff + (size_t)r * tstride);
            }
        }
        if (wave == 0) {
            const bool ok = base + lane < len;
            const size_t t = (size_t)bos + base + lane;
            rg = ok ? g[t * H + h] : 0.f;
            rbeta = ok ? beta[t * H + h] : 0.f;
        }
    };
    if (nchunks > 0) fetch(0);

    for (int ch = 0; ch < nchunks; ++ch) {
        const int base = ch * C;
        // Lane-derived indices are recomputed every chunk (the empty asm hides
        // the thread id from loop-invariant hoisting, which would otherwise
        // keep hundreds of precomputed LDS addresses live across the loop).
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, lr = lane & 15, lq = lane >> 4;
        // ---------------- load: registers -> LDS; decay prefix sums ----------------
#pragma unroll
        for (int u = 0; u < 2; ++u)
            *reinterpret_cast<bf16x8 *>(sQ + (qrow0 + 32 * u) * LD_QK + 8 * (tid & 15)) = rq[u];
        if (blk_k || blk_v) {
            bf16x8 tr[8];
            transpose8x8(rb, tr);
            if (blk_k) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    *reinterpret_cast<bf16x8 *>(sK + (8 * blk_jb + r) * LD_QK + 8 * blk_cb) = rb[r];
                    *reinterpret_cast<bf16x8 *>(sKt + (8 * blk_cb + r) * LD_T + 8 * blk_jb) = tr[r];
                }
            } else {
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    *reinterpret_cast<bf16x8 *>(sVt + (8 * blk_cb + r) * LD_T + 8 * blk_jb) = tr[r];
            }
        }
        if (wave == 0) {
            const float gam = wave_inclusive_scan(rg);
            const float glast = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gam), 63));
            float *sc = sSc;
            sc[SC_GAM * C + lane] = gam;
            sc[SC_BETA * C + lane] = rbeta;
            const float eg = __expf(gam);
            sc[SC_EG * C + lane] = eg;
            sc[SC_BEG * C + lane] = rbeta * eg;
            sc[SC_DEND * C + lane] = __expf(glast - gam);
        }
        lds_barrier();
        if (ch + 1 < nchunks) fetch(ch + 1);   // in flight during this chunk

        // ---------------- gram: A = -strict_lower(diag(beta) K K^T * Gamma) -------
#pragma unroll
        for (int item = 0; item < 10; ++item) {
            if ((item & 7) != wave || item >= 10) continue;     // wave-uniform
            const int ti = TI[item], tj = TJ[item];
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma<4>(acc, sK, LD_QK, 16 * ti, sK, LD_QK, 16 * tj, lane);
            const int i0 = 16 * ti + 4 * lq, j = 16 * tj + lr;
            const f32x4 gi = *reinterpret_cast<const f32x4 *>(sGam + i0);
            const f32x4 bi = *reinterpret_cast<const f32x4 *>(sBeta + i0);
            const float gj = sGam[j];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sA[(i0 + r) * LD_A + j] = j < i0 + r ? -bi[r] * acc[r] * __expf(gi[r] - gj) : 0.f;
        }
        lds_barrier();

        // store a finished fp32 block of T, and its bf16 T diag(beta e^gamma),
        // T diag(beta) images
        auto store_T = [&](int I, int J, f32x4 acc) {
            const int j = 16 * J + lr;
            const float bw = sBeg[j], bu = sBeta[j];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * I + 4 * lq + r;
                sT[i * LD_A + j] = acc[r];
                sTw[i * LD_T + j] = (bf16)(acc[r] * bw);
                sTu[i * LD_T + j] = (bf16)(acc[r] * bu);
            }
        };
        auto blkA = [&](int I, int J) { return sA + (16 * I) * LD_A + 16 * J; };
        auto blkT = [&](int I, int J) { return sT + (16 * I) * LD_A + 16 * J; };
        auto slot = [&](int s) { return sY + s * 16 * LD_Y; };

        if (wave < 4) {
            // ---- diagonal block D_b = (I - A_bb)^-1, b = wave: lane j < 16 owns
            // column j; x_i = [i == j] + sum_{m<i} A_bb[i][m] x_m
            if (lane < 16) {
                const int b = wave, j = lane;
                const float *ab = sA + (16 * b) * LD_A + 16 * b;
                float x[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float row[16];
#pragma unroll
                    for (int m4 = 0; m4 < 4; ++m4) {
                        const f32x4 v4 = *reinterpret_cast<const f32x4 *>(ab + i * LD_A + 4 * m4);
                        row[4 * m4] = v4[0]; row[4 * m4 + 1] = v4[1];
                        row[4 * m4 + 2] = v4[2]; row[4 * m4 + 3] = v4[3];
                    }
                    float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
                    for (int m = 0; m < i; ++m) acc += row[m] * x[m];
                    x[i] = acc;
                }
                const float bw = sBeg[16 * b + j], bu = sBeta[16 * b + j];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int ii = 16 * b + i, jj = 16 * b + j;
                    sT[ii * LD_A + jj] = x[i];
                    sTw[ii * LD_T + jj] = (bf16)(x[i] * bw);
                    sTu[ii * LD_T + jj] = (bf16)(x[i] * bu);
                }
            }
        } else {
            // ---- waves 4..7: P = lower_incl_diag(Q K^T * Gamma) ---------------------
#pragma unroll
            for (int item = 0; item < 10; ++item) {
                if ((item & 3) != wave - 4) continue;           // wave-uniform
                const int ti = TI[item], tj = TJ[item];
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mma<4>(acc, sQ, LD_QK, 16 * ti, sK, LD_QK, 16 * tj, lane);
                const int i0 = 16 * ti + 4 * lq, j = 16 * tj + lr;
                const f32x4 gi = *reinterpret_cast<const f32x4 *>(sGam + i0);
                const float gj = sGam[j];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sP[(i0 + r) * LD_T + j] = (bf16)(j <= i0 + r ? acc[r] * __expf(gi[r] - gj) : 0.f);
            }
        }
        lds_barrier();

        // ---- off-diagonal blocks. With D_b the diagonal inverses:
        //   T10 = D1 A10 D0,  T32 = D3 A32 D2                      (16-level)
        //   Y = [A20 A21; A30 A31] [D0 0; T10 D1] = [Y00 P21; Y10 P31]
        //   [T20 T21; T30 T31] = [D2 0; T32 D3] Y                  (32-level)
        // slots: 0, 1, 6, 7, 8 wave-private; 2 = P21 = A21 D1; 3 = R20 = A20 D0;
        //        4 = P31 = A31 D1; 5 = Q30 = A30 D0
        {
            const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
            f32x4 acc31 = z4;
            if (wave == 0) {
                st16(slot(0), LD_Y, mm16(z4, blkA(1, 0), LD_A, blkT(0, 0), LD_A, lane), lane);
                wave_lds_order();
                store_T(1, 0, mm16(z4, blkT(1, 1), LD_A, slot(0), LD_Y, lane));
            } else if (wave == 1) {
                st16(slot(1), LD_Y, mm16(z4, blkA(3, 2), LD_A, blkT(2, 2), LD_A, lane), lane);
                wave_lds_order();
                store_T(3, 2, mm16(z4, blkT(3, 3), LD_A, slot(1), LD_Y, lane));
            } else if (wave == 2) {
                st16(slot(2), LD_Y, mm16(z4, blkA(2, 1), LD_A, blkT(1, 1), LD_A, lane), lane);
                wave_lds_order();
                store_T(2, 1, mm16(z4, blkT(2, 2), LD_A, slot(2), LD_Y, lane));
            } else if (wave == 3) {
                st16(slot(3), LD_Y, mm16(z4, blkA(2, 0), LD_A, blkT(0, 0), LD_A, lane), lane);
            } else if (wave == 4) {
                st16(slot(4), LD_Y, mm16(z4, blkA(3, 1), LD_A, blkT(1, 1), LD_A, lane), lane);
                wave_lds_order();
                acc31 = mm16(z4, blkT(3, 3), LD_A, slot(4), LD_Y, lane);
            } else if (wave == 5) {
                st16(slot(5), LD_Y, mm16(z4, blkA(3, 0), LD_A, blkT(0, 0), LD_A, lane), lane);
            }
            lds_barrier();
            if (wave == 0) {
                // T20 = D2 (R20 + A21 T10)
                st16(slot(6), LD_Y, mm16(ld16(slot(3), LD_Y, lane), blkA(2, 1), LD_A, blkT(1, 0), LD_A, lane), lane);
                wave_lds_order();
                store_T(2, 0, mm16(z4, blkT(2, 2), LD_A, slot(6), LD_Y, lane));
            } else if (wave == 1) {
                // T30 = T32 (R20 + A21 T10) + D3 (Q30 + A31 T10)
                st16(slot(7), LD_Y, mm16(ld16(slot(3), LD_Y, lane), blkA(2, 1), LD_A, blkT(1, 0), LD_A, lane), lane);
                st16(slot(8), LD_Y, mm16(ld16(slot(5), LD_Y, lane), blkA(3, 1), LD_A, blkT(1, 0), LD_A, lane), lane);
                wave_lds_order();
                const f32x4 t = mm16(z4, blkT(3, 2), LD_A, slot(7), LD_Y, lane);
                store_T(3, 0, mm16(t, blkT(3, 3), LD_A, slot(8), LD_Y, lane));
            } else if (wave == 4) {
                // T31 = T32 P21 + D3 P31
                store_T(3, 1, mm16(acc31, blkT(3, 2), LD_A, slot(2), LD_Y, lane));
            }
            lds_barrier();
        }

        // ---------------- W = T_w K -> sWn = -W ; U = T_u V (registers) ------------
        {
            // wave w: d_k column tile w over the four row tiles
            const int d0 = 16 * wave;
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mma_tri(acc, ti, sTw, LD_T, sKt, LD_T, d0, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sWn[(16 * ti + 4 * lq + r) * LD_QK + d0 + lr] = (bf16)(-acc[r]);
            }
        }
        // wave w owns row tile ti = w/2 and d_v column tile ct = w%2 of U, Delta, O
        const int ti = wave >> 1, ct = wave & 1;
        const int i0 = 16 * ti + 4 * lq;           // first of this lane's 4 rows
        f32x4 accD = {0.f, 0.f, 0.f, 0.f};
        accD = mma_tri(accD, ti, sTu, LD_T, sVt, LD_T, 16 * ct, lane);
        lds_barrier();

        // ---------------- chain 1: Delta = U - W S^T ; O = Q S^T ----------------------
        accD = mma<4>(accD, sWn, LD_QK, 16 * ti, sS, LD_S, 16 * ct, lane);
        f32x4 accO = {0.f, 0.f, 0.f, 0.f};
        accO = mma<4>(accO, sQ, LD_QK, 16 * ti, sS, LD_S, 16 * ct, lane);
        {
            const f32x4 eg = *reinterpret_cast<const f32x4 *>(sEg + i0);
            const f32x4 de = *reinterpret_cast<const f32x4 *>(sDend + i0);
            const int c = 16 * ct + lr;
            bf16x4 dv, dw;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                dv[r] = (bf16)accD[r];
                dw[r] = (bf16)(accD[r] * de[r]);
                accO[r] *= eg[r];
            }
            *reinterpret_cast<bf16x4 *>(sDt + c * LD_T + i0) = dv;
            *reinterpret_cast<bf16x4 *>(sDtw + c * LD_T + i0) = dw;
        }
        lds_barrier();

        // ---------------- chain 2: O += P Delta ; S <- e^{g63} S + Delta~^T K ----------
        accO = mma_tri(accO, ti, sP, LD_T, sDt, LD_T, 16 * ct, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) sO[(i0 + r) * LD_O + 16 * ct + lr] = (bf16)(scale * accO[r]);
        {
            const float eend = sEg[C - 1];
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
                for (int r = 0; r < 4; ++r) accS[t2][r] *= eend;
                accS[t2] = mma<2>(accS[t2], sDtw, LD_T, cs0, sKt, LD_T, 16 * (dt0 + t2), lane);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sS[(cs0 + 4 * lq + r) * LD_S + 16 * (dt0 + t2) + lr] = (bf16)accS[t2][r];
            }
        }
        lds_barrier();
        // output tile 64 x 32 bf16: one 16-byte store per thread of the first 256
        if (tid < 256) {
            const int row = tid >> 2, col = 8 * (tid & 3);
            if (base + row < len)
                *reinterpret_cast<bf16x8 *>(o + ((size_t)bos + base + row) * H * DV + (size_t)h * DV + cbase + col) =
                    *reinterpret_cast<const bf16x8 *>(sO + row * LD_O + col);
        }
    }

    if (s_final) {
        const int lane = tid0 & 63, lr = lane & 15, lq = lane >> 4;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = cs0 + 4 * lq + r, d = 16 * (dt0 + t2) + lr;
                s_final[sbase + (size_t)(cbase + c) * DK + d] = accS[t2][r];
            }
    }
}

hipError_t launch_prefill_chunk(const void *q, const void *k, const void *v, const float *g,
                                const float *beta, const float *s_init, float *s_final, void *o,
                                const int32_t *cu, int T, int H, int N, float scale,
                                hipStream_t stream)
{
    static bool attr_done = false;
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute((const void *)prefill_chunk_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_done = true;
    }
    dim3 grid((unsigned)((DV / DVT) * H * N)), block(NT);
    hipLaunchKernelGGL(prefill_chunk_kernel, grid, block, LDS_BYTES, stream, (const bf16 *)q,
                       (const bf16 *)k, (const bf16 *)v, g, beta, s_init, s_final, (bf16 *)o, cu,
                       T, H, scale);
    return hipGetLastError();
}

}  // namespace gdn
