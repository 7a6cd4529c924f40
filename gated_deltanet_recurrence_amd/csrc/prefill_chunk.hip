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
static_assert(4 * 256 * 4 <= SZ_Y, "solve scratch fits");
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
    // this tile). g, beta: wave 3, one token per lane.
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
        if (wave == 3) {
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
        if (wave == 3) {
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
        // one 16 x 16 tile of A = -strict_lower(diag(beta) K K^T * Gamma), in
        // accumulator layout
        auto gram_tile = [&](int ti, int tj) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma<4>(acc, sK, LD_QK, 16 * ti, sK, LD_QK, 16 * tj, lane);
            const int i0 = 16 * ti + 4 * lq, j = 16 * tj + lr;
            const f32x4 gi = *reinterpret_cast<const f32x4 *>(sGam + i0);
            const f32x4 bi = *reinterpret_cast<const f32x4 *>(sBeta + i0);
            const float gj = sGam[j];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[r] = j < i0 + r ? -bi[r] * acc[r] * __expf(gi[r] - gj) : 0.f;
            return acc;
        };
        // one 16 x 16 tile of P = lower_incl_diag(Q K^T * Gamma) -> sP
        auto p_tile = [&](int item) {
            const int ti = TI[item], tj = TJ[item];
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma<4>(acc, sQ, LD_QK, 16 * ti, sK, LD_QK, 16 * tj, lane);
            const int i0 = 16 * ti + 4 * lq, j = 16 * tj + lr;
            const f32x4 gi = *reinterpret_cast<const f32x4 *>(sGam + i0);
            const float gj = sGam[j];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sP[(i0 + r) * LD_T + j] = (bf16)(j <= i0 + r ? acc[r] * __expf(gi[r] - gj) : 0.f);
        };

        // ---------------- gram + diagonal blocks of T = (I - A)^-1 -----------------
        if (wave < 4) {
            // Wave b forms the diagonal tile A_bb and inverts I - A_bb by forward
            // substitution, D[i][j] = [i == j] + sum_{m<i} A_bb[i][m] D[m][j].
            // Lane 4j + p owns column j and the terms m = p (mod 4); the four
            // partial sums meet by DPP inside the quad. A_bb goes through a
            // wave-private LDS copy laid out [p][i][m/4] so each lane reads its
            // terms of row i as one float4.
            const int b = wave;
            const f32x4 ab = gram_tile(b, b);
            float *ap = sY + b * 256;                   // [4][16][4] floats
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * lq + r, m = lr;
                ap[(m & 3) * 64 + i * 4 + (m >> 2)] = ab[r];
            }
            wave_lds_order();
            const int jc = lane >> 2, p = lane & 3;
            const float *myp = ap + p * 64;
            f32x4 arow[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) arow[i] = *reinterpret_cast<const f32x4 *>(myp + 4 * i);
            float xs[4] = {0.f, 0.f, 0.f, 0.f};          // xs[t] = D[p + 4t][jc]
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float part = arow[i][0] * xs[0] + arow[i][1] * xs[1] + arow[i][2] * xs[2]
                           + arow[i][3] * xs[3];
                part += dpp_f32<DPP_QUAD_XOR1>(part);
                part += dpp_f32<DPP_QUAD_XOR2>(part);
                const float xi = part + (i == jc ? 1.f : 0.f);
                if (p == (i & 3)) xs[i >> 2] = xi;
            }
            const int jj = 16 * b + jc;
            const float bw = sBeg[jj], bu = sBeta[jj];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int ii = 16 * b + p + 4 * t;
                sT[ii * LD_A + jj] = xs[t];
                sTw[ii * LD_T + jj] = (bf16)(xs[t] * bw);
                sTu[ii * LD_T + jj] = (bf16)(xs[t] * bu);
            }
        } else {
            // waves 4..7: the six off-diagonal tiles of A
            auto put = [&](int ti, int tj) {
                const f32x4 a = gram_tile(ti, tj);
#pragma unroll
                for (int r = 0; r < 4; ++r) sA[(16 * ti + 4 * lq + r) * LD_A + 16 * tj + lr] = a[r];
            };
            if (wave == 4) { put(1, 0); put(3, 0); }
            else if (wave == 5) { put(2, 0); put(3, 1); }
            else if (wave == 6) put(2, 1);
            else put(3, 2);
        }
        lds_barrier();

        // ---- off-diagonal blocks of T. With D_b the diagonal inverses:
        //   T10 = D1 A10 D0,  T32 = D3 A32 D2                      (16-level)
        //   Y = [A20 A21; A30 A31] [D0 0; T10 D1] = [Y00 P21; Y10 P31]
        //   [T20 T21; T30 T31] = [D2 0; T32 D3] Y                  (32-level)
        // Right factors produced by a wave stay in its registers (acc_to_bop);
        // waves without a block product form tiles of P meanwhile.
        {
            const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
            f32x4 h0 = z4, h1 = z4;                     // products kept for the 32-level
            if (wave == 0) {
                const f32x4 c = mm16(z4, blkA(1, 0), LD_A, blkT(0, 0), LD_A, lane);
                store_T(1, 0, mm16_rb(z4, blkT(1, 1), LD_A, acc_to_bop(c), lane));
            } else if (wave == 1) {
                const f32x4 c = mm16(z4, blkA(3, 2), LD_A, blkT(2, 2), LD_A, lane);
                store_T(3, 2, mm16_rb(z4, blkT(3, 3), LD_A, acc_to_bop(c), lane));
            } else if (wave == 2) {
                const f32x4 c = mm16(z4, blkA(2, 1), LD_A, blkT(1, 1), LD_A, lane);
                store_T(2, 1, mm16_rb(z4, blkT(2, 2), LD_A, acc_to_bop(c), lane));
            } else if (wave == 3) {
                h0 = mm16(z4, blkA(2, 0), LD_A, blkT(0, 0), LD_A, lane);            // R20
            } else if (wave == 4) {
                h0 = mm16(z4, blkA(2, 1), LD_A, blkT(1, 1), LD_A, lane);            // P21
                h1 = mm16(z4, blkA(3, 1), LD_A, blkT(1, 1), LD_A, lane);            // P31
            } else if (wave == 5) {
                h0 = mm16(z4, blkA(2, 0), LD_A, blkT(0, 0), LD_A, lane);            // R20
                h1 = mm16(z4, blkA(3, 0), LD_A, blkT(0, 0), LD_A, lane);            // Q30
            } else if (wave == 6) {
                p_tile(0); p_tile(2);
            } else {
                p_tile(1); p_tile(3);
            }
            lds_barrier();
            if (wave == 3) {
                // T20 = D2 (R20 + A21 T10)
                const f32x4 y00 = mm16(h0, blkA(2, 1), LD_A, blkT(1, 0), LD_A, lane);
                store_T(2, 0, mm16_rb(z4, blkT(2, 2), LD_A, acc_to_bop(y00), lane));
            } else if (wave == 4) {
                // T31 = T32 P21 + D3 P31
                const f32x4 t = mm16_rb(z4, blkT(3, 2), LD_A, acc_to_bop(h0), lane);
                store_T(3, 1, mm16_rb(t, blkT(3, 3), LD_A, acc_to_bop(h1), lane));
            } else if (wave == 5) {
                // T30 = T32 (R20 + A21 T10) + D3 (Q30 + A31 T10)
                const f32x4 y00 = mm16(h0, blkA(2, 1), LD_A, blkT(1, 0), LD_A, lane);
                const f32x4 y10 = mm16(h1, blkA(3, 1), LD_A, blkT(1, 0), LD_A, lane);
                const f32x4 t = mm16_rb(z4, blkT(3, 2), LD_A, acc_to_bop(y00), lane);
                store_T(3, 0, mm16_rb(t, blkT(3, 3), LD_A, acc_to_bop(y10), lane));
            } else if (wave == 0) {
                p_tile(4);
            } else if (wave == 1) {
                p_tile(5);
            } else if (wave == 2) {
                p_tile(6);
            } else if (wave == 6) {
                p_tile(7); p_tile(9);
            } else {
                p_tile(8);
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
