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
// Everything up to T_w and T_u depends on one chunk of one head only, and
// is the same for every d_v column. The first pass (chunk_prep) computes it
// once per (chunk, head), fully in parallel over all chunks; the second pass
// (chunk_chain) walks the chunks of each sequence in order and carries the
// state. Splitting takes the triangular solve off the sequential path and
// stops the d_v tiles of a head from each repeating it; the price is 12 KiB
// of bf16 T_w / T_u per (chunk, head) written to the caller's workspace and
// read back: 384 B of HBM traffic per token-head on top of the 1032 B of
// q, k, v, o, g and beta.
//
// Workspace layout: for head h and chunk slot s, 6144 bf16 at
// ((h * nslots) + s) * 6144: T_w then T_u, each as the three non-zero 32 x 32
// blocks (rows 0-31 x cols 0-31, rows 32-63 x cols 0-31, rows 32-63 x cols
// 32-63), row-major. Chunk c of sequence n has slot (bos_n / 64) + n + c,
// where bos_n is its first token: slots of different sequences never
// collide and every slot is below nslots = total_tokens / 64 + N + 1.
#include "chunk_common.h"

namespace gdn {

namespace split {

using namespace chunk;

constexpr int C = 64;
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int TWU_ELEMS = 2 * 3 * 32 * 32;    // bf16 per (chunk, head) in the workspace

// ---------------------------------------------------------------------------
// Pass 1: chunk_prep. One workgroup of 4 waves per (chunk slot, head).
// ---------------------------------------------------------------------------
constexpr int P_NT = 256;
constexpr int P_LD_K = DK + 8;                 // bf16 row stride of K
constexpr int P_LD_A = C + 4;                  // fp32 row stride of A and T
constexpr int P_QB = 4 * 68;                   // one 16 x 16 block in the quad layout (floats)
constexpr int P_SZ_R1 = C * P_LD_K * 2;        // 17408: K, then T
constexpr int P_SZ_A = C * P_LD_A * 4;         // 17408
constexpr int P_SZ_Y = 2 * 4 * P_QB * 4;       // 8704: two diagonal 32 x 32 tiles, quad layout
constexpr int P_SZ_SC = 3 * C * 4;             // gamma, beta, beta e^gamma
constexpr int P_OFF_R1 = 0;
constexpr int P_OFF_A = P_OFF_R1 + P_SZ_R1;
constexpr int P_OFF_Y = P_OFF_A + P_SZ_A;
constexpr int P_OFF_SC = P_OFF_Y + P_SZ_Y;
constexpr int P_LDS_BYTES = P_OFF_SC + P_SZ_SC;
static_assert(C * P_LD_A * 4 <= P_SZ_R1, "T fits where K was");
static_assert(P_LDS_BYTES <= 48 * 1024, "three prep workgroups per CU");

// ---------------------------------------------------------------------------
// Pass 2: chunk_chain. One workgroup of 8 waves per (32-wide d_v tile, head,
// sequence).
// ---------------------------------------------------------------------------
constexpr int DVT = 32;
constexpr int NT = 512;
constexpr int LD_QK = DK + 8;                  // sQ, sK, sWn rows (bf16)
constexpr int LD_T = C + 8;                    // token-contiguous bf16 rows
constexpr int LD_S = DK + 8;                   // sS rows (bf16)
constexpr int LD_O = DVT + 8;                  // output staging (bf16)
constexpr int SZ_QK = C * LD_QK * 2;           // 17408
constexpr int SZ_KT = DK * LD_T * 2;           // 18432
constexpr int SZ_VT = DVT * LD_T * 2;          // 4608
constexpr int SZ_TT = C * LD_T * 2;            // 9216
constexpr int SZ_S = DVT * LD_S * 2;           // 8704
constexpr int SZ_O = C * LD_O * 2;             // 5120
constexpr int SZ_SC = 3 * C * 4;               // gamma, e^gamma, e^{gamma_63 - gamma}
constexpr int OFF_Q = 0;
constexpr int OFF_K = OFF_Q + SZ_QK;
constexpr int OFF_KT = OFF_K + SZ_QK;
constexpr int OFF_VT = OFF_KT + SZ_KT;
constexpr int OFF_TW = OFF_VT + SZ_VT;
constexpr int OFF_TU = OFF_TW + SZ_TT;
constexpr int OFF_WN = OFF_TU + SZ_TT;
constexpr int OFF_P = OFF_WN + SZ_QK;
constexpr int OFF_S = OFF_P + SZ_TT;
constexpr int OFF_DT = OFF_S + SZ_S;
constexpr int OFF_DTW = OFF_DT + SZ_VT;
constexpr int OFF_O = OFF_DTW + SZ_VT;
constexpr int OFF_SC = OFF_O + SZ_O;
constexpr int LDS_BYTES = OFF_SC + SZ_SC;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

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

// ---------------------------------------------------------------------------
// chunk_prep: T_w and T_u of one (chunk, head).
//
//   load   K (64 x 128) into LDS; gamma = prefix sum of g (wave 0, DPP scan)
//   gram   wave 0: tile (0,0) of A, wave 1: tile (1,1), wave 2: tile (1,0)
//          (v_mfma_f32_32x32x16_bf16, masked and scaled in registers)
//   solve  wave w inverts the 16 x 16 diagonal block w of I - A by forward
//          substitution: lane 4j + p owns column j and the terms m = p mod 4
//          of every row's dot product, finished with two DPP quad sums
//   L1/L2  the off-diagonal blocks of T by two levels of 2 x 2 block
//          inversion, (L^-1)_21 = L22^-1 A21 L11^-1 (fp32 16x16x4 MFMA)
//   store  T diag(beta e^gamma) and T diag(beta), bf16, to the workspace
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(P_NT)
chunk_prep_kernel(const bf16 *__restrict__ k, const float *__restrict__ g,
                  const float *__restrict__ beta, const int32_t *__restrict__ cu_seqlens,
                  bf16 *__restrict__ ws, int T, int H, int N, int nslots)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    bf16 *sK = reinterpret_cast<bf16 *>(smem + P_OFF_R1);
    float *sT = reinterpret_cast<float *>(smem + P_OFF_R1);
    float *sA = reinterpret_cast<float *>(smem + P_OFF_A);
    float *sY = reinterpret_cast<float *>(smem + P_OFF_Y);
    float *sGam = reinterpret_cast<float *>(smem + P_OFF_SC);
    float *sBeta = sGam + C;
    float *sBeg = sBeta + C;

    const int slot = (int)blockIdx.x, h = (int)blockIdx.y;
    const int tid = (int)threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;

    // sequence of this slot: the last n whose first slot is <= slot
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (first_slot(cu_seqlens, mid, T) <= slot) lo = mid;
        else hi = mid - 1;
    }
    const int n = lo;
    long bos, eos;
    seq_bounds(cu_seqlens, n, T, bos, eos);
    const long c = slot - ((bos >> 6) + n);
    const long len = eos - bos;
    if (c < 0 || c * C >= len) return;         // unused slot (uniform)
    const long row0 = bos + c * C;
    const int nvalid = (int)(len - c * C < C ? len - c * C : C);

    // ---- load K rows (zero past the end of the sequence), g and beta ----
    {
        const int col = 8 * (tid & 15);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = (tid >> 4) + 16 * u;
            bf16x8 x = {};
            if (r < nvalid)
                x = *reinterpret_cast<const bf16x8 *>(k + (size_t)(row0 + r) * H * DK + (size_t)h * DK + col);
            *reinterpret_cast<bf16x8 *>(sK + r * P_LD_K + col) = x;
        }
    }
    if (wave == 0) {
        const bool ok = lane < nvalid;
        const size_t t = (size_t)(row0 + lane) * H + h;
        const float gv = ok ? g[t] : 0.f, bv = ok ? beta[t] : 0.f;
        const float gam = wave_inclusive_scan(gv);
        sGam[lane] = gam;
        sBeta[lane] = bv;
        sBeg[lane] = bv * __expf(gam);
    }
    lds_barrier();

    const int l32 = lane & 31, lh = lane >> 5, lr = lane & 15, lq = lane >> 4;
    auto rows4 = [&](const float *v, int i0, int qq) {
        return *reinterpret_cast<const f32x4 *>(v + i0 + 8 * qq + 4 * lh);
    };

    // ---- gram tiles of A = -strict_lower(diag(beta) K K^T * Gamma) ----
    if (wave < 3) {
        const int ti = wave == 0 ? 0 : 1, tj = wave == 1 ? 1 : 0;
        const int j = 32 * tj + l32;
        const float gj = sGam[j];
        f32x4 gi[4], bi[4];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            gi[qq] = rows4(sGam, 32 * ti, qq);
            bi[qq] = rows4(sBeta, 32 * ti, qq);
        }
        f32x16 at = {};
        at = mma32_2<4>(at, sK, P_LD_K, 32 * ti, sK, P_LD_K, 32 * tj, lane);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const int r = 4 * qq + s2, i = 32 * ti + acc_row(r, lane);
                at[r] = j < i ? -bi[qq][s2] * at[r] * __expf(gi[qq][s2] - gj) : 0.f;
            }
        // whole tile into sA (only the off-diagonal 16 x 16 blocks are read there)
#pragma unroll
        for (int r = 0; r < 16; ++r) sA[(32 * ti + acc_row(r, lane)) * P_LD_A + j] = at[r];
        if (wave < 2) {
            // and the diagonal tile in the solve's quad layout: element (i, m) of
            // 16 x 16 block b at b * P_QB + (m % 4) * 68 + 4 i + m / 4
            float *ap = sY + wave * (4 * P_QB);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int it = acc_row(r, lane), jt = l32;
                const int blk = 2 * (it >> 4) + (jt >> 4), i = it & 15, m = jt & 15;
                ap[blk * P_QB + (m & 3) * 68 + i * 4 + (m >> 2)] = at[r];
            }
        }
    }
    lds_barrier();                             // A complete; K no longer read

    // ---- diagonal blocks: D_w = (I - A_ww)^-1, D[i][j] = [i==j] + sum_{m<i} A[i][m] D[m][j]
    {
        const int jc = lane >> 2, p = lane & 3;
        const float *myp = sY + (wave >> 1) * (4 * P_QB) + 3 * (wave & 1) * P_QB + p * 68;
        f32x4 arow[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) arow[i] = *reinterpret_cast<const f32x4 *>(myp + 4 * i);
        float xs[4] = {0.f, 0.f, 0.f, 0.f};   // xs[t] = D[p + 4t][jc]
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float part = arow[i][0] * xs[0] + arow[i][1] * xs[1] + arow[i][2] * xs[2]
                       + arow[i][3] * xs[3];
            part += dpp_f32<DPP_QUAD_XOR1>(part);
            part += dpp_f32<DPP_QUAD_XOR2>(part);
            const float xi = part + (i == jc ? 1.f : 0.f);
            if (p == (i & 3)) xs[i >> 2] = xi;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) sT[(16 * wave + p + 4 * t) * P_LD_A + 16 * wave + jc] = xs[t];
    }
    lds_barrier();

    // ---- off-diagonal blocks of T. With D_b the diagonal inverses:
    //   T10 = D1 A10 D0,  T32 = D3 A32 D2,  T21 = D2 A21 D1           (16-level)
    //   T20 = D2 (A20 D0 + A21 T10)
    //   T31 = T32 (A21 D1) + D3 (A31 D1)
    //   T30 = T32 (A20 D0 + A21 T10) + D3 (A30 D0 + A31 T10)          (32-level)
    auto blkA = [&](int I, int J) { return sA + (16 * I) * P_LD_A + 16 * J; };
    auto blkT = [&](int I, int J) { return sT + (16 * I) * P_LD_A + 16 * J; };
    auto store_T = [&](int I, int J, f32x4 acc) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sT[(16 * I + 4 * lq + r) * P_LD_A + 16 * J + lr] = acc[r];
    };
    {
        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
        f32x4 h0 = z4, h1 = z4;
        if (wave == 0) {
            const f32x4 c10 = mm16(z4, blkA(1, 0), P_LD_A, blkT(0, 0), P_LD_A, lane);
            h0 = mm16(z4, blkA(2, 0), P_LD_A, blkT(0, 0), P_LD_A, lane);              // A20 D0
            store_T(1, 0, mm16_rb(z4, blkT(1, 1), P_LD_A, acc_to_bop(c10), lane));
        } else if (wave == 1) {
            const f32x4 c32 = mm16(z4, blkA(3, 2), P_LD_A, blkT(2, 2), P_LD_A, lane);
            store_T(3, 2, mm16_rb(z4, blkT(3, 3), P_LD_A, acc_to_bop(c32), lane));
        } else if (wave == 2) {
            h0 = mm16(z4, blkA(2, 1), P_LD_A, blkT(1, 1), P_LD_A, lane);              // A21 D1
            h1 = mm16(z4, blkA(3, 1), P_LD_A, blkT(1, 1), P_LD_A, lane);              // A31 D1
            store_T(2, 1, mm16_rb(z4, blkT(2, 2), P_LD_A, acc_to_bop(h0), lane));
        } else {
            h0 = mm16(z4, blkA(2, 0), P_LD_A, blkT(0, 0), P_LD_A, lane);              // A20 D0
            h1 = mm16(z4, blkA(3, 0), P_LD_A, blkT(0, 0), P_LD_A, lane);              // A30 D0
        }
        lds_barrier();
        if (wave == 0) {
            const f32x4 y00 = mm16(h0, blkA(2, 1), P_LD_A, blkT(1, 0), P_LD_A, lane);
            store_T(2, 0, mm16_rb(z4, blkT(2, 2), P_LD_A, acc_to_bop(y00), lane));
        } else if (wave == 2) {
            const f32x4 t = mm16_rb(z4, blkT(3, 2), P_LD_A, acc_to_bop(h0), lane);
            store_T(3, 1, mm16_rb(t, blkT(3, 3), P_LD_A, acc_to_bop(h1), lane));
        } else if (wave == 3) {
            const f32x4 y00 = mm16(h0, blkA(2, 1), P_LD_A, blkT(1, 0), P_LD_A, lane);
            const f32x4 y10 = mm16(h1, blkA(3, 1), P_LD_A, blkT(1, 0), P_LD_A, lane);
            const f32x4 t = mm16_rb(z4, blkT(3, 2), P_LD_A, acc_to_bop(y00), lane);
            store_T(3, 0, mm16_rb(t, blkT(3, 3), P_LD_A, acc_to_bop(y10), lane));
        }
        lds_barrier();
    }

    // ---- T_w = T diag(beta e^gamma), T_u = T diag(beta) -> workspace (bf16,
    //      three 32 x 32 blocks each; 16-byte pieces, consecutive per thread) ----
    bf16 *dst = ws + ((size_t)h * nslots + slot) * TWU_ELEMS;
#pragma unroll
    for (int u = 0; u < 3; ++u) {
        const int e = tid + P_NT * u;          // 0..767
        const int mat = e >= 384 ? 1 : 0;
        const int rem = e - 384 * mat;
        const int blk = rem >> 7, row = (rem >> 2) & 31, cc = rem & 3;
        const int i = 32 * (blk > 0 ? 1 : 0) + row, j0 = 32 * (blk == 2 ? 1 : 0) + 8 * cc;
        const float *sc = mat ? sBeta : sBeg;
        const f32x4 t0 = *reinterpret_cast<const f32x4 *>(sT + i * P_LD_A + j0);
        const f32x4 t1 = *reinterpret_cast<const f32x4 *>(sT + i * P_LD_A + j0 + 4);
        const f32x4 s0 = *reinterpret_cast<const f32x4 *>(sc + j0);
        const f32x4 s1 = *reinterpret_cast<const f32x4 *>(sc + j0 + 4);
        // the 16 x 16 blocks above the diagonal of T are zero (not stored in sT)
        const bool zero = (j0 >> 4) > (i >> 4);
        bf16x8 out;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            out[e2] = (bf16)(zero ? 0.f : t0[e2] * s0[e2]);
            out[e2 + 4] = (bf16)(zero ? 0.f : t1[e2] * s1[e2]);
        }
        *reinterpret_cast<bf16x8 *>(dst + 8 * e) = out;
    }
}

// ---------------------------------------------------------------------------
// chunk_chain: the sequential pass. One workgroup of 8 waves per (32-wide d_v
// tile, head, sequence); waves 0-3 keep S^T (128 x 32, fp32) in MFMA
// accumulators for the whole sequence, 32 x 32 each; a bf16 copy of S in LDS
// is the operand of the next chunk. The next chunk's q, k, v, T_w, T_u are
// loaded into registers while the current one is computed.
//
//   load   Q, K row-major, K^T and V^T (token-contiguous, column-swizzled),
//          T_w, T_u into LDS; gamma (wave 3); the previous chunk's output
//          rows leave LDS for HBM
//   prep   W^T = K^T T_w^T (one 32 x 32 tile per wave) -> LDS as -W;
//          U = T_u V (waves 0-1, registers); P^T tiles of
//          P = lower_incl_diag(Q K^T * Gamma) (waves 2, 3, 5) -> LDS;
//          (Q S^T)^T = S Q^T (waves 6-7, registers)
//   delta  Delta = U - W S^T (waves 0-1) -> LDS as Delta^T and Delta~^T
//   out    O^T = (Q S^T)^T diag(e^gamma) + Delta^T P^T (waves 6-7) -> LDS;
//          S^T <- e^{gamma_63} S^T + K^T Delta~ (waves 0-3)
//
// Every product is arranged so that a lane's accumulator holds 4 consecutive
// elements of a stored row (8-byte LDS writes).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(NT, 1)
chunk_chain_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                   const bf16 *__restrict__ v, const float *__restrict__ g,
                   const bf16 *__restrict__ ws, const float *s_init, float *s_final,
                   bf16 *__restrict__ o, const int32_t *__restrict__ cu_seqlens, int T, int H,
                   int nslots, float scale)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    bf16 *sQ = reinterpret_cast<bf16 *>(smem + OFF_Q);
    bf16 *sK = reinterpret_cast<bf16 *>(smem + OFF_K);
    bf16 *sKt = reinterpret_cast<bf16 *>(smem + OFF_KT);
    bf16 *sVt = reinterpret_cast<bf16 *>(smem + OFF_VT);
    bf16 *sTw = reinterpret_cast<bf16 *>(smem + OFF_TW);
    bf16 *sTu = reinterpret_cast<bf16 *>(smem + OFF_TU);
    bf16 *sWn = reinterpret_cast<bf16 *>(smem + OFF_WN);
    bf16 *sP = reinterpret_cast<bf16 *>(smem + OFF_P);
    bf16 *sS = reinterpret_cast<bf16 *>(smem + OFF_S);
    bf16 *sDt = reinterpret_cast<bf16 *>(smem + OFF_DT);
    bf16 *sDtw = reinterpret_cast<bf16 *>(smem + OFF_DTW);
    bf16 *sO = reinterpret_cast<bf16 *>(smem + OFF_O);
    float *sGam = reinterpret_cast<float *>(smem + OFF_SC);
    float *sEg = sGam + C;
    float *sDend = sEg + C;

    const int tid0 = (int)threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    // work item (sequence n, head h, d_v tile); workgroup w runs on XCD w % 8,
    // so each XCD gets a contiguous range and the four tiles of a head share
    // an L2
    int work = (int)blockIdx.x;
    const int total = (int)gridDim.x;
    if (total % (8 * (DV / DVT)) == 0) work = (work % 8) * (total / 8) + work / 8;
    const int tile = work % (DV / DVT);
    const int h = (work / (DV / DVT)) % H;
    const int n = work / ((DV / DVT) * H);
    const int cbase = tile * DVT;

    long bos, eos;
    seq_bounds(cu_seqlens, n, T, bos, eos);
    const int len = (int)(eos - bos);
    const int nchunks = (len + C - 1) / C;
    const bf16 *wsh = ws + ((size_t)h * nslots + (size_t)((bos >> 6) + n)) * TWU_ELEMS;

    // ---- state: wave w < 4 holds S^T rows d = 32w.., columns c (this tile):
    //      accS[r] = S[cbase + lane%32][32w + acc_row(r)] ----
    f32x16 accS = {};
    const size_t sbase = ((size_t)n * H + h) * DV * DK;
    if (wave < 4) {
        const int lane = tid0 & 63;
        if (s_init) {
            const float *src = s_init + sbase + (size_t)(cbase + (lane & 31)) * DK + 32 * wave + 4 * (lane >> 5);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(src + 8 * qq);
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) accS[4 * qq + s2] = x[s2];
            }
        }
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            bf16x4 x;
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) x[s2] = (bf16)accS[4 * qq + s2];
            *reinterpret_cast<bf16x4 *>(sS + (lane & 31) * LD_S + 32 * wave + 8 * qq + 4 * (lane >> 5)) = x;
        }
    }

    // ---- register prefetch of one chunk ----
    // Q: 2 x 16 B per thread. One 8 x 8 block per thread of threads 0..159: K
    // for 0..127 (token block jb, d_k block cb), V for 128..159. T_w / T_u: one
    // 16-byte piece of each per thread of threads 128..511. g: wave 3.
    const int tid = tid0;
    const int tstride = H * DK;
    const bool blk_k = tid < 128, blk_v = tid >= 128 && tid < 160, has_tt = tid >= 128;
    const int blk_jb = blk_k ? (tid >> 4) : ((tid - 128) >> 2);
    const int blk_cb = blk_k ? (tid & 15) : ((tid - 128) & 3);
    const int qrow0 = tid >> 4;
    const int tt_e = tid - 128;                // piece index within T_w (and T_u)
    const bf16 *qbase = q + (size_t)bos * tstride + (size_t)h * DK;
    const bf16 *kbase = k + (size_t)bos * tstride + (size_t)h * DK;
    const bf16 *vbase = v + (size_t)bos * tstride + (size_t)h * DV + cbase;
    const int qoff = qrow0 * tstride + 8 * (tid & 15);
    const int boff = 8 * blk_jb * tstride + 8 * blk_cb;
    bf16x8 rq[2], rb[8], rtt[2];
    float rg = 0.f;
    auto fetch = [&](int ch) {
        const bf16x8 z8 = {};
        const size_t coff = (size_t)ch * C * tstride;
        const int base = ch * C;
        const int lane = tid & 63;
        const bf16 *qc = qbase + coff, *kc = kbase + coff, *vc = vbase + coff;
        if (base + C <= len) {
#pragma unroll
            for (int u = 0; u < 2; ++u)
                rq[u] = *reinterpret_cast<const bf16x8 *>(qc + qoff + 32 * u * tstride);
            if (blk_k) {
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    rb[r] = *reinterpret_cast<const bf16x8 *>(kc + boff + r * tstride);
            } else if (blk_v) {
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    rb[r] = *reinterpret_cast<const bf16x8 *>(vc + boff + r * tstride);
            }
        } else {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                rq[u] = z8;
                if (base + qrow0 + 32 * u < len)
                    rq[u] = *reinterpret_cast<const bf16x8 *>(qc + qoff + 32 * u * tstride);
            }
            if (blk_k || blk_v) {
                const bf16 *bc = blk_k ? kc : vc;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    rb[r] = z8;
                    if (base + 8 * blk_jb + r < len)
                        rb[r] = *reinterpret_cast<const bf16x8 *>(bc + boff + r * tstride);
                }
            }
        }
        if (has_tt) {
            const bf16 *wc = wsh + (size_t)ch * TWU_ELEMS;
            rtt[0] = *reinterpret_cast<const bf16x8 *>(wc + 8 * tt_e);
            rtt[1] = *reinterpret_cast<const bf16x8 *>(wc + 8 * (tt_e + 384));
        }
        if (wave == 3) {
            const bool ok = base + lane < len;
            rg = ok ? g[((size_t)bos + base + lane) * H + h] : 0.f;
        }
    };
    if (nchunks > 0) fetch(0);

    for (int ch = 0; ch < nchunks; ++ch) {
        const int base = ch * C;
        int tidl = tid0;
        asm volatile("" : "+v"(tidl));         // keep lane-derived addresses out of loop-invariant hoisting
        const int lane = tidl & 63;
        const int l32 = lane & 31, lh = lane >> 5;

        // ---------------- load: registers -> LDS; decay prefix sums ----------------
        // the previous chunk's output rows (64 x 32 bf16) leave LDS first
        if (ch > 0 && tidl < 256) {
            const int row = tidl >> 2, col = 8 * (tidl & 3);
            if (base - C + row < len)
                *reinterpret_cast<bf16x8 *>(o + ((size_t)bos + base - C + row) * H * DV + (size_t)h * DV + cbase + col) =
                    *reinterpret_cast<const bf16x8 *>(sO + row * LD_O + col);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
            *reinterpret_cast<bf16x8 *>(sQ + (qrow0 + 32 * u) * LD_QK + 8 * (tidl & 15)) = rq[u];
        if (blk_k || blk_v) {
            bf16x8 tr[8];
            transpose8x8(rb, tr);
            if (blk_k) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    *reinterpret_cast<bf16x8 *>(sK + (8 * blk_jb + r) * LD_QK + 8 * blk_cb) = rb[r];
                    *reinterpret_cast<bf16x8 *>(sKt + (8 * blk_cb + r) * LD_T + 8 * (blk_jb ^ ((blk_cb >> 1) & 7))) = tr[r];
                }
            } else {
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    *reinterpret_cast<bf16x8 *>(sVt + (8 * blk_cb + r) * LD_T + 8 * (blk_jb ^ (blk_cb >> 1))) = tr[r];
            }
        }
        if (has_tt) {
            const int e = tidl - 128;
            const int blk = e >> 7, row = (e >> 2) & 31, cc = e & 3;
            const int off = (32 * (blk > 0 ? 1 : 0) + row) * LD_T + 32 * (blk == 2 ? 1 : 0) + 8 * cc;
            *reinterpret_cast<bf16x8 *>(sTw + off) = rtt[0];
            *reinterpret_cast<bf16x8 *>(sTu + off) = rtt[1];
        }
        if (wave == 3) {
            const float gam = wave_inclusive_scan(rg);
            const float glast = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gam), 63));
            sGam[lane] = gam;
            sEg[lane] = __expf(gam);
            sDend[lane] = __expf(glast - gam);
        }
        lds_barrier();
        if (ch + 1 < nchunks) fetch(ch + 1);   // in flight during this chunk

        auto rows4 = [&](const float *vv, int i0, int qq) {
            return *reinterpret_cast<const f32x4 *>(vv + i0 + 8 * qq + 4 * lh);
        };

        // ---------------- prep: -W, U, P, Q S^T (no dependence on the state but Q S^T) ----
        f32x16 accD = {}, accOi = {};
        {
            // W^T tile: d_k rows 32 ct.., tokens 32 rt..; T_w is lower triangular,
            // so token tile 0 needs tokens 0..31 only
            const int rt = wave >> 2, ct = wave & 3;
            f32x16 acc = {};
            acc = rt == 0 ? mma32s<2, true, false>(acc, sKt, LD_T, 32 * ct, sTw, LD_T, 0, lane)
                          : mma32s<4, true, false>(acc, sKt, LD_T, 32 * ct, sTw, LD_T, 32, lane);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                bf16x4 x;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) x[s2] = (bf16)(-acc[4 * qq + s2]);
                *reinterpret_cast<bf16x4 *>(sWn + (32 * rt + l32) * LD_QK + 32 * ct + 8 * qq + 4 * lh) = x;
            }
        }
        if (wave == 0) {
            accD = mma32s<2, false, true>(accD, sTu, LD_T, 0, sVt, LD_T, 0, lane);
        } else if (wave == 1) {
            accD = mma32s<4, false, true>(accD, sTu, LD_T, 32, sVt, LD_T, 0, lane);
        } else if (wave == 2 || wave == 3 || wave == 5) {
            // P^T tile: rows j (keys) of tile tj, columns i (queries) of tile ti
            const int ti = wave == 2 ? 0 : 1, tj = wave == 5 ? 1 : 0;
            const int i = 32 * ti + l32;
            const float gi = sGam[i];
            f32x4 gj[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) gj[qq] = rows4(sGam, 32 * tj, qq);
            f32x16 acc = {};
            acc = mma32_2<4>(acc, sK, LD_QK, 32 * tj, sQ, LD_QK, 32 * ti, lane);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                bf16x4 x;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                    const int j = 32 * tj + 8 * qq + 4 * lh + s2;
                    x[s2] = (bf16)(j <= i ? acc[4 * qq + s2] * __expf(gi - gj[qq][s2]) : 0.f);
                }
                *reinterpret_cast<bf16x4 *>(sP + i * LD_T + 32 * tj + 8 * qq + 4 * lh) = x;
            }
        } else if (wave >= 6) {
            // (Q S^T)^T tile: rows c (this d_v tile), columns tokens 32 (wave - 6)..
            accOi = mma32_2<4>(accOi, sS, LD_S, 0, sQ, LD_QK, 32 * (wave - 6), lane);
        }
        lds_barrier();

        // ---------------- delta: Delta = U - W S^T (waves 0, 1; tokens 32 w ..) ----------
        if (wave < 2) {
            const int i0 = 32 * wave;
            f32x4 de4[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) de4[qq] = rows4(sDend, i0, qq);
            accD = mma32_2<4>(accD, sWn, LD_QK, i0, sS, LD_S, 0, lane);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const f32x4 de = de4[qq];
                bf16x4 dv, dw;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                    const float d = accD[4 * qq + s2];
                    dv[s2] = (bf16)d;
                    dw[s2] = (bf16)(d * de[s2]);
                }
                const int i = i0 + 8 * qq + 4 * lh;
                *reinterpret_cast<bf16x4 *>(sDt + l32 * LD_T + i) = dv;
                *reinterpret_cast<bf16x4 *>(sDtw + l32 * LD_T + i) = dw;
            }
        }
        lds_barrier();

        // ---------------- out: O^T and the state update ----------------
        if (wave >= 6) {
            const int rt = wave - 6, tok = 32 * rt + l32;
            const float eg = sEg[tok];
#pragma unroll
            for (int r = 0; r < 16; ++r) accOi[r] *= eg;
            accOi = rt == 0 ? mma32s<2, false, false>(accOi, sDt, LD_T, 0, sP, LD_T, 0, lane)
                            : mma32s<4, false, false>(accOi, sDt, LD_T, 0, sP, LD_T, 32, lane);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                bf16x4 x;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) x[s2] = (bf16)(scale * accOi[4 * qq + s2]);
                *reinterpret_cast<bf16x4 *>(sO + tok * LD_O + 8 * qq + 4 * lh) = x;
            }
        } else if (wave < 4) {
            const float eend = sEg[C - 1];
#pragma unroll
            for (int r = 0; r < 16; ++r) accS[r] *= eend;
            accS = mma32s<4, true, false>(accS, sKt, LD_T, 32 * wave, sDtw, LD_T, 0, lane);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                bf16x4 x;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) x[s2] = (bf16)accS[4 * qq + s2];
                *reinterpret_cast<bf16x4 *>(sS + l32 * LD_S + 32 * wave + 8 * qq + 4 * lh) = x;
            }
        }
        lds_barrier();
    }
    // the last chunk's output rows
    if (nchunks > 0 && tid0 < 256) {
        const int row = tid0 >> 2, col = 8 * (tid0 & 3);
        const int base = (nchunks - 1) * C;
        if (base + row < len)
            *reinterpret_cast<bf16x8 *>(o + ((size_t)bos + base + row) * H * DV + (size_t)h * DV + cbase + col) =
                *reinterpret_cast<const bf16x8 *>(sO + row * LD_O + col);
    }

    if (s_final && wave < 4) {
        const int lane = tid0 & 63;
        float *dst = s_final + sbase + (size_t)(cbase + (lane & 31)) * DK + 32 * wave + 4 * (lane >> 5);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
            *reinterpret_cast<f32x4 *>(dst + 8 * qq) =
                f32x4{accS[4 * qq], accS[4 * qq + 1], accS[4 * qq + 2], accS[4 * qq + 3]};
    }
}

// Workspace bytes of the two-pass path for `tokens` packed tokens in N
// sequences of H heads.
size_t prefill_split_workspace_bytes(long tokens, int H, int N) {
    const long nslots = tokens / C + N + 1;
    return (size_t)nslots * H * TWU_ELEMS * sizeof(bf16);
}

hipError_t launch_prefill_prepare(const void *k, const float *g, const float *beta,
                                  const int32_t *cu, int T, int H, int N, void *ws,
                                  hipStream_t stream)
{
    const long tokens = cu ? (long)T : (long)N * T;
    const long nslots = tokens / C + N + 1;
    if (tokens == 0) return hipSuccess;        // no chunk: nothing to prepare
    dim3 grid((unsigned)nslots, (unsigned)H), block(P_NT);
    hipLaunchKernelGGL(chunk_prep_kernel, grid, block, P_LDS_BYTES, stream, (const bf16 *)k, g,
                       beta, cu, (bf16 *)ws, T, H, N, (int)nslots);
    return hipGetLastError();
}

hipError_t launch_prefill_apply(const void *q, const void *k, const void *v, const float *g,
                                const float *s_init, float *s_final, void *o, const int32_t *cu,
                                int T, int H, int N, float scale, const void *ws,
                                hipStream_t stream)
{
    static bool attr_done = false;
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute((const void *)chunk_chain_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_done = true;
    }
    const long tokens = cu ? (long)T : (long)N * T;
    const long nslots = tokens / C + N + 1;
    dim3 grid((unsigned)((DV / DVT) * H * N)), block(NT);
    hipLaunchKernelGGL(chunk_chain_kernel, grid, block, LDS_BYTES, stream, (const bf16 *)q,
                       (const bf16 *)k, (const bf16 *)v, g, (const bf16 *)ws, s_init, s_final,
                       (bf16 *)o, cu, T, H, (int)nslots, scale);
    return hipGetLastError();
}

}  // namespace gdn
