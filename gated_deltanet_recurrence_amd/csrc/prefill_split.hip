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
// ((h * nslots) + s) * 6144: -T_w then T_u, each as the three non-zero 32 x 32
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
// sequence). Row strides are chosen for the v_mfma_f32_16x16x32_bf16 operand
// reads (16 consecutive rows, four 16-byte column chunks): with a stride of
// 32 bytes modulo 128 they hit every LDS bank equally.
// ---------------------------------------------------------------------------
constexpr int DVT = 32;
constexpr int NT = 512;
constexpr int LD_R = DK + 16;                  // rows of 128 bf16 (288 B): Q, K, S
constexpr int LD_64 = C + 16;                  // rows of 64 bf16 (160 B): T_w, T_u, P, Delta^T
constexpr int LD_V = DVT + 8;                  // V rows (32 bf16 of this tile)
constexpr int LD_O = DVT + 8;                  // output staging rows
constexpr int SZ_R = C * LD_R * 2;             // 18432
constexpr int SZ_V = C * LD_V * 2;             // 5120
constexpr int SZ_64 = C * LD_64 * 2;           // 10240
constexpr int SZ_S = DVT * LD_R * 2;           // 9216
constexpr int SZ_DT = DVT * LD_64 * 2;         // 5120
constexpr int SZ_O = C * LD_O * 2;             // 5120
constexpr int SZ_SC = 3 * C * 4;               // gamma, e^gamma, e^{gamma_63 - gamma}
constexpr int OFF_Q = 0;
constexpr int OFF_K = OFF_Q + SZ_R;
constexpr int OFF_V = OFF_K + SZ_R;
constexpr int OFF_TW = OFF_V + SZ_V;
constexpr int OFF_TU = OFF_TW + SZ_64;
constexpr int OFF_P = OFF_TU + SZ_64;
constexpr int OFF_S = OFF_P + SZ_64;           // two buffers
constexpr int OFF_DT = OFF_S + 2 * SZ_S;
constexpr int OFF_O = OFF_DT + SZ_DT;
constexpr int OFF_SC = OFF_O + SZ_O;
constexpr int LDS_BYTES = OFF_SC + SZ_SC;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16 x 8 operand slice of a row-major bf16 LDS matrix for
// v_mfma_f32_16x16x32_bf16: row r0 + lane%16, columns k0 + 8 (lane/16) .. +8
__device__ __forceinline__ bf16x8 frag16(const bf16 *m, int ld, int r0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8 *>(m + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}
// The same slice of a matrix stored with its 16-byte column chunks swizzled
// by row: chunk c of row r sits at c ^ ((r / 4) % 4). Accumulator tiles are
// written into such matrices 8 bytes per lane (row lane%16, columns 4 (lane/16)
// ..), which without the swizzle would hit the same LDS banks 3x over; the
// swizzle leaves these 16-byte reads conflict-free. r0 must be a multiple of 16.
__device__ __forceinline__ int swz(int lane) { return ((lane & 15) >> 2) << 3; }
__device__ __forceinline__ bf16x8 frag16_sw(const bf16 *m, int ld, int r0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8 *>(m + (r0 + (lane & 15)) * ld + ((k0 + 8 * (lane >> 4)) ^ swz(lane)));
}
// The same slice with the columns in the row order of a 16x16 accumulator
// pair: k0 + 4 (lane/16) + {0..3} and k0 + 16 + 4 (lane/16) + {0..3}. A
// product whose other operand is taken from accumulators (rows 4 (lane/16) +
// r of two consecutive 16-row tiles) contracts over that order.
__device__ __forceinline__ bf16x8 frag16_acc(const bf16 *m, int ld, int r0, int k0, int lane) {
    const bf16 *p = m + (r0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
    const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(p);
    const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(p + 16);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane L
// names row k0 + L/4, columns c0 + 4 (L%4) .. +4 of a row-major matrix M, and
// lane m receives M[k0 .. k0 + 3][c0 + m]. k0 may differ between groups.
__device__ __forceinline__ bf16x4 tr4(const bf16 *m, int ld, int k0, int c0, int lane) {
    const int L = lane & 15;
    const bf16 *p = m + (k0 + (L >> 2)) * ld + c0 + 4 * (L & 3);
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p));
}
// Same with the four column groups at c0 + cstep (L%4): lane m receives
// M[k0 .. k0 + 3][c0 + cstep (m/4) + m%4].
__device__ __forceinline__ bf16x4 tr4s(const bf16 *m, int ld, int k0, int c0, int cstep, int lane) {
    const int L = lane & 15;
    const bf16 *p = m + (k0 + (L >> 2)) * ld + c0 + cstep * (L & 3);
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p));
}
// 16 x 8 operand slice whose row is chosen per lane (columns k0 + 8 (lane/16) ..)
__device__ __forceinline__ bf16x8 frag16_row(const bf16 *m, int ld, int row, int k0, int lane) {
    return *reinterpret_cast<const bf16x8 *>(m + row * ld + k0 + 8 * (lane >> 4));
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
//   store  -T diag(beta e^gamma) and T diag(beta), bf16, to the workspace
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
        const float sgn = mat ? 1.f : -1.f;    // T_w is stored negated
        const f32x4 t0 = *reinterpret_cast<const f32x4 *>(sT + i * P_LD_A + j0);
        const f32x4 t1 = *reinterpret_cast<const f32x4 *>(sT + i * P_LD_A + j0 + 4);
        const f32x4 s0 = *reinterpret_cast<const f32x4 *>(sc + j0);
        const f32x4 s1 = *reinterpret_cast<const f32x4 *>(sc + j0 + 4);
        // the 16 x 16 blocks above the diagonal of T are zero (not stored in sT)
        const bool zero = (j0 >> 4) > (i >> 4);
        bf16x8 out;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            out[e2] = (bf16)(zero ? 0.f : sgn * t0[e2] * s0[e2]);
            out[e2 + 4] = (bf16)(zero ? 0.f : sgn * t1[e2] * s1[e2]);
        }
        *reinterpret_cast<bf16x8 *>(dst + 8 * e) = out;
    }
}

// ---------------------------------------------------------------------------
// chunk_chain: the sequential pass. One workgroup of 8 waves per (32-wide d_v
// tile, head, sequence), two LDS barriers per chunk.
//
// Waves 0 and 1 carry the recurrence, each for 16 of the tile's d_v columns:
// the wave keeps its slice of S^T (128 x 16, fp32) in eight 16x16 MFMA
// accumulators for the whole sequence, and per chunk computes
//   X     = K S^T                       (B operand: the state accumulators)
//   Delta = T_u V - T_w X               (B operand: X's accumulators)
//   S^T  <- e^{gamma_63} S^T + K^T Delta~,  Delta~_j = e^{gamma_63 - gamma_j} Delta_j
//                                       (B operand: Delta~'s accumulators)
// entirely in registers: an accumulator pair holds rows 4 (lane/16) + r of
// two consecutive 16-row tiles, which is a B operand over that row order, and
// the matching A operand is read from LDS in the same order (frag16_acc) or
// transposed on the fly (tr4). Grouping T_w K S^T as T_w (K S^T) means W =
// T_w K is never formed.
// Waves 2 and 3 form the output, O^T = (S Q^T) diag(e^gamma) + Delta^T P^T,
// for the same column halves; waves 6 and 7 form
// P = lower_incl_diag(Q K^T * Gamma) (as P^T tiles, stored row-major);
// waves 4 and 5 copy the previous chunk's output rows to HBM.
//
//   phase A  waves 0-1: the recurrence step of chunk c (Delta^T and the new
//            S as bf16 into LDS); waves 2-3: S Q^T; waves 6-7: P
//   phase B  waves 2-3: + Delta^T P^T -> output staging; the other waves store
//            chunk c+1 (loaded into registers one chunk earlier) into LDS and
//            issue the loads of chunk c+2
//
// Tokens past the end of a sequence are identity steps (q = k = v = 0,
// g = 0, and T_w, T_u vanish on them) and their outputs are not stored.
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
    bf16 *sV = reinterpret_cast<bf16 *>(smem + OFF_V);
    bf16 *sTw = reinterpret_cast<bf16 *>(smem + OFF_TW);     // -T_w
    bf16 *sTu = reinterpret_cast<bf16 *>(smem + OFF_TU);
    bf16 *sP = reinterpret_cast<bf16 *>(smem + OFF_P);
    bf16 *sS = reinterpret_cast<bf16 *>(smem + OFF_S);       // [2][DVT][LD_R]
    bf16 *sDt = reinterpret_cast<bf16 *>(smem + OFF_DT);
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
    const size_t sbase = ((size_t)n * H + h) * DV * DK;

    // ---- state: wave hv < 2 holds Sacc[d][r] = S[cbase + 16 hv + lane%16][dk(d, lane/16, r)]
    //      with dk(d, q, r) = 32 (d/2) + 8 q + 4 (d%2) + r: accumulator pair (2s, 2s+1)
    //      then covers d_k 32 s + 8 q + 0..7 contiguously (see the state update)
    f32x4 Sacc[8];
    bf16x8 Sb[4];                           // the same as four bf16 B operands (32 d_k each)
#pragma unroll
    for (int d = 0; d < 8; ++d) Sacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (wave < 2) {
        const int lane = tid0 & 63, m = lane & 15, qq = lane >> 4;
        const int col = cbase + 16 * wave + m;
        if (s_init) {
#pragma unroll
            for (int d = 0; d < 8; ++d)
                Sacc[d] = *reinterpret_cast<const f32x4 *>(s_init + sbase + (size_t)col * DK + 32 * (d >> 1) + 8 * qq + 4 * (d & 1));
        }
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) Sb[s2] = acc_pair_bf16(Sacc[2 * s2], Sacc[2 * s2 + 1]);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            bf16x4 x = {(bf16)Sacc[d][0], (bf16)Sacc[d][1], (bf16)Sacc[d][2], (bf16)Sacc[d][3]};
            *reinterpret_cast<bf16x4 *>(sS + (16 * wave + m) * LD_R + ((32 * (d >> 1) + 8 * qq + 4 * (d & 1)) ^ swz(lane))) = x;
        }
    }

    // ---- loads of one chunk into registers, by waves 2-7 (loader index
    //      lt = tid - 128 in [0, 384)); each issues eight 16-byte loads p + r * stride:
    //        lt in [0, 128)    Q rows row0 + 8 r, columns 8 (lt % 16) ..
    //        lt in [128, 256)  K rows, the same pattern
    //        lt in [256, 288)  V rows vrow0 + 8 r, 8 columns of this d_v tile
    //        lt in [288, 384)  pieces e0 + 96 r of -T_w | T_u
    //      and every loader loads g. Rows past the end of the sequence are read from
    //      its last token and zeroed when stored (straight-line loads: a
    //      data-dependent branch around them makes the compiler wait for them
    //      at the join). ----
    const int tid = tid0;
    const int tstride = H * DK;
    const bool loader = wave >= 2;
    const int lt = tid - 128;
    const int role = lt < 128 ? 0 : lt < 256 ? 1 : lt < 288 ? 2 : 3;
    const int qk = lt & 127;
    const int row0 = role <= 1 ? (qk >> 4) : ((lt - 256) >> 2);
    const int lcol = role <= 1 ? 8 * (qk & 15) : 8 * ((lt - 256) & 3);
    const int tt_e0 = lt - 288;
    const bf16 *qbase = q + (size_t)bos * tstride + (size_t)h * DK;
    const bf16 *kbase = k + (size_t)bos * tstride + (size_t)h * DK;
    const bf16 *vbase = v + (size_t)bos * tstride + (size_t)h * DV + cbase;
    bf16x8 rb[8];
    float rg = 0.f;
    bool rg_ok = true;
    unsigned rvalid = 0xFF;
    auto fetch = [&](int ch) {
        const int base = ch * C;
        const int lane = tid & 63;
        if (role == 3) {
            const bf16 *src = wsh + (size_t)ch * TWU_ELEMS + 8 * tt_e0;
#pragma unroll
            for (int r = 0; r < 8; ++r) rb[r] = *reinterpret_cast<const bf16x8 *>(src + r * 8 * 96);
            rvalid = 0xFF;
        } else {
            const bf16 *src = (role == 0 ? qbase : role == 1 ? kbase : vbase) + (size_t)base * tstride + lcol;
            rvalid = 0;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int t = row0 + 8 * r;
                const bool ok = base + t < len;
                rvalid |= (ok ? 1u : 0u) << r;
                rb[r] = *reinterpret_cast<const bf16x8 *>(src + (size_t)(ok ? t : len - 1 - base) * tstride);
            }
        }
        // every loader loads g (only wave 7 uses it): a load under a wave-dependent
        // branch would again make the compiler wait for it at the join
        rg_ok = base + lane < len;
        rg = g[((size_t)bos + base + (rg_ok ? lane : len - 1 - base)) * H + h];
    };
    auto store = [&]() {
        if (rvalid != 0xFF) {
            const bf16x8 z8 = {};
#pragma unroll
            for (int r = 0; r < 8; ++r) rb[r] = (rvalid >> r) & 1 ? rb[r] : z8;
        }
        if (role <= 1) {
            bf16 *dst = (role == 0 ? sQ : sK) + row0 * LD_R + lcol;
#pragma unroll
            for (int r = 0; r < 8; ++r) *reinterpret_cast<bf16x8 *>(dst + 8 * r * LD_R) = rb[r];
        } else if (role == 2) {
            bf16 *dst = sV + row0 * LD_V + lcol;
#pragma unroll
            for (int r = 0; r < 8; ++r) *reinterpret_cast<bf16x8 *>(dst + 8 * r * LD_V) = rb[r];
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int e = tt_e0 + 96 * r;          // 0..767
                const int mat = e >= 384 ? 1 : 0, rem = e - 384 * mat;
                const int blk = rem >> 7, row = (rem >> 2) & 31, cc = rem & 3;
                const int off = (32 * (blk > 0 ? 1 : 0) + row) * LD_64 + 32 * (blk == 2 ? 1 : 0) + 8 * cc;
                *reinterpret_cast<bf16x8 *>((mat ? sTu : sTw) + off) = rb[r];
            }
        }
        if (wave == 7) {
            const int lane = tid & 63;
            const float gam = wave_inclusive_scan(rg_ok ? rg : 0.f);
            const float glast = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gam), 63));
            sGam[lane] = gam;
            sEg[lane] = __expf(gam);
            sDend[lane] = __expf(glast - gam);
        }
    };
    // P's 16 x 16 tiles (0, 1) and (2, 3) lie above the diagonal but inside the
    // 32-key k-steps of the output product: zero once, never written again.
    // (The upper-right 32 x 32 blocks of T_w and T_u are never read.)
    for (int e = tid; e < C * LD_64 / 8; e += NT)
        reinterpret_cast<bf16x8 *>(sP)[e] = bf16x8{};
    if (nchunks > 0 && loader) {
        fetch(0);
        store();
        fetch(nchunks > 1 ? 1 : 0);
    }
    lds_barrier();

    // Each wave role runs its own loop with the same two barriers per chunk;
    // the loaders' register prefetch is then straight-line code (every
    // iteration loads, the last two re-read the last chunk), so the compiler
    // never waits for it at the loop back-edge.
    if (wave < 2) {
        // ============ waves 0-1: the recurrence ============
        // the sequential path: these waves win instruction arbitration on their SIMDs
        __builtin_amdgcn_s_setprio(3);
        const int hv = wave;
        for (int ch = 0; ch < nchunks; ++ch) {
            int tidl = tid0;
            asm volatile("" : "+v"(tidl));  // keep lane-derived addresses out of loop-invariant hoisting
            const int lane = tidl & 63, m = lane & 15, qq = lane >> 4;
            const int cur = ch & 1;
            // U = T_u V and X = K S^T
            f32x4 dacc[4], xacc[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) { dacc[t] = f32x4{0.f, 0.f, 0.f, 0.f}; xacc[t] = dacc[t]; }
            {
                // X tile t takes K rows 32 (t/2) + 8 (m/4) + 4 (t%2) + m%4, so that its
                // accumulator pairs run over tokens 32 s + 8 q + 0..7 contiguously
                bf16x8 fk[4][4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int row = 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3);
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) fk[t][s2] = frag16_row(sK, LD_R, row, 32 * s2, lane);
                }
                bf16x8 fv[2], fu[4][2];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    fv[s2] = cat4(tr4(sV, LD_V, 32 * s2 + 8 * qq, 16 * hv, lane),
                                  tr4(sV, LD_V, 32 * s2 + 8 * qq + 4, 16 * hv, lane));
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        if (s2 <= (t >> 1)) fu[t][s2] = frag16(sTu, LD_64, 16 * t, 32 * s2, lane);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
                    for (int t = 0; t < 4; ++t) xacc[t] = mfma16(fk[t][s2], Sb[s2], xacc[t]);
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        if (s2 <= (t >> 1)) dacc[t] = mfma16(fu[t][s2], fv[s2], dacc[t]);
            }
            // Delta = U + (-T_w) X
            {
                bf16x8 fw[4][2];
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        if (s2 <= (t >> 1)) fw[t][s2] = frag16(sTw, LD_64, 16 * t, 32 * s2, lane);
                const bf16x8 xb0 = acc_pair_bf16(xacc[0], xacc[1]);
                const bf16x8 xb1 = acc_pair_bf16(xacc[2], xacc[3]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    dacc[t] = mfma16(fw[t][0], xb0, dacc[t]);
                    if (t >= 2) dacc[t] = mfma16(fw[t][1], xb1, dacc[t]);
                }
            }
            // Delta^T -> LDS (output term); Delta~ as the B operand of the update
            bf16x8 db[2];
            {
                f32x4 dend[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    dend[t] = *reinterpret_cast<const f32x4 *>(sDend + 16 * t + 4 * qq);
                    bf16x4 x = {(bf16)dacc[t][0], (bf16)dacc[t][1], (bf16)dacc[t][2], (bf16)dacc[t][3]};
                    *reinterpret_cast<bf16x4 *>(sDt + (16 * hv + m) * LD_64 + ((16 * t + 4 * qq) ^ swz(lane))) = x;
                }
                db[0] = acc_pair_bf16(dacc[0] * dend[0], dacc[1] * dend[1]);
                db[1] = acc_pair_bf16(dacc[2] * dend[2], dacc[3] * dend[3]);
            }
            // S^T <- e^{gamma_63} S^T + K^T Delta~ (A operand: K transposed on read)
            {
                const float eend = sEg[C - 1];
                bf16x8 fkt[8][2];
#pragma unroll
                for (int d = 0; d < 8; ++d)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        fkt[d][s2] = cat4(tr4s(sK, LD_R, 32 * s2 + 4 * qq, 32 * (d >> 1) + 4 * (d & 1), 8, lane),
                                          tr4s(sK, LD_R, 32 * s2 + 16 + 4 * qq, 32 * (d >> 1) + 4 * (d & 1), 8, lane));
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int d = 0; d < 8; ++d) {
                    Sacc[d] = Sacc[d] * eend;
                    Sacc[d] = mfma16(fkt[d][0], db[0], Sacc[d]);
                    Sacc[d] = mfma16(fkt[d][1], db[1], Sacc[d]);
                }
            }
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) Sb[s2] = acc_pair_bf16(Sacc[2 * s2], Sacc[2 * s2 + 1]);
            bf16 *sSn = sS + (cur ^ 1) * DVT * LD_R;
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                bf16x4 x = {(bf16)Sacc[d][0], (bf16)Sacc[d][1], (bf16)Sacc[d][2], (bf16)Sacc[d][3]};
                *reinterpret_cast<bf16x4 *>(sSn + (16 * hv + m) * LD_R + ((32 * (d >> 1) + 8 * qq + 4 * (d & 1)) ^ swz(lane))) = x;
            }
            lds_barrier();
            lds_barrier();
        }
    } else if (wave < 4) {
        // ============ waves 2-3: the output for d_v rows 16 hv .. ============
        const int hv = wave - 2;
        f32x4 oacc[4];
        for (int ch = 0; ch < nchunks; ++ch) {
            int tidl = tid0;
            asm volatile("" : "+v"(tidl));
            const int lane = tidl & 63, m = lane & 15, qq = lane >> 4;
            const int cur = ch & 1;
            // (Q S^T)^T = S Q^T, all 64 tokens, then e^gamma per token
            {
                const bf16 *sSc = sS + cur * DVT * LD_R;
                bf16x8 fs[4], fq[4][4];
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                    fs[s2] = frag16_sw(sSc, LD_R, 16 * hv, 32 * s2, lane);
#pragma unroll
                    for (int t = 0; t < 4; ++t) fq[t][s2] = frag16(sQ, LD_R, 16 * t, 32 * s2, lane);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int t = 0; t < 4; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
                    for (int t = 0; t < 4; ++t) oacc[t] = mfma16(fs[s2], fq[t][s2], oacc[t]);
#pragma unroll
                for (int t = 0; t < 4; ++t) oacc[t] = oacc[t] * sEg[16 * t + m];
            }
            lds_barrier();
            // O^T += Delta^T P^T; token tile t needs keys 0 .. 16 t + 15
            {
                bf16x8 fd[2], fp[4][2];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    fd[s2] = frag16_sw(sDt, LD_64, 16 * hv, 32 * s2, lane);
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (s2 <= (t >> 1)) fp[t][s2] = frag16_sw(sP, LD_64, 16 * t, 32 * s2, lane);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        if (s2 <= (t >> 1)) oacc[t] = mfma16(fd[s2], fp[t][s2], oacc[t]);
                // oacc[t][r] = O[token 16 t + m][d_v 16 hv + 4 qq + r]
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    bf16x4 x = {(bf16)(scale * oacc[t][0]), (bf16)(scale * oacc[t][1]),
                                (bf16)(scale * oacc[t][2]), (bf16)(scale * oacc[t][3])};
                    *reinterpret_cast<bf16x4 *>(sO + (16 * t + m) * LD_O + 16 * hv + 4 * qq) = x;
                }
            }
            if (ch + 1 < nchunks) store();     // chunk ch + 1
            fetch(ch + 2 < nchunks ? ch + 2 : nchunks - 1);
            lds_barrier();
        }
    } else {
        // ============ waves 4-7: P (one query row each; wave 5 also moves the
        //              previous chunk's output rows to HBM), then loads ============
        // a chunk's output rows (64 x 32 bf16) from the staging buffer to HBM
        auto ostore = [&](int chp) {
            const int e = (int)threadIdx.x & 63;        // one wave: 256 16-byte pieces
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int piece = e + 64 * u, row = piece >> 2, col = 8 * (piece & 3);
                const int tok = chp * C + row;
                if (tok < len)
                    *reinterpret_cast<bf16x8 *>(o + ((size_t)bos + tok) * H * DV + (size_t)h * DV + cbase + col) =
                        *reinterpret_cast<const bf16x8 *>(sO + row * LD_O + col);
            }
        };
        for (int ch = 0; ch < nchunks; ++ch) {
            int tidl = tid0;
            asm volatile("" : "+v"(tidl));
            const int lane = tidl & 63, m = lane & 15, qq = lane >> 4;
            {
                // P^T tiles (keys 16 J.., queries 16 I..) for J <= I, one query row
                // I per wave: I = 3 (wave 6), 2 (wave 7), 1 (wave 4), 0 (wave 5);
                // the row's Q fragments are loaded once
                const int I = wave == 6 ? 3 : wave == 7 ? 2 : wave == 4 ? 1 : 0;
                bf16x8 fq[4];
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) fq[s2] = frag16(sQ, LD_R, 16 * I, 32 * s2, lane);
                const int i = 16 * I + m;
                const float gi = sGam[i];
                for (int J = 0; J <= I; ++J) {
                    bf16x8 fk[4];
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) fk[s2] = frag16(sK, LD_R, 16 * J, 32 * s2, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) acc = mfma16(fk[s2], fq[s2], acc);
                    // acc[r] = q_i . k_j with i = 16 I + m, j = 16 J + 4 qq + r
                    const int j0 = 16 * J + 4 * qq;
                    const f32x4 gj = *reinterpret_cast<const f32x4 *>(sGam + j0);
                    bf16x4 x;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        x[r] = (bf16)(j0 + r <= i ? acc[r] * __expf(gi - gj[r]) : 0.f);
                    *reinterpret_cast<bf16x4 *>(sP + i * LD_64 + (j0 ^ swz(lane))) = x;
                }
            }
            if (wave == 5 && ch > 0) {
                ostore(ch - 1);
            }
            lds_barrier();
            if (ch + 1 < nchunks) store();     // chunk ch + 1
            fetch(ch + 2 < nchunks ? ch + 2 : nchunks - 1);
            lds_barrier();
        }
        if (wave == 5 && nchunks > 0) ostore(nchunks - 1);  // the last chunk's output rows
    }
    if (s_final && wave < 2) {
        const int lane = tid0 & 63, m = lane & 15, qq = lane >> 4;
        float *dst = s_final + sbase + (size_t)(cbase + 16 * wave + m) * DK + 8 * qq;
#pragma unroll
        for (int d = 0; d < 8; ++d) *reinterpret_cast<f32x4 *>(dst + 32 * (d >> 1) + 4 * (d & 1)) = Sacc[d];
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
