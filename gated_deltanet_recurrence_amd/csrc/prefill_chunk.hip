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
// q and k may have fewer heads (H_k) than v, g, beta, o and the state (H):
// value head h reads query/key head h / (H / H_k) (the repeat_interleave head
// expansion of the "Gated DeltaNet body" layer code in the same chapter).
//
// Work mapping: one workgroup of 8 waves (two per SIMD) per (32-wide d_v
// tile, head, sequence); the columns of S (rows of our d_v x d_k state)
// evolve independently, so the four d_v tiles of a head never communicate.
// Waves 0-3 keep the state tile (32 x 128 fp32) in MFMA accumulators for the
// whole sequence, 32 x 32 each; a bf16 copy in LDS is the operand of the next
// chunk. The next chunk's q, k, v are loaded into registers while the current
// one is computed. Inside a chunk (one LDS barrier between phases):
//   load   Q, K row-major and K^T, V^T (token-contiguous, column-swizzled)
//          into LDS; gamma = inclusive prefix sum of g (wave 3, DPP scan)
//   G      waves 0-3: a 32 x 32 tile of A = -strict_lower(diag(beta) K K^T *
//          Gamma) and the inverse of one 16 x 16 diagonal block of I - A by
//          forward substitution (lane 4j + p owns column j and the terms
//          m = p mod 4; DPP quad sums); wave 4: the off-diagonal 32 x 32 tile
//          of A; waves 5-7: tiles of P = lower_incl_diag(Q K^T * Gamma)
//   L1/L2  the off-diagonal blocks of T = (I - A)^-1 by two levels of 2 x 2
//          block inversion, (L^-1)_21 = L22^-1 A21 L11^-1, on fp32 MFMA with
//          intermediate right factors kept in registers; meanwhile waves 6-7
//          form the inter-chunk output term Q S^T. Each finished block of T
//          is also written as bf16 T diag(beta e^gamma) and T diag(beta).
//   WU     W = T diag(beta e^gamma) K (one 32 x 32 tile per wave) -> LDS as -W;
//          U = T diag(beta) V (waves 0-1, kept in registers)
//   C1     Delta = U - W S^T (waves 0-1, two split-K accumulators)
//   C2     O = scale (e^gamma * Q S^T + P Delta) (waves 6-7);
//          S <- e^{gamma_63} S + Delta~^T K (waves 0-3)
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
// Matrix cores: v_mfma_f32_32x32x16_bf16 for every bf16 product (its operand
// reads, 32 consecutive LDS rows per half-wave, are free of bank conflicts
// with the row paddings used here) and v_mfma_f32_16x16x4f32 for the solve.
// Lane l of the 32x32x16 form holds A[l%32][8(l/32)+e] and B[8(l/32)+e][l%32]
// (e = 0..7); accumulator element r is C[8(r/4) + 4(l/32) + r%4][l%32].
#include "chunk_common.h"
#include "launch.h"

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
static_assert(DV / DVT == PAIR_TILES, "one workgroup per d_v tile of a pair");
static_assert(C * LD_QK * 2 <= SZ_A, "-W fits in the A region");
static_assert(4 * 4 * 4 * 68 * 4 <= SZ_Y, "solve scratch fits");
static_assert(2 * DVT * LD_T * 2 + C * LD_O * 2 <= SZ_Y, "chain buffers fit");

// per-token scalar slots in the SC region
enum { SC_GAM = 0, SC_BETA, SC_BEG, SC_EG, SC_DEND };

}  // namespace chunk

using namespace chunk;

__global__ void __launch_bounds__(NT, 1)
prefill_chunk_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                     const bf16 *__restrict__ v, const float *__restrict__ g,
                     const float *__restrict__ beta, const float *s_init, float *s_final,
                     bf16 *__restrict__ o, const int32_t *__restrict__ cu_seqlens, int T, int H,
                     int Hk, int npairs, float scale)
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
    int pair, tile;                            // (sequence, head) pair and d_v tile
    if (!pair_tile((int)blockIdx.x, npairs, pair, tile)) return;   // uniform
    const int h = pair % H, n = pair / H;
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

    // ---- state tile: waves 0-3 own S[c][d], c = 0..31 (this d_v tile), d in
    //      [32w, 32w + 32), as one 32x32 accumulator ---------------------------------
    f32x16 accS = {};
    const size_t sbase = ((size_t)n * H + h) * DV * DK;
    if (wave < 4) {
        const int lane = tid0 & 63;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int c = acc_row(r, lane), d = 32 * wave + (lane & 31);
            accS[r] = s_init ? s_init[sbase + (size_t)(cbase + c) * DK + d] : 0.0f;
        }
    }

    // ---- one-time LDS initialisation: the blocks above the diagonal of P, T_w
    //      and T_u are never written again; the bf16 copy of the state ---------
    for (int e = tid0; e < C * LD_T; e += NT) {
        sP[e] = (bf16)0.0f;
        sTw[e] = (bf16)0.0f;
        sTu[e] = (bf16)0.0f;
    }
    if (wave < 4) {
        const int lane = tid0 & 63;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            sS[acc_row(r, lane) * LD_S + 32 * wave + (lane & 31)] = (bf16)accS[r];
    }

    // ---- register prefetch of one chunk ---------------------------------------
    // Q: 2 x 16 B per thread (token row id/16, 8 columns). One 8 x 8 block (8
    // tokens x 8 channels) per thread of threads 0..159: K for 0..127 (token
    // block jb, d_k block cb), V for 128..159 (token block jb, d_v block cb of
    // this tile). g, beta: wave 3, one token per lane.
    const int tid = tid0;
    const int tstride = H * DK;                // elements between tokens of v
    const int tsqk = Hk * DK;                  // ... and of q, k (H_k <= H heads)
    const int kh = h / (H / Hk);               // query/key head of value head h
    const bool blk_k = tid < 128, blk_v = tid >= 128 && tid < 160;
    const int blk_jb = blk_k ? (tid >> 4) : ((tid - 128) >> 2);
    const int blk_cb = blk_k ? (tid & 15) : ((tid - 128) & 3);
    const int qrow0 = tid >> 4;                // rows qrow0 and qrow0 + 32
    // uniform bases; per-lane offsets fit in 32 bits (row < 64, H * 128 < 2^23)
    const bf16 *qbase = q + (size_t)bos * tsqk + (size_t)kh * DK;
    const bf16 *kbase = k + (size_t)bos * tsqk + (size_t)kh * DK;
    const bf16 *vbase = v + (size_t)bos * tstride + (size_t)h * DV + cbase;
    const int bstride = blk_k ? tsqk : tstride;   // K or V rows of this thread's block
    const int qoff = qrow0 * tsqk + 8 * (tid & 15);
    const int boff = 8 * blk_jb * bstride + 8 * blk_cb;
    bf16x8 rq[2], rb[8];
    float rg = 0.f, rbeta = 0.f;
    auto fetch = [&](int ch) {
        const bf16x8 z8 = {};
        const size_t coff = (size_t)ch * C * tstride, coffqk = (size_t)ch * C * tsqk;   // uniform
        const int base = ch * C;
        const int lane = tid & 63;
        const bf16 *qc = qbase + coffqk, *kc = kbase + coffqk, *vc = vbase + coff;
        if (base + C <= len) {                 // whole chunk inside the sequence (uniform)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                rq[u] = *reinterpret_cast<const bf16x8 *>(qc + qoff + 32 * u * tsqk);
            if (blk_k) {
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    rb[r] = *reinterpret_cast<const bf16x8 *>(kc + boff + r * tsqk);
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
                    rq[u] = *reinterpret_cast<const bf16x8 *>(qc + qoff + 32 * u * tsqk);
            }
            if (blk_k || blk_v) {
                const bf16 *bc = blk_k ? kc : vc;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    rb[r] = z8;
                    if (base + 8 * blk_jb + r < len)
                        rb[r] = *reinterpret_cast<const bf16x8 *>(bc + boff + r * bstride);
                }
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
        int tidl = tid0;
        asm volatile("" : "+v"(tidl));
        const int lane = tidl & 63, lr = lane & 15, lq = lane >> 4;
        const int l32 = lane & 31, lh = lane >> 5;   // 32x32x16 lane coordinates

        // ---------------- load: registers -> LDS; decay prefix sums ----------------
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

        // per-row scalars of accumulator elements r = 4q'..4q'+3 of a 32x32 tile
        // whose first row is i0: rows i0 + 8q' + 4*lh + 0..3
        auto rows4 = [&](const float *v, int i0, int qq) {
            return *reinterpret_cast<const f32x4 *>(v + i0 + 8 * qq + 4 * lh);
        };
        // one 32x32 tile of A = -strict_lower(diag(beta) K K^T * Gamma)
        auto gram32 = [&](int ti, int tj) {
            const int j = 32 * tj + l32;
            const float gj = sGam[j];
            f32x4 gi[4], bi[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                gi[qq] = rows4(sGam, 32 * ti, qq);
                bi[qq] = rows4(sBeta, 32 * ti, qq);
            }
            f32x16 acc = {};
            acc = mma32_2<4>(acc, sK, LD_QK, 32 * ti, sK, LD_QK, 32 * tj, lane);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                    const int r = 4 * qq + s2, i = 32 * ti + acc_row(r, lane);
                    acc[r] = j < i ? -bi[qq][s2] * acc[r] * __expf(gi[qq][s2] - gj) : 0.f;
                }
            }
            return acc;
        };
        // one 32x32 tile of P = lower_incl_diag(Q K^T * Gamma) -> sP
        auto p32 = [&](int ti, int tj) {
            const int j = 32 * tj + l32;
            const float gj = sGam[j];
            f32x4 gi[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) gi[qq] = rows4(sGam, 32 * ti, qq);
            f32x16 acc = {};
            acc = mma32_2<4>(acc, sQ, LD_QK, 32 * ti, sK, LD_QK, 32 * tj, lane);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                    const int r = 4 * qq + s2, i = 32 * ti + acc_row(r, lane);
                    sP[i * LD_T + j] = (bf16)(j <= i ? acc[r] * __expf(gi[qq][s2] - gj) : 0.f);
                }
            }
        };
        // store a finished 16x16 fp32 block of T, and its bf16 T diag(beta e^gamma),
        // T diag(beta) images (16x16x4 accumulator layout)
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

        // ---------------- G: A tiles, diagonal blocks of T, P -----------------------
        if (wave < 4) {
            // wave w = 2 tt + bt: tile (tt, tt) of A; invert its diagonal block bt
            // (global diagonal block w) by forward substitution,
            // D[i][j] = [i == j] + sum_{m<i} A_ww[i][m] D[m][j]
            const int tt = wave >> 1, bt = wave & 1;
            const f32x16 at = gram32(tt, tt);
            // whole 32x32 tile, unconditionally: into this wave's private copy laid
            // out [16x16 block][p][i][t] (element (i, m) of a block at
            // p = m % 4, t = m / 4; p stride 68 floats), and, by the even waves,
            // into sA (only its lower off-diagonal block is read later)
            float *ap = sY + wave * (4 * 4 * 68);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int it = acc_row(r, lane), jt = l32;
                const int blk = 2 * (it >> 4) + (jt >> 4), i = it & 15, m = jt & 15;
                ap[blk * (4 * 68) + (m & 3) * 68 + i * 4 + (m >> 2)] = at[r];
            }
            if (bt == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sA[(32 * tt + acc_row(r, lane)) * LD_A + 32 * tt + l32] = at[r];
            }
            wave_lds_order();
            // lane 4 jc + p owns column jc and the terms m = p (mod 4)
            const int jc = lane >> 2, p = lane & 3;
            const float *myp = ap + (3 * bt) * (4 * 68) + p * 68;   // diagonal block bt
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
            const int jj = 16 * wave + jc;
            const float bw = sBeg[jj], bu = sBeta[jj];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int ii = 16 * wave + p + 4 * t;
                sT[ii * LD_A + jj] = xs[t];
                sTw[ii * LD_T + jj] = (bf16)(xs[t] * bw);
                sTu[ii * LD_T + jj] = (bf16)(xs[t] * bu);
            }
        } else if (wave == 4) {
            // the off-diagonal 32x32 tile of A (rows 32..63, columns 0..31)
            const f32x16 at = gram32(1, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) sA[(32 + acc_row(r, lane)) * LD_A + l32] = at[r];
        } else {
            p32(wave == 5 ? 0 : 1, wave == 7 ? 1 : 0);   // tiles (0,0), (1,0), (1,1)
        }
        lds_barrier();

        // ---- off-diagonal blocks of T. With D_b the diagonal inverses:
        //   T10 = D1 A10 D0,  T32 = D3 A32 D2                      (16-level)
        //   Y = [A20 A21; A30 A31] [D0 0; T10 D1] = [Y00 P21; Y10 P31]
        //   [T20 T21; T30 T31] = [D2 0; T32 D3] Y                  (32-level)
        // Right factors produced by a wave stay in its registers (acc_to_bop).
        // Waves 6-7 form the inter-chunk output term Q S^T meanwhile.
        f32x16 accOi = {};
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
            } else {
                accOi = mma32_2<4>(accOi, sQ, LD_QK, 32 * (wave - 6), sS, LD_S, 0, lane);
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
            }
            lds_barrier();
        }

        // ---------------- WU: W = T_w K -> sWn = -W ; U = T_u V (waves 0, 1) ---------
        f32x16 accD = {};
        {
            // wave w: W rows 32 (w/4) .., d_k columns 32 (w%4) ..; T_w is lower
            // triangular, so row tile 0 needs tokens 0..31 only
            const int rt = wave >> 2, ct = wave & 3;
            f32x16 acc = {};
            acc = rt == 0 ? mma32<2, true>(acc, sTw, LD_T, 0, sKt, LD_T, 32 * ct, lane)
                          : mma32<4, true>(acc, sTw, LD_T, 32, sKt, LD_T, 32 * ct, lane);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sWn[(32 * rt + acc_row(r, lane)) * LD_QK + 32 * ct + l32] = (bf16)(-acc[r]);
            if (wave == 0) accD = mma32<2, true>(accD, sTu, LD_T, 0, sVt, LD_T, 0, lane);
            if (wave == 1) accD = mma32<4, true>(accD, sTu, LD_T, 32, sVt, LD_T, 0, lane);
        }
        lds_barrier();

        // ---------------- C1: Delta = U - W S^T (waves 0, 1; rows 32 w ..) ----------
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

        // ---------------- C2: O = scale (e^g Q S^T + P Delta); state update -----------
        if (wave >= 6) {
            const int rt = wave - 6, i0 = 32 * rt;
            f32x4 eg4[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) eg4[qq] = rows4(sEg, i0, qq);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) accOi[4 * qq + s2] *= eg4[qq][s2];
            accOi = rt == 0 ? mma32<2>(accOi, sP, LD_T, 0, sDt, LD_T, 0, lane)
                            : mma32<4>(accOi, sP, LD_T, 32, sDt, LD_T, 0, lane);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sO[(i0 + acc_row(r, lane)) * LD_O + l32] = (bf16)(scale * accOi[r]);
        } else if (wave < 4) {
            const float eend = sEg[C - 1];
#pragma unroll
            for (int r = 0; r < 16; ++r) accS[r] *= eend;
            accS = mma32<4, true>(accS, sDtw, LD_T, 0, sKt, LD_T, 32 * wave, lane);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sS[acc_row(r, lane) * LD_S + 32 * wave + l32] = (bf16)accS[r];
        }
        lds_barrier();
        // output tile 64 x 32 bf16: one 16-byte store per thread of the first 256
        if (tidl < 256) {
            const int row = tidl >> 2, col = 8 * (tidl & 3);
            if (base + row < len)
                *reinterpret_cast<bf16x8 *>(o + ((size_t)bos + base + row) * H * DV + (size_t)h * DV + cbase + col) =
                    *reinterpret_cast<const bf16x8 *>(sO + row * LD_O + col);
        }
    }

    if (s_final && wave < 4) {
        const int lane = tid0 & 63;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int c = acc_row(r, lane), d = 32 * wave + (lane & 31);
            s_final[sbase + (size_t)(cbase + c) * DK + d] = accS[r];
        }
    }
}

hipError_t launch_prefill_chunk(const void *q, const void *k, const void *v, const float *g,
                                const float *beta, const float *s_init, float *s_final, void *o,
                                const int32_t *cu, int T, int H, int Hk, int N, float scale,
                                hipStream_t stream)
{
    // the dynamic LDS limit, raised once per process (thread-safe static)
    static const hipError_t attr = hipFuncSetAttribute(
        (const void *)prefill_chunk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (attr != hipSuccess) return attr;
    const int npairs = H * N;
    dim3 grid(pair_grid(npairs)), block(NT);
    hipLaunchKernelGGL(prefill_chunk_kernel, grid, block, LDS_BYTES, stream, (const bf16 *)q,
                       (const bf16 *)k, (const bf16 *)v, g, beta, s_init, s_final, (bf16 *)o, cu,
                       T, H, Hk, npairs, scale);
    return hipGetLastError();
}

}  // namespace gdn
