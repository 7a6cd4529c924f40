// seqpar.hip - sequence-parallel chunked prefill: long sequences are cut
// into segments whose chains run side by side.
//
// "[LLM Algorithms-2] Gated DeltaNet: Teaching Linear Attention to Overwrite
// and Forget", section 7: a run of tokens acts on the state as one affine map,
// S_end = S_start A + B (A = the product of the tokens' alpha (I - beta k k^T),
// B = the decayed sum of their writes), so a sequence cut into segments can
// walk every segment at once and patch the start states afterwards.
//
// Plan (made on the device by seqpar_plan_kernel, where the offsets live):
// the longest sequence has M chunks of 64 tokens; a segment holds L =
// ceil(M / P) chunks, and sequence n is cut into P_n = max(1, ceil(M_n / L))
// segments of L chunks, its last one shorter. Then
//   pass 1  segment 0 of every sequence runs from the caller's initial state
//           and writes its outputs; its final state is the start state S_1 of
//           segment 1 (the sequence's final state when P_n = 1). Side by side,
//           every middle segment (0 < s < P_n - 1) runs twice: from a zero
//           state on its own values (final state B_s) and with v = 0 from the
//           identity (final state, d_v = d_k rows e_j A_s: A_s);
//   compose S_{s+1} = S_s A_s + B_s over the middle segments, in order;
//   pass 2  segments 1 .. P_n - 1 run from S_s and write their outputs; the
//           last one writes the sequence's final state.
// A sequence's last segment never needs its map, and a sequence of one or two
// segments needs none, so a batch whose short sequences stay whole pays the
// extra chain work only on its long ones. Each pass is one launch of the
// chain kernel driven by a job table (chunk_common.h SegJob); the per-chunk
// systems are solved once, over all segments. Critical path: two segments'
// chains instead of one sequence's; extra work: two chain walks of every
// middle segment and P_n - 2 dependent 128 x 128 x 128 products per head.
#include "chunk_common.h"
#include "launch.h"

namespace gdn {

using chunk::RANK_MAX;
constexpr int SP_D = 128;                      // d_k = d_v of the chunk kernels
constexpr size_t SP_MAT = (size_t)SP_D * SP_D; // floats per head state

// Bounds of sequence n as the chain kernels see them (seq_bounds there):
// packed offsets clamped into [0, T], a decreasing pair empty.
__device__ __forceinline__ void plan_bounds(const int32_t *cu, int n, int T, long &a, long &b)
{
    if (cu) {
        a = cu[n];
        b = cu[n + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        b = b < a ? a : (b > T ? T : b);
    } else {
        a = (long)n * T;
        b = a + T;
    }
}

// The plan, by one workgroup. Outputs (workspace):
//   cu_seg[nsmax + 1]  segment offsets along the packed token axis, sequences
//                      in order, each cut into its segments; the unused
//                      tail (segments past the total) empty at the end
//   job1[2 nsmax]      pass 1: [0, nsmax) segment 0 runs and the B runs,
//                      [nsmax, 2 nsmax) the A runs; inactive entries seg -1
//   job2[nsmax]        pass 2
//   seg_first[N], seg_count[N]   segment range of each sequence (compose)
// Jobs of sequence n occupy positions pos_n .. pos_n + P_n - 1 of each table,
// with sequences taken longest first (ties by index) when N <= RANK_MAX, so
// that the long chains start first; else in index order.
constexpr int PL_NT = 256;
static_assert(RANK_MAX <= PL_NT, "one thread per ranked sequence");
__global__ void __launch_bounds__(PL_NT)
seqpar_plan_kernel(const int32_t *cu, int T, int N, int P, int H, int nsmax,
                   const float *s_init, float *s_final, float *inits, float *Am, float *Bm,
                   int32_t *cu_seg, SegJob *job1, SegJob *job2, int32_t *seg_first,
                   int32_t *seg_count)
{
    __shared__ int s_max, s_carry;
    __shared__ int s_scan[PL_NT];
    __shared__ int s_cnt[RANK_MAX];            // segment count by rank, then job position
    const int tid = (int)threadIdx.x;
    auto chunks_of = [&](int n) {
        long a, b;
        plan_bounds(cu, n, T, a, b);
        return (int)((b - a + 63) >> 6);
    };
    if (tid == 0) { s_max = 0; s_carry = 0; }
    __syncthreads();
    int mx = 0;
    for (int n = tid; n < N; n += PL_NT) mx = max(mx, chunks_of(n));
    atomicMax(&s_max, mx);
    __syncthreads();
    const int L = max(1, (s_max + P - 1) / P);   // chunks per segment
    auto count_of = [&](int n) { return max(1, (chunks_of(n) + L - 1) / L); };

    // segment index of each sequence's first segment: exclusive scan of P_n
    for (int n0 = 0; n0 < N; n0 += PL_NT) {
        const int n = n0 + tid;
        const int x = n < N ? count_of(n) : 0;
        s_scan[tid] = x;
        __syncthreads();
        for (int d = 1; d < PL_NT; d <<= 1) {
            const int y = tid >= d ? s_scan[tid - d] : 0;
            __syncthreads();
            s_scan[tid] += y;
            __syncthreads();
        }
        if (n < N) {
            seg_first[n] = s_carry + s_scan[tid] - x;
            seg_count[n] = x;
        }
        __syncthreads();
        if (tid == PL_NT - 1) s_carry += s_scan[tid];
        __syncthreads();
    }
    const int total = s_carry;                 // <= N * P = nsmax

    // job position of each sequence's first job
    const bool ranked = N <= RANK_MAX;
    if (ranked) {
        if (tid < N) s_scan[tid] = chunks_of(tid);
        __syncthreads();
        int rank = 0, x = 0;
        if (tid < N) {
            const int c = s_scan[tid];
            for (int m = 0; m < N; ++m) {
                const int cm = s_scan[m];
                rank += (cm > c) | ((cm == c) & (m < tid));
            }
            x = max(1, (c + L - 1) / L);
        }
        __syncthreads();
        if (tid < N) s_cnt[rank] = x;
        __syncthreads();
        // exclusive scan over ranks (N <= RANK_MAX = PL_NT entries)
        const int xr = tid < N ? s_cnt[tid] : 0;
        s_scan[tid] = xr;
        __syncthreads();
        for (int d = 1; d < PL_NT; d <<= 1) {
            const int y = tid >= d ? s_scan[tid - d] : 0;
            __syncthreads();
            s_scan[tid] += y;
            __syncthreads();
        }
        if (tid < N) s_cnt[tid] = s_scan[tid] - xr;   // position of rank tid
        __syncthreads();
        if (tid < N) s_scan[tid] = s_cnt[rank];       // position of sequence tid
        __syncthreads();
    }

    const size_t hmat = (size_t)H * SP_MAT;
    for (int n = tid; n < N; n += PL_NT) {
        long a, b;
        plan_bounds(cu, n, T, a, b);
        const int j0 = seg_first[n], pn = seg_count[n];
        const int r0 = ranked ? s_scan[n] : j0;
        const float *sin_n = s_init ? s_init + (size_t)n * hmat : nullptr;
        float *sfin_n = s_final ? s_final + (size_t)n * hmat : nullptr;
        for (int s = 0; s < pn; ++s) {
            const int j = j0 + s, r = r0 + s;
            const long start = a + (long)s * L * 64;
            cu_seg[j] = (int32_t)(start < b ? start : b);
            SegJob main = {-1, 0, nullptr, nullptr}, amap = main, late = main;
            if (s == 0) {
                main = {j, CHAIN_OUTPUT, sin_n, pn == 1 ? sfin_n : inits + (size_t)(j + 1) * hmat};
            } else {
                late = {j, CHAIN_OUTPUT, inits + (size_t)j * hmat, s == pn - 1 ? sfin_n : nullptr};
                if (s < pn - 1) {
                    main = {j, 0, nullptr, Bm + (size_t)j * hmat};
                    amap = {j, CHAIN_ZERO_V | CHAIN_INIT_IDENTITY, nullptr, Am + (size_t)j * hmat};
                }
            }
            job1[r] = main;
            job1[nsmax + r] = amap;
            job2[r] = late;
        }
    }
    // the unused tail: empty segments at the end, no jobs
    long aN, bN;
    plan_bounds(cu, N - 1, T, aN, bN);
    for (int j = total + tid; j <= nsmax; j += PL_NT) {
        cu_seg[j] = (int32_t)bN;
        if (j < nsmax) {
            const SegJob none = {-1, 0, nullptr, nullptr};
            job1[j] = none;
            job1[nsmax + j] = none;
            job2[j] = none;
        }
    }
}

// The final state when there is no token: the initial state, or zeros.
__global__ void state_copy_kernel(const float *src, float *dst, long n4)
{
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n4)
        reinterpret_cast<f32x4 *>(dst)[i] =
            src ? reinterpret_cast<const f32x4 *>(src)[i] : f32x4{0.f, 0.f, 0.f, 0.f};
}

// Compose. One workgroup of 8 waves per (sequence, head, block of 16 state
// rows), the row block of S in LDS: S = S_1 (segment 1's start state), then
// for the middle segments s = 1 .. P_n - 2 in order S <- S A_s + B_s, stored
// as segment s + 1's start state, on the fp32 matrix cores
// (v_mfma_f32_16x16x4f32), wave w forming columns 16 w .. 16 w + 15. The k
// index of the product is dealt as k = 32 (lane / 16) + q over the 32
// k-steps q, so that a lane's S operands are 32 consecutive floats of its row
// (eight 16-byte LDS reads) and its A_s operands one column of rows
// 32 (lane / 16) .. + 31, read from memory one segment ahead; two
// accumulators halve the dependent chain.
constexpr int SC_NT = 512;
constexpr int SC_LDS_BYTES = 16 * (SP_D + 4) * 4;
static_assert(SC_LDS_BYTES <= 65536, "within the default dynamic LDS limit");
__global__ void __launch_bounds__(SC_NT)
seg_compose_kernel(const float *__restrict__ Amat, const float *__restrict__ Bmat,
                   float *__restrict__ inits, const int32_t *__restrict__ seg_first,
                   const int32_t *__restrict__ seg_count, int H)
{
    extern __shared__ __attribute__((aligned(16))) float sm[];
    float(*sS)[SP_D + 4] = reinterpret_cast<float(*)[SP_D + 4]>(sm);
    const int bh = blockIdx.x, n = bh / H, h = bh - n * H;
    const int j0 = seg_first[n], pn = seg_count[n];
    if (pn <= 2) return;                       // uniform: no middle segment
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, kq = lane >> 4;
    const int r0 = blockIdx.y * 16, col = 16 * wave + m;
    const int vr = tid >> 5, vc = 4 * (tid & 31);      // this thread's 16-byte piece of the row block
    auto mat = [&](auto *base, int j) { return base + ((size_t)j * H + h) * SP_MAT; };
    auto load_a = [&](int s2, float (&dst)[32]) {
        const float *a = mat(Amat, j0 + s2) + (size_t)(32 * kq) * SP_D + col;
#pragma unroll
        for (int q = 0; q < 32; ++q) dst[q] = a[(size_t)q * SP_D];
    };
    *reinterpret_cast<f32x4 *>(&sS[vr][vc]) =
        *reinterpret_cast<const f32x4 *>(mat(inits, j0 + 1) + (size_t)(r0 + vr) * SP_D + vc);
    __syncthreads();
    // middle segment s with its A_s operands in `cur`; the next one's go to `nxt`
    auto step = [&](int s, const float (&cur)[32], float (&nxt)[32]) {
        if (s + 1 < pn - 1) load_a(s + 1, nxt);
        const float *bp = mat(Bmat, j0 + s) + (size_t)(r0 + 4 * kq) * SP_D + col;
        float bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) bv[i] = bp[(size_t)i * SP_D];
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
        const float *srow = &sS[m][32 * kq];
#pragma unroll
        for (int q4 = 0; q4 < 8; ++q4) {
            const f32x4 a4 = *reinterpret_cast<const f32x4 *>(srow + 4 * q4);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[0], cur[4 * q4], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[1], cur[4 * q4 + 1], acc1, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[2], cur[4 * q4 + 2], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[3], cur[4 * q4 + 3], acc1, 0, 0, 0);
        }
        __syncthreads();                       // every wave has read the row block
#pragma unroll
        for (int i = 0; i < 4; ++i) sS[4 * kq + i][col] = (acc0[i] + acc1[i]) + bv[i];
        __syncthreads();                       // the new row block complete
        *reinterpret_cast<f32x4 *>(mat(inits, j0 + s + 1) + (size_t)(r0 + vr) * SP_D + vc) =
            *reinterpret_cast<const f32x4 *>(&sS[vr][vc]);
    };
    float a0[32], a1[32];
    load_a(1, a0);
    for (int s = 1; s < pn - 1; s += 2) {
        step(s, a0, a1);
        if (s + 1 < pn - 1) step(s + 1, a1, a0);
    }
}

// Workspace: the two-pass workspace for N * P segments, the plan, and the
// start states, A and B of every (segment, head).
struct SeqparLayout {
    size_t prep, cu, job1, job2, first, count, inits, amat, bmat, total;
};
static SeqparLayout seqpar_layout(long tokens, int H, int N, int P)
{
    const long nsmax = (long)N * P;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    SeqparLayout L;
    L.prep = 0;
    L.cu = up(prefill_split_workspace_bytes(tokens, H, (int)nsmax));
    L.job1 = L.cu + up((size_t)(nsmax + 1) * sizeof(int32_t));
    L.job2 = L.job1 + up((size_t)2 * nsmax * sizeof(SegJob));
    L.first = L.job2 + up((size_t)nsmax * sizeof(SegJob));
    L.count = L.first + up((size_t)N * sizeof(int32_t));
    const size_t mats = (size_t)nsmax * H * SP_MAT * sizeof(float);
    L.inits = L.count + up((size_t)N * sizeof(int32_t));
    L.amat = L.inits + up(mats);
    L.bmat = L.amat + up(mats);
    L.total = L.bmat + up(mats);
    return L;
}

size_t prefill_seqpar_workspace_bytes(long tokens, int H, int N, int P)
{
    return seqpar_layout(tokens, H, N, P).total;
}

hipError_t launch_prefill_seqpar(const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *s_init, float *s_final, void *o,
                                 const int32_t *cu, int T, int H, int Hk, int N, int P,
                                 float scale, void *ws, hipStream_t stream)
{
    const long tokens = cu ? (long)T : (long)N * T;
    if (tokens == 0) {
        // nothing to run: every final state is its initial state (or zero),
        // copied by a kernel (no memset or copy node if the caller captures)
        if (!s_final) return hipSuccess;
        const long n4 = (long)N * H * SP_MAT / 4;
        hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0,
                           stream, s_init, s_final, n4);
        return hipGetLastError();
    }
    const SeqparLayout Ly = seqpar_layout(tokens, H, N, P);
    unsigned char *base = static_cast<unsigned char *>(ws);
    void *prep = base + Ly.prep;
    int32_t *cu_seg = reinterpret_cast<int32_t *>(base + Ly.cu);
    SegJob *job1 = reinterpret_cast<SegJob *>(base + Ly.job1);
    SegJob *job2 = reinterpret_cast<SegJob *>(base + Ly.job2);
    int32_t *first = reinterpret_cast<int32_t *>(base + Ly.first);
    int32_t *count = reinterpret_cast<int32_t *>(base + Ly.count);
    float *In = reinterpret_cast<float *>(base + Ly.inits);
    float *Am = reinterpret_cast<float *>(base + Ly.amat);
    float *Bm = reinterpret_cast<float *>(base + Ly.bmat);
    const int nsmax = N * P;
    const int total = (int)tokens;             // the segments' packed axis

    hipLaunchKernelGGL(seqpar_plan_kernel, dim3(1), dim3(PL_NT), 0, stream, cu, T, N, P, H, nsmax,
                       s_init, s_final, In, Am, Bm, cu_seg, job1, job2, first, count);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess)
        e = launch_prefill_prepare(q, k, g, beta, cu_seg, total, H, Hk, nsmax, prep, stream);
    if (e == hipSuccess)          // pass 1: segment 0 of each sequence, B and A of the middle ones
        e = launch_prefill_apply(q, k, v, g, nullptr, nullptr, o, cu_seg, total, H, Hk, nsmax,
                                 scale, prep, stream, 0, false, job1, 2 * nsmax);
    if (e == hipSuccess) {        // compose: the start states, in order (8.4 KB of LDS:
                                  // within the default dynamic limit)
        hipLaunchKernelGGL(seg_compose_kernel, dim3((unsigned)(N * H), SP_D / 16), dim3(SC_NT),
                           SC_LDS_BYTES, stream, Am, Bm, In, first, count, H);
        e = hipGetLastError();
    }
    if (e == hipSuccess)          // pass 2: the other segments from their true start states
        e = launch_prefill_apply(q, k, v, g, nullptr, nullptr, o, cu_seg, total, H, Hk, nsmax,
                                 scale, prep, stream, 0, false, job2, nsmax);
    return e;
}

}  // namespace gdn
