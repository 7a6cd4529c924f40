// seqpar.hip - sequence-parallel chunked prefill: one long sequence is cut
// into segments whose chains run side by side.
//
// "[LLM Algorithms-2] Gated DeltaNet: Teaching Linear Attention to Overwrite
// and Forget", section 7: a run of tokens acts on the state as one affine map,
// S_end = S_start A + B (A = the product of the tokens' alpha (I - beta k k^T),
// B = the decayed sum of their writes). So, with the sequence cut into P
// segments of whole 64-token chunks:
//   1. every segment's chain runs from a zero state on its own values:
//      its final state is B_s;
//   2. every segment's chain runs with v = 0 from the identity: its final
//      state (d_v = d_k rows e_j A_s) is A_s;
//   3. the segment start states follow in order, S_{s+1} = S_s A_s + B_s,
//      S_0 the caller's initial state; S_P is the final state;
//   4. every segment's chain runs again from S_s and writes the outputs.
// Steps 1, 2 and 4 are the chain pass over P times more (shorter) sequences,
// so a batch with too few (sequence, head) pairs to fill the GPU fills it;
// the price is three chain passes instead of one, and step 3's P dependent
// 128 x 128 x 128 products per head.
#include "chunk_common.h"

namespace gdn {

constexpr int SP_D = 128;                      // d_k = d_v of the chunk kernels

hipError_t launch_prefill_prepare(const void *, const void *, const float *, const float *,
                                  const int32_t *, int, int, int, int, void *, hipStream_t,
                                  bool per_channel = false);
hipError_t launch_prefill_apply(const void *, const void *, const void *, const float *,
                                const float *, float *, void *, const int32_t *, int, int, int,
                                int, float, const void *, hipStream_t, int flags,
                                bool per_channel = false);
size_t prefill_split_workspace_bytes(long tokens, int H, int N, bool per_channel = false);

namespace split {
constexpr int CHAIN_ZERO_V = 1;                // as in prefill_split.hip
constexpr int CHAIN_INIT_IDENTITY = 2;
}

// Segment offsets of B sequences of T tokens cut into P segments of L tokens
// (the last ones shorter or empty), packed along the token axis.
__global__ void seg_offsets_kernel(int32_t *cu, int B, int T, int P, int L)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int n = B * P;
    if (i > n) return;
    if (i == n) { cu[i] = B * T; return; }
    const int b = i / P, s = i - b * P;
    const long start = (long)s * L;
    cu[i] = (int32_t)((long)b * T + (start < T ? start : T));
}

// The final state when there is no token: the initial state, or zeros.
__global__ void state_copy_kernel(const float *src, float *dst, long n4)
{
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n4)
        reinterpret_cast<f32x4 *>(dst)[i] =
            src ? reinterpret_cast<const f32x4 *>(src)[i] : f32x4{0.f, 0.f, 0.f, 0.f};
}

// Step 3. One workgroup of 8 waves per (sequence, head, block of 16 state
// rows), the row block of S in LDS. For s = 0 .. P-1: inits[s] = S, then
// S <- S A_s + B_s on the fp32 matrix cores (v_mfma_f32_16x16x4f32), wave w
// forming columns 16 w .. 16 w + 15. The k index of the product is dealt as
// k = 32 (lane / 16) + q over the 32 k-steps q, so that a lane's S operands
// are 32 consecutive floats of its row (eight 16-byte LDS reads) and its A_s
// operands one column of rows 32 (lane / 16) .. + 31, read from memory one
// segment ahead; two accumulators halve the dependent chain.
constexpr int SC_NT = 512;
constexpr int SC_LDS_BYTES = 16 * (SP_D + 4) * 4;
__global__ void __launch_bounds__(SC_NT)
seg_compose_kernel(const float *__restrict__ Amat, const float *__restrict__ Bmat,
                   const float *s_init, float *__restrict__ inits, float *s_final, int H, int P)
{
    extern __shared__ __attribute__((aligned(16))) float sm[];
    float(*sS)[SP_D + 4] = reinterpret_cast<float(*)[SP_D + 4]>(sm);
    const int bh = blockIdx.x, b = bh / H, h = bh - b * H;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, kq = lane >> 4;
    const int r0 = blockIdx.y * 16, col = 16 * wave + m;
    const int vr = tid >> 5, vc = 4 * (tid & 31);      // this thread's 16-byte piece of the row block
    const size_t mat = (size_t)SP_D * SP_D;
    auto seg_of = [&](int s2) { return ((size_t)b * P + s2) * H + h; };
    auto load_a = [&](int s2, float (&dst)[32]) {
        const float *a = Amat + seg_of(s2) * mat + (size_t)(32 * kq) * SP_D + col;
#pragma unroll
        for (int q = 0; q < 32; ++q) dst[q] = a[(size_t)q * SP_D];
    };
    *reinterpret_cast<f32x4 *>(&sS[vr][vc]) =
        s_init ? *reinterpret_cast<const f32x4 *>(s_init + ((size_t)bh * SP_D + r0 + vr) * SP_D + vc)
               : f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    // one segment with the A_s operands in `cur`; the next segment's go to `nxt`
    auto step = [&](int s, const float (&cur)[32], float (&nxt)[32]) {
        const size_t seg = seg_of(s);
        *reinterpret_cast<f32x4 *>(inits + seg * mat + (size_t)(r0 + vr) * SP_D + vc) =
            *reinterpret_cast<const f32x4 *>(&sS[vr][vc]);
        if (s + 1 < P) load_a(s + 1, nxt);
        const float *bp = Bmat + seg * mat + (size_t)(r0 + 4 * kq) * SP_D + col;
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
    };
    float a0[32], a1[32];
    if (P > 0) load_a(0, a0);
    for (int s = 0; s < P; s += 2) {
        step(s, a0, a1);
        if (s + 1 < P) step(s + 1, a1, a0);
    }
    if (s_final)
        *reinterpret_cast<f32x4 *>(s_final + ((size_t)bh * SP_D + r0 + vr) * SP_D + vc) =
            *reinterpret_cast<const f32x4 *>(&sS[vr][vc]);
}

// Workspace: the two-pass workspace for B * P segments, their offsets, and
// A, B and the start states of every (segment, head).
struct SeqparLayout {
    size_t prep, cu, amat, bmat, inits, total;
};
static SeqparLayout seqpar_layout(int B, int T, int H, int P)
{
    const int nseg = B * P;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    SeqparLayout L;
    L.prep = 0;
    L.cu = up(prefill_split_workspace_bytes((long)B * T, H, nseg));
    const size_t mats = (size_t)nseg * H * SP_D * SP_D * sizeof(float);
    L.amat = L.cu + up((size_t)(nseg + 1) * sizeof(int32_t));
    L.bmat = L.amat + up(mats);
    L.inits = L.bmat + up(mats);
    L.total = L.inits + up(mats);
    return L;
}

size_t prefill_seqpar_workspace_bytes(int B, int T, int H, int P)
{
    return seqpar_layout(B, T, H, P).total;
}

hipError_t launch_prefill_seqpar(const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *s_init, float *s_final,
                                 void *o, int B, int T, int H, int Hk, int P, float scale,
                                 void *ws, hipStream_t stream)
{
    if ((long)B * T == 0) {
        // nothing to run: the final state is the initial state (or zero),
        // copied by a kernel (no memset or copy node if the caller captures)
        if (!s_final) return hipSuccess;
        const long n4 = (long)B * H * SP_D * SP_D / 4;
        hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0,
                           stream, s_init, s_final, n4);
        return hipGetLastError();
    }
    const SeqparLayout Ly = seqpar_layout(B, T, H, P);
    unsigned char *base = static_cast<unsigned char *>(ws);
    void *prep = base + Ly.prep;
    int32_t *cu = reinterpret_cast<int32_t *>(base + Ly.cu);
    float *Am = reinterpret_cast<float *>(base + Ly.amat);
    float *Bm = reinterpret_cast<float *>(base + Ly.bmat);
    float *In = reinterpret_cast<float *>(base + Ly.inits);
    const int nseg = B * P;
    const int chunks = (T + 63) / 64;
    const int L = ((chunks + P - 1) / P) * 64;     // tokens per segment, whole chunks
    const int total = B * T;

    hipLaunchKernelGGL(seg_offsets_kernel, dim3((nseg + 1 + 255) / 256), dim3(256), 0, stream,
                       cu, B, T, P, L);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess)
        e = launch_prefill_prepare(q, k, g, beta, cu, total, H, Hk, nseg, prep, stream);
    if (e == hipSuccess)          // 1: B_s, the segments from a zero state
        e = launch_prefill_apply(q, k, v, g, nullptr, Bm, nullptr, cu, total, H, Hk, nseg, scale,
                                 prep, stream, 0);
    if (e == hipSuccess)          // 2: A_s, v = 0 from the identity
        e = launch_prefill_apply(q, k, v, g, nullptr, Am, nullptr, cu, total, H, Hk, nseg, scale,
                                 prep, stream, split::CHAIN_ZERO_V | split::CHAIN_INIT_IDENTITY);
    if (e == hipSuccess) {        // 3: the start states, in order
        static const hipError_t attr = hipFuncSetAttribute(
            (const void *)seg_compose_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, SC_LDS_BYTES);
        e = attr;
        if (e == hipSuccess) {
            hipLaunchKernelGGL(seg_compose_kernel, dim3((unsigned)(B * H), SP_D / 16), dim3(SC_NT),
                               SC_LDS_BYTES, stream, Am, Bm, s_init, In, s_final, H, P);
            e = hipGetLastError();
        }
    }
    if (e == hipSuccess)          // 4: the outputs
        e = launch_prefill_apply(q, k, v, g, In, nullptr, o, cu, total, H, Hk, nseg, scale, prep,
                                 stream, 0);
    return e;
}

}  // namespace gdn
