// prefill_recurrent.hip - token-serial form of the gated delta rule over whole
// sequences, fp32 arithmetic throughout.
//
// This is the recurrent execution path of "[LLM Algorithms-2] Gated DeltaNet:
// Teaching Linear Attention to Overwrite and Forget" (section 5 pseudo-code,
// section 7 table: recurrent vs chunkwise): for each token, decay the state,
// retrieve at k, write the gated error along k, read the updated state with q.
// It serves fp32 inputs (where a bf16 matrix-core path would not meet fp32
// accuracy), head sizes other than 128, and is the on-GPU cross-check of the
// chunkwise kernel.
//
// Grouped heads: q and k may have fewer heads (H_k) than v, g, beta, o and
// the state (H); value head h reads query/key head h / (H / H_k), the
// repeat_interleave head expansion of the "Gated DeltaNet body" layer code in
// "5. Linear Attention" (LinkQwen ch. 5).
//
// Per-channel decay (PERCH; "6.6 Gated DeltaNet", section 6.6.7, the Kimi
// Linear gate): g is [T][H][d_k] and column j of the state decays by
// exp(g[j]) before the retrieval, S_t = S_{t-1} diag(alpha_t)(I - beta k k^T)
// + beta v k^T. Each lane decays its own 8 columns, so the mapping is
// unchanged.
//
// Work mapping: grid (row blocks, H, N). A state row (d_k floats) lives in
// the registers of G = d_k/8 lanes for the whole sequence; rows never
// exchange data. Per token each lane group needs two length-d_k dot
// products, reduced with DPP: S.k on the decayed row before the write and
// S.q on the updated row. Tokens are staged through LDS
// in blocks of TB: the workgroup's 256 threads fetch a block's q, k, g and
// beta with 16-byte loads (once per workgroup, not once per lane group) and
// its rows of v, one block ahead in registers, so the memory latency is paid
// once per block and overlaps the previous block's tokens. One barrier per
// block.
#include "common.h"
#include "launch.h"

namespace gdn {

template <int DK, typename TIO, bool PERCH>
struct RecurrentShape {
    static constexpr int G = DK / 8;                    // lanes per state row
    static constexpr int RPB = 256 / G;                 // state rows per workgroup
    static constexpr int TB = 32;                       // tokens per staged block
    static constexpr int SZ = (int)sizeof(TIO);
    static constexpr int CPT = DK * SZ / 16;            // 16-byte chunks of a q or k row
    static constexpr int NQK = (2 * TB * CPT + 255) / 256;
    static constexpr int NV = (TB * RPB + 255) / 256;   // v elements per thread
    static constexpr int GCH = PERCH ? TB * DK / 4 : 0; // 16-byte chunks of per-channel g
    static constexpr int NG = PERCH ? (GCH + 255) / 256 : 0;
    static constexpr int GD = PERCH ? DK : 1;           // g values per token
    // LDS bytes of one block buffer: q, k [TB][DK] TIO; g [TB][GD] (per channel:
    // exp(g), the decay factors), beta [TB] fp32;
    // v [TB][RPB] fp32
    static constexpr int L_Q = 0;
    static constexpr int L_K = L_Q + TB * DK * SZ;
    static constexpr int L_G = L_K + TB * DK * SZ;
    static constexpr int L_B = L_G + TB * GD * 4;
    static constexpr int L_V = L_B + TB * 4;
    static constexpr int L_BUF = L_V + TB * RPB * 4;
    static_assert(L_BUF % 16 == 0 && L_G % 16 == 0, "16-byte aligned block buffers");
    static_assert(TB % 4 == 0, "token groups of four never run past the block buffer");
};

template <int DK, typename TIO, bool PERCH>
__global__ void __launch_bounds__(256)
prefill_recurrent_kernel(const TIO *__restrict__ q, const TIO *__restrict__ k,
                         const TIO *__restrict__ v, const float *__restrict__ g,
                         const float *__restrict__ beta, const float *s_init,
                         float *s_final, TIO *__restrict__ o,
                         const int32_t *__restrict__ cu_seqlens, int T, int H, int Hk,
                         int d_v, float scale)
{
    using Sh = RecurrentShape<DK, TIO, PERCH>;
    constexpr int G = Sh::G, RPB = Sh::RPB, TB = Sh::TB, CPT = Sh::CPT;
    __shared__ __attribute__((aligned(16))) unsigned char sbuf[2 * Sh::L_BUF];

    const int h = blockIdx.y, n = blockIdx.z;
    const int kh = h / (H / Hk);              // query/key head of value head h
    const int tid = threadIdx.x;
    const int lr = tid % G;
    const int row0 = blockIdx.x * RPB;
    const int rip = tid / G;                  // row within the block
    const int row = row0 + rip;
    const bool active = row < d_v;            // uniform inside a row group
    const int c0 = 4 * lr, c1 = DK / 2 + 4 * lr;

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

    const size_t sbase = (((size_t)n * H + h) * d_v + (active ? row : 0)) * DK;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    if (s_init && active) {
        s0 = load4(s_init + sbase + c0);
        s1 = load4(s_init + sbase + c1);
    }

    // ---- one block's loads, into registers (tokens past the sequence read
    //      as zero: identity steps, and their outputs are not stored) ----
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    u32x4 rqk[Sh::NQK], rg[Sh::NG > 0 ? Sh::NG : 1];
    float rv[Sh::NV], rgs = 0.f, rbs = 0.f;
    auto fetch = [&](long t0) {
#pragma unroll
        for (int i = 0; i < Sh::NQK; ++i) {
            const int c = tid + 256 * i;
            rqk[i] = u32x4{0u, 0u, 0u, 0u};
            if (c < 2 * TB * CPT) {
                const int mat = c / (TB * CPT), rem = c - mat * TB * CPT;
                const int tok = rem / CPT, part = rem - tok * CPT;
                const long t = t0 + tok;
                if (t < eos)
                    rqk[i] = *reinterpret_cast<const u32x4 *>((mat ? k : q) + ((size_t)t * Hk + kh) * DK +
                                                              part * (16 / Sh::SZ));
            }
        }
#pragma unroll
        for (int i = 0; i < Sh::NV; ++i) {
            const int e = tid + 256 * i;
            const int tok = e / RPB, r = e - tok * RPB;
            const long t = t0 + tok;
            rv[i] = (e < TB * RPB && t < eos && row0 + r < d_v)
                        ? to_f32(v[((size_t)t * H + h) * d_v + row0 + r]) : 0.f;
        }
        if constexpr (PERCH) {
#pragma unroll
            for (int i = 0; i < Sh::NG; ++i) {
                const int c = tid + 256 * i;
                const int tok = c / (DK / 4), part = c - tok * (DK / 4);
                const long t = t0 + tok;
                rg[i] = u32x4{0u, 0u, 0u, 0u};
                if (c < Sh::GCH && t < eos)
                    rg[i] = *reinterpret_cast<const u32x4 *>(g + ((size_t)t * H + h) * DK + 4 * part);
            }
        } else {
            rgs = (tid < TB && t0 + tid < eos) ? g[(size_t)(t0 + tid) * H + h] : 0.f;
        }
        rbs = (tid < TB && t0 + tid < eos) ? beta[(size_t)(t0 + tid) * H + h] : 0.f;
    };
    auto stage = [&](int buf) {
        unsigned char *base = sbuf + buf * Sh::L_BUF;
#pragma unroll
        for (int i = 0; i < Sh::NQK; ++i) {
            const int c = tid + 256 * i;
            if (c < 2 * TB * CPT) *reinterpret_cast<u32x4 *>(base + 16 * c) = rqk[i];   // q then k
        }
        float *sv = reinterpret_cast<float *>(base + Sh::L_V);
#pragma unroll
        for (int i = 0; i < Sh::NV; ++i) {
            const int e = tid + 256 * i;
            if (e < TB * RPB) sv[e] = rv[i];
        }
        if constexpr (PERCH) {
#pragma unroll
            for (int i = 0; i < Sh::NG; ++i) {
                const int c = tid + 256 * i;
                if (c < Sh::GCH) {             // stored as the decay factors exp(g)
                    const f32x4 gv = __builtin_bit_cast(f32x4, rg[i]);
                    *reinterpret_cast<f32x4 *>(base + Sh::L_G + 16 * c) =
                        f32x4{__expf(gv[0]), __expf(gv[1]), __expf(gv[2]), __expf(gv[3])};
                }
            }
        } else {
            if (tid < TB) reinterpret_cast<float *>(base + Sh::L_G)[tid] = rgs;
        }
        if (tid < TB) reinterpret_cast<float *>(base + Sh::L_B)[tid] = rbs;
    };

    const long len = eos - bos;
    const int nblocks = (int)((len + TB - 1) / TB);
    if (nblocks > 0) {
        fetch(bos);
        stage(0);
    }
    for (int blk = 0; blk < nblocks; ++blk) {
        __syncthreads();                       // block blk staged; buffer (blk + 1) % 2 free
        const long t0 = bos + (long)blk * TB;
        if (blk + 1 < nblocks) fetch(t0 + TB);
        const unsigned char *base = sbuf + (blk & 1) * Sh::L_BUF;
        const TIO *sq = reinterpret_cast<const TIO *>(base + Sh::L_Q);
        const TIO *sk = reinterpret_cast<const TIO *>(base + Sh::L_K);
        const float *sg = reinterpret_cast<const float *>(base + Sh::L_G);
        const float *sb = reinterpret_cast<const float *>(base + Sh::L_B);
        const float *sv = reinterpret_cast<const float *>(base + Sh::L_V);
        const int nt = (int)(eos - t0 < TB ? eos - t0 : TB);
        // four tokens' operands are read from LDS together, then the four
        // steps run in order: the reads of a group overlap the previous
        // group's arithmetic instead of sitting on every token's critical path
        constexpr int U = 4;
        for (int j0 = 0; j0 < nt; j0 += U) {
            f32x4 k0[U], k1[U], q0[U], q1[U], g0[U], g1[U];
            float bb[U], vv[U], ga[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = j0 + u;           // < TB: the buffers hold TB tokens
                k0[u] = load4(sk + j * DK + c0); k1[u] = load4(sk + j * DK + c1);
                q0[u] = load4(sq + j * DK + c0); q1[u] = load4(sq + j * DK + c1);
                if constexpr (PERCH) {
                    g0[u] = load4(sg + j * DK + c0);
                    g1[u] = load4(sg + j * DK + c1);
                } else {
                    ga[u] = sg[j];
                }
                bb[u] = sb[j];
                vv[u] = sv[j * RPB + rip];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (j0 + u >= nt) break;        // uniform
                // retrieve at k, write the gated error along k, then read the
                // updated row with q (two reductions per token; the read is off
                // the next token's dependency chain)
                float sk_ = 0.f;
                if constexpr (PERCH) {
                    // decay each column first (the block holds exp(g)), then read
                    // the decayed row
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        s0[e] *= g0[u][e];
                        s1[e] *= g1[u][e];
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) sk_ += s0[e] * k0[u][e] + s1[e] * k1[u][e];
                    sk_ = group_sum<G>(sk_);
                    const float delta = bb[u] * (vv[u] - sk_);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        s0[e] += delta * k0[u][e];
                        s1[e] += delta * k1[u][e];
                    }
                } else {
                    const float alpha = __expf(ga[u]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) sk_ += s0[e] * k0[u][e] + s1[e] * k1[u][e];
                    sk_ = group_sum<G>(sk_);
                    const float delta = bb[u] * (vv[u] - alpha * sk_);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        s0[e] = alpha * s0[e] + delta * k0[u][e];
                        s1[e] = alpha * s1[e] + delta * k1[u][e];
                    }
                }
                float sq_ = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) sq_ += s0[e] * q0[u][e] + s1[e] * q1[u][e];
                sq_ = group_sum<G>(sq_);
                if (active && lr == 0)
                    o[((size_t)(t0 + j0 + u) * H + h) * d_v + row] = from_f32<TIO>(scale * sq_);
            }
        }
        if (blk + 1 < nblocks) stage((blk + 1) & 1);
    }
    if (s_final && active) {
        store4(s_final + sbase + c0, s0);
        store4(s_final + sbase + c1, s1);
    }
}

template <typename TIO>
hipError_t launch_prefill_recurrent(const void *q, const void *k, const void *v, const float *g,
                                    const float *beta, const float *s_init, float *s_final,
                                    void *o, const int32_t *cu_seqlens, int T, int H, int Hk,
                                    int d_k, int d_v, int N, float scale, bool per_channel,
                                    hipStream_t stream)
{
    auto go = [&](auto kern, int rpb) {
        dim3 grid((unsigned)((d_v + rpb - 1) / rpb), (unsigned)H, (unsigned)N), block(256);
        hipLaunchKernelGGL(kern, grid, block, 0, stream, (const TIO *)q, (const TIO *)k,
                           (const TIO *)v, g, beta, s_init, s_final, (TIO *)o, cu_seqlens, T,
                           H, Hk, d_v, scale);
        return hipGetLastError();
    };
    if (per_channel) {
        switch (d_k) {
        case 16: return go(prefill_recurrent_kernel<16, TIO, true>, 256 / 2);
        case 32: return go(prefill_recurrent_kernel<32, TIO, true>, 256 / 4);
        case 64: return go(prefill_recurrent_kernel<64, TIO, true>, 256 / 8);
        case 128: return go(prefill_recurrent_kernel<128, TIO, true>, 256 / 16);
        default: return hipErrorInvalidValue;
        }
    }
    switch (d_k) {
    case 16: return go(prefill_recurrent_kernel<16, TIO, false>, 256 / 2);
    case 32: return go(prefill_recurrent_kernel<32, TIO, false>, 256 / 4);
    case 64: return go(prefill_recurrent_kernel<64, TIO, false>, 256 / 8);
    case 128: return go(prefill_recurrent_kernel<128, TIO, false>, 256 / 16);
    default: return hipErrorInvalidValue;
    }
}

template hipError_t launch_prefill_recurrent<float>(const void *, const void *, const void *,
                                                    const float *, const float *, const float *,
                                                    float *, void *, const int32_t *, int, int,
                                                    int, int, int, int, float, bool,
                                                    hipStream_t);
template hipError_t launch_prefill_recurrent<bf16>(const void *, const void *, const void *,
                                                   const float *, const float *, const float *,
                                                   float *, void *, const int32_t *, int, int,
                                                   int, int, int, int, float, bool,
                                                   hipStream_t);

}  // namespace gdn
