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
// exchange data, so there is no barrier anywhere. Per token each lane group
// needs three length-d_k dot products (S.k, S.q, k.q), reduced with DPP.
// The next token's q, k, v, g, beta are fetched while the current token is
// being processed.
#include "common.h"

namespace gdn {

template <int DK, typename TIO, bool PERCH>
__global__ void __launch_bounds__(256)
prefill_recurrent_kernel(const TIO *__restrict__ q, const TIO *__restrict__ k,
                         const TIO *__restrict__ v, const float *__restrict__ g,
                         const float *__restrict__ beta, const float *s_init,
                         float *s_final, TIO *__restrict__ o,
                         const int32_t *__restrict__ cu_seqlens, int T, int H, int Hk,
                         int d_v, float scale)
{
    constexpr int G = DK / 8;
    constexpr int RPB = 256 / G;              // state rows per workgroup
    const int h = blockIdx.y, n = blockIdx.z;
    const int kh = h / (H / Hk);              // query/key head of value head h
    const int tid = threadIdx.x;
    const int lr = tid % G;
    const int row = blockIdx.x * RPB + tid / G;
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

    const int vrow = active ? row : 0;
    // gg: the scalar log-decay; with PERCH, gc0/gc1 those of this lane's columns
    auto fetch = [&](long t, f32x4 &k0, f32x4 &k1, f32x4 &q0, f32x4 &q1, float &vv, float &gg,
                     f32x4 &gc0, f32x4 &gc1, float &bb) {
        const size_t tk = ((size_t)t * Hk + kh) * DK;
        k0 = load4(k + tk + c0);
        k1 = load4(k + tk + c1);
        q0 = load4(q + tk + c0);
        q1 = load4(q + tk + c1);
        vv = to_f32(v[((size_t)t * H + h) * d_v + vrow]);
        if constexpr (PERCH) {
            const float *gp = g + ((size_t)t * H + h) * DK;
            gc0 = load4(gp + c0);
            gc1 = load4(gp + c1);
        } else {
            gg = g[(size_t)t * H + h];
        }
        bb = beta[(size_t)t * H + h];
    };

    f32x4 k0, k1, q0, q1, gc0 = {0.f, 0.f, 0.f, 0.f}, gc1 = gc0;
    float vv = 0.f, gg = 0.f, bb = 0.f;
    if (bos < eos)
        fetch(bos, k0, k1, q0, q1, vv, gg, gc0, gc1, bb);
    for (long t = bos; t < eos; ++t) {
        f32x4 nk0 = k0, nk1 = k1, nq0 = q0, nq1 = q1, ngc0 = gc0, ngc1 = gc1;
        float nvv = vv, ngg = gg, nbb = bb;
        if (t + 1 < eos)
            fetch(t + 1, nk0, nk1, nq0, nq1, nvv, ngg, ngc0, ngc1, nbb);

        float delta, sq, kq = 0.f;
        if constexpr (PERCH) {
            // decay each column first, then read the decayed row
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s0[e] *= __expf(gc0[e]);
                s1[e] *= __expf(gc1[e]);
            }
            float sk = 0.f;
            sq = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sk += s0[e] * k0[e] + s1[e] * k1[e];
                sq += s0[e] * q0[e] + s1[e] * q1[e];
                kq += k0[e] * q0[e] + k1[e] * q1[e];
            }
            sk = group_sum<G>(sk);
            sq = group_sum<G>(sq);
            kq = group_sum<G>(kq);
            delta = bb * (vv - sk);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s0[e] += delta * k0[e];
                s1[e] += delta * k1[e];
            }
        } else {
            const float alpha = __expf(gg);
            float sk = 0.f;
            sq = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sk += s0[e] * k0[e] + s1[e] * k1[e];
                sq += s0[e] * q0[e] + s1[e] * q1[e];
                kq += k0[e] * q0[e] + k1[e] * q1[e];
            }
            sk = group_sum<G>(sk);
            sq = group_sum<G>(sq);
            kq = group_sum<G>(kq);
            delta = bb * (vv - alpha * sk);
            sq *= alpha;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s0[e] = alpha * s0[e] + delta * k0[e];
                s1[e] = alpha * s1[e] + delta * k1[e];
            }
        }
        if (active && lr == 0)
            o[((size_t)t * H + h) * d_v + row] = from_f32<TIO>(scale * (sq + delta * kq));

        k0 = nk0; k1 = nk1; q0 = nq0; q1 = nq1;
        vv = nvv; gg = ngg; bb = nbb; gc0 = ngc0; gc1 = ngc1;
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
