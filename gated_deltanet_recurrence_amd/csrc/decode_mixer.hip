// decode_mixer.hip - one token of the whole token mixer for B sequences in a
// single kernel: the prologue on the new token (depthwise causal conv against
// a cache of each channel's last three inputs, SiLU, L2-norm of q and k, the
// gates), the gated delta rule step on the HBM-resident state, and the gated
// RMSNorm of the result.
//
// Sources:
//  "6.6 Gated DeltaNet (linear attention)", LLM full-stack book, section 6.6.8
//   (inference flow: new q, k, v and gates; update the state; read it with q;
//   gate the output with RMSNorm(y) * SiLU(g)); 6.6.3 (gates) and 6.6.4
//   (l2norm with 1e-6 under the square root).
//  "5. Linear Attention" (LinkQwen ch. 5): "Causal Conv1d" (4 taps, SiLU, the
//   window is the three previous inputs and the current one), "Gated RMSNorm",
//   and the layer body (channel order q | k | v, repeat_interleave of q and k
//   over value heads).
//  "[LLM Algorithms-2] Gated DeltaNet: Teaching Linear Attention to Overwrite
//   and Forget", section 13.4: what a deployment caches per sequence is the
//   matrix state plus, in implementations with a short convolution, the
//   convolution's recent inputs; section 5 for the step itself.
//
// Conv cache: per sequence, [3][C] inputs in the I/O dtype, C = 2 H_k d_k +
// H d_v conv channels; row 0 holds the input three tokens back, row 2 the
// previous token. A zero cache is the zero left padding of a fresh sequence.
// The step reads the window (rows 0-2, new input), then shifts the cache by
// one token in place.
//
// Work mapping: one 1024-thread workgroup per (sequence, query/key head): it
// owns the q and k channels of that head and everything of the H / H_k value
// heads that read it (their v channels, gates, state rows and outputs), so
// every cache entry and state row is read and written by exactly one thread
// of the grid and the update can be in place. A state row is owned by
// G = d_k/8 lanes (16-byte loads of both row halves, DPP reductions, as in
// the plain decode step); the first two rows of each lane group are requested
// before the prologue work starts, so the state stream is in flight while the
// convolution is computed. Per-head sums of the RMSNorm run through LDS.
#include "common.h"
#include "launch.h"

namespace gdn {

constexpr int DM_NT = 1024;
constexpr int DM_HIST = 3;                     // cached inputs per channel (4-tap kernel)

template <int DK, typename TIO>
__global__ void __launch_bounds__(DM_NT)
decode_mixer_kernel(const TIO *__restrict__ q_raw, const TIO *__restrict__ k_raw,
                    const TIO *__restrict__ v_raw, const TIO *__restrict__ conv_w,
                    TIO *__restrict__ conv_state, const TIO *__restrict__ a,
                    const TIO *__restrict__ b, const float *__restrict__ A,
                    const float *__restrict__ dt_bias, const TIO *__restrict__ z,
                    const float *__restrict__ norm_w, float *__restrict__ state,
                    TIO *__restrict__ out, int H, int Hk, int d_v, float scale, float eps)
{
    constexpr int G = DK / 8;                  // lanes per state row
    constexpr int RPP = DM_NT / G;             // rows per pass of the workgroup
    const int grp = H / Hk;                    // value heads per query/key head
    const int bk = blockIdx.x;                 // sequence * H_k + query/key head
    const int bb = bk / Hk, kh = bk - bb * Hk;
    const int h0 = kh * grp;                   // first value head of the group
    const int R = grp * d_v;                   // state rows (and outputs) of this workgroup
    const long C = 2L * Hk * DK + (long)H * d_v;   // conv channels
    const int tid = (int)threadIdx.x;
    const int lr = tid % G, gid = tid / G;
    const int c0 = 4 * lr, c1 = DK / 2 + 4 * lr;

    // rows r of this workgroup: value head h0 + r / d_v, state row r % d_v
    auto row_ptr = [&](int r) {
        const int j = r / d_v;
        return state + (((size_t)bb * H + h0 + j) * d_v + (r - j * d_v)) * DK;
    };
    f32x4 s0[2], s1[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int r = gid + p * RPP;
        if (r < R) {
            const float *rp = row_ptr(r);
            s0[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(rp + c0));
            s1[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(rp + c1));
        }
    }

    // this thread's first output gate z and norm weight, requested with the
    // state so that the epilogue does not wait for memory
    const int oc = tid - (tid / d_v) * d_v;
    const size_t oi0 = ((size_t)bb * H + h0) * d_v + tid;
    TIO zraw{};
    float wpre = 1.0f;
    if (tid < R) {
        zraw = z[oi0];
        if (norm_w) wpre = norm_w[oc];
    }

    extern __shared__ __attribute__((aligned(16))) float sm[];
    float *sq = sm;                            // conv + SiLU outputs: q [DK], k [DK], v [R]
    float *sk = sq + DK;
    float *sv = sk + DK;
    float *sy = sv + R;                        // recurrence outputs [R]
    float *salpha = sy + R;                    // per value head of the group: alpha, beta,
    float *sbeta = salpha + grp;               // sum of squared outputs
    float *sss = sbeta + grp;

    // ---- prologue: conv window (three cached inputs, the new one) + SiLU,
    //      cache shifted by one token; the gates of the group's value heads ----
    TIO *cs = conv_state + (size_t)bb * DM_HIST * C;
    for (int i = tid; i < 2 * DK + R; i += DM_NT) {
        long ch;
        float x;
        if (i < DK) {
            ch = (long)kh * DK + i;
            x = to_f32(q_raw[(size_t)bk * DK + i]);
        } else if (i < 2 * DK) {
            ch = (long)Hk * DK + (long)kh * DK + (i - DK);
            x = to_f32(k_raw[(size_t)bk * DK + (i - DK)]);
        } else {
            const int r = i - 2 * DK;
            ch = 2L * Hk * DK + (long)h0 * d_v + r;
            x = to_f32(v_raw[((size_t)bb * H + h0) * d_v + r]);
        }
        const TIO x3 = cs[ch], x2 = cs[C + ch], x1 = cs[2 * C + ch];
        const TIO *w = conv_w + ch * 4;
        const float pre = to_f32(w[3]) * x + to_f32(w[2]) * to_f32(x1) + to_f32(w[1]) * to_f32(x2)
                        + to_f32(w[0]) * to_f32(x3);
        sq[i] = silu_f32(pre);                 // sq, sk, sv are consecutive
        cs[ch] = x2;
        cs[C + ch] = x1;
        cs[2 * C + ch] = from_f32<TIO>(x);
    }
    if (tid < grp) {
        const int h = h0 + tid;
        const size_t i = (size_t)bb * H + h;
        const float bias = dt_bias ? dt_bias[h] : 0.f;
        salpha[tid] = __expf(-A[h] * softplus_f32(to_f32(a[i]) + bias));
        sbeta[tid] = 1.0f / (1.0f + expf(-to_f32(b[i])));
        sss[tid] = 0.f;
    }
    __syncthreads();

    // ---- recurrence: L2-normalised q, k slices per lane group, then the
    //      rows of the group's value heads ----
    f32x4 q0 = *reinterpret_cast<const f32x4 *>(sq + c0), q1 = *reinterpret_cast<const f32x4 *>(sq + c1);
    f32x4 k0 = *reinterpret_cast<const f32x4 *>(sk + c0), k1 = *reinterpret_cast<const f32x4 *>(sk + c1);
    float ssq = 0.f, ssk = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        ssq += q0[e] * q0[e] + q1[e] * q1[e];
        ssk += k0[e] * k0[e] + k1[e] * k1[e];
    }
    ssq = group_sum<G>(ssq);
    ssk = group_sum<G>(ssk);
    const float iq = rsqrt_f32(ssq + 1e-6f), ik = rsqrt_f32(ssk + 1e-6f);
    q0 *= iq; q1 *= iq; k0 *= ik; k1 *= ik;
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) kq += k0[e] * q0[e] + k1[e] * q1[e];
    kq = group_sum<G>(kq);

    for (int base = 0; base < R; base += 2 * RPP) {
        if (base > 0) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int r = base + gid + p * RPP;
                if (r < R) {
                    const float *rp = row_ptr(r);
                    s0[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(rp + c0));
                    s1[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(rp + c1));
                }
            }
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int r = base + gid + p * RPP;
            if (r < R) {                       // uniform across a lane group
                const int j = r / d_v;
                const float alpha = salpha[j], beta = sbeta[j], vv = sv[r];
                float sk_ = 0.f, sq_ = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sk_ += s0[p][e] * k0[e] + s1[p][e] * k1[e];
                    sq_ += s0[p][e] * q0[e] + s1[p][e] * q1[e];
                }
                sk_ = group_sum<G>(sk_);
                sq_ = group_sum<G>(sq_);
                const float delta = beta * (vv - alpha * sk_);
                f32x4 n0, n1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    n0[e] = alpha * s0[p][e] + delta * k0[e];
                    n1[e] = alpha * s1[p][e] + delta * k1[e];
                }
                float *rp = row_ptr(r);
                __builtin_nontemporal_store(n0, reinterpret_cast<f32x4 *>(rp + c0));
                __builtin_nontemporal_store(n1, reinterpret_cast<f32x4 *>(rp + c1));
                if (lr == 0) sy[r] = scale * (alpha * sq_ + delta * kq);
            }
        }
    }
    __syncthreads();

    // ---- gated RMSNorm per value head: sums of squares over d_v outputs
    //      (a wave's 64 outputs belong to one head when d_v >= 64; smaller
    //      heads are summed over their 16 or 32 lanes), then the outputs ----
    for (int i = tid; i < R; i += DM_NT) {
        const float y = sy[i];
        float ss = y * y;
        if (d_v >= 64) ss = group_sum<64>(ss);
        else if (d_v == 32) ss = group_sum<32>(ss);
        else ss = group_sum<16>(ss);
        const int seg = d_v < 64 ? d_v : 64;
        if ((i & (seg - 1)) == 0) atomicAdd(&sss[i / d_v], ss);
    }
    __syncthreads();
    for (int i = tid; i < R; i += DM_NT) {
        const int j = i / d_v, c = i - j * d_v;
        const size_t oi = ((size_t)bb * H + h0) * d_v + i;
        const float inv = rsqrt_f32(sss[j] * (1.0f / d_v) + eps);
        const bool first = i == tid;
        const float wv = first ? wpre : (norm_w ? norm_w[c] : 1.0f);
        const float zv = to_f32(first ? zraw : z[oi]);
        out[oi] = from_f32<TIO>(wv * (sy[i] * inv) * silu_f32(zv));
    }
}

size_t decode_mixer_lds_bytes(int H, int Hk, int d_k, int d_v)
{
    const int grp = H / Hk;
    return sizeof(float) * (2 * (size_t)d_k + 2 * (size_t)grp * d_v + 3 * (size_t)grp);
}

template <typename TIO>
hipError_t launch_decode_mixer(const void *q_raw, const void *k_raw, const void *v_raw,
                               const void *conv_w, void *conv_state, const void *a,
                               const void *b, const float *A, const float *dt_bias,
                               const void *z, const float *norm_w, float eps, float *state,
                               void *out, int B, int H, int Hk, int d_k, int d_v, float scale,
                               hipStream_t stream)
{
    const size_t lds = decode_mixer_lds_bytes(H, Hk, d_k, d_v);
    dim3 grid((unsigned)((long)B * Hk)), block(DM_NT);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, lds, stream, (const TIO *)q_raw, (const TIO *)k_raw,
                           (const TIO *)v_raw, (const TIO *)conv_w, (TIO *)conv_state,
                           (const TIO *)a, (const TIO *)b, A, dt_bias, (const TIO *)z, norm_w,
                           state, (TIO *)out, H, Hk, d_v, scale, eps);
        return hipGetLastError();
    };
    switch (d_k) {
    case 16: return go(decode_mixer_kernel<16, TIO>);
    case 32: return go(decode_mixer_kernel<32, TIO>);
    case 64: return go(decode_mixer_kernel<64, TIO>);
    case 128: return go(decode_mixer_kernel<128, TIO>);
    default: return hipErrorInvalidValue;
    }
}

template hipError_t launch_decode_mixer<float>(const void *, const void *, const void *,
                                               const void *, void *, const void *, const void *,
                                               const float *, const float *, const void *,
                                               const float *, float, float *, void *, int, int,
                                               int, int, int, float, hipStream_t);
template hipError_t launch_decode_mixer<bf16>(const void *, const void *, const void *,
                                              const void *, void *, const void *, const void *,
                                              const float *, const float *, const void *,
                                              const float *, float, float *, void *, int, int,
                                              int, int, int, float, hipStream_t);

}  // namespace gdn
