// decode.hip - one recurrent step of the gated delta rule on an HBM-resident
// fp32 state, updated in place.
//
// Method ("[LLM Algorithms-2] Gated DeltaNet: Teaching Linear Attention to
// Overwrite and Forget", sections 4.3 and 5): decay the state, retrieve what
// it holds at k, write the gated error along k, read with q:
//   r_v     = alpha * (S_v . k)                  (retrieval from the decayed row)
//   delta_v = beta * (v_v - r_v)
//   S_v    <- alpha * S_v + delta_v * k          (row v of the d_v x d_k state)
//   o_v     = scale * (alpha * (S_v . q) + delta_v * (k . q))   (= scale * S_v' . q)
//
// Every row v of the state updates independently of the others, so the step
// is one streaming pass: each state row is read once and written once, and
// the only reductions run along d_k, inside a group of d_k/8 lanes, with DPP.
//
// Work mapping: one 256-thread workgroup per (batch, head). A row of d_k
// floats is owned by G = d_k/8 consecutive lanes; lane j of the group holds
// columns [4j, 4j+4) and [d_k/2 + 4j, d_k/2 + 4j + 4), so each 16-byte load
// instruction of a group covers one contiguous half row (256 B at d_k = 128)
// and a wave's load covers whole cache lines. All rows of the workgroup are
// loaded before any is updated, to keep many 16-byte requests in flight.
#include "common.h"

namespace gdn {

template <int DK, int NPASS, typename TIO>
__global__ void __launch_bounds__(256)
decode_step_kernel(const TIO *__restrict__ q, const TIO *__restrict__ k,
                   const TIO *__restrict__ v, const float *__restrict__ g,
                   const float *__restrict__ beta, float *__restrict__ state,
                   TIO *__restrict__ o, int H, int d_v, float scale)
{
    constexpr int G = DK / 8;                 // lanes per state row
    constexpr int RPP = 256 / G;              // rows per pass of the workgroup
    const int bh = blockIdx.x;                // b * H + h
    const int tid = threadIdx.x;
    const int lr = tid % G;                   // lane within its row group
    const int rip = tid / G;                  // row within a pass
    const int c0 = 4 * lr, c1 = DK / 2 + 4 * lr;

    const TIO *qp = q + (size_t)bh * DK;
    const TIO *kp = k + (size_t)bh * DK;
    const f32x4 k0 = load4(kp + c0), k1 = load4(kp + c1);
    const f32x4 q0 = load4(qp + c0), q1 = load4(qp + c1);
    const float alpha = __expf(g[bh]);
    const float b = beta[bh];
    float kq = k0[0] * q0[0] + k0[1] * q0[1] + k0[2] * q0[2] + k0[3] * q0[3]
             + k1[0] * q1[0] + k1[1] * q1[1] + k1[2] * q1[2] + k1[3] * q1[3];
    kq = group_sum<G>(kq);

    float *sp = state + (size_t)bh * d_v * DK;
    const TIO *vp = v + (size_t)bh * d_v;
    TIO *op = o + (size_t)bh * d_v;

    for (int base = 0; base < d_v; base += NPASS * RPP) {
        f32x4 s0[NPASS], s1[NPASS];
        float vv[NPASS];
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int row = base + p * RPP + rip;
            if (row < d_v) {
                const float *rp = sp + (size_t)row * DK;
                s0[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(rp + c0));
                s1[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(rp + c1));
                vv[p] = to_f32(vp[row]);
            }
        }
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int row = base + p * RPP + rip;
            if (row < d_v) {                 // uniform across a row group
                float sk = s0[p][0] * k0[0] + s0[p][1] * k0[1] + s0[p][2] * k0[2] + s0[p][3] * k0[3]
                         + s1[p][0] * k1[0] + s1[p][1] * k1[1] + s1[p][2] * k1[2] + s1[p][3] * k1[3];
                float sq = s0[p][0] * q0[0] + s0[p][1] * q0[1] + s0[p][2] * q0[2] + s0[p][3] * q0[3]
                         + s1[p][0] * q1[0] + s1[p][1] * q1[1] + s1[p][2] * q1[2] + s1[p][3] * q1[3];
                sk = group_sum<G>(sk);
                sq = group_sum<G>(sq);
                const float delta = b * (vv[p] - alpha * sk);
                f32x4 n0, n1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    n0[e] = alpha * s0[p][e] + delta * k0[e];
                    n1[e] = alpha * s1[p][e] + delta * k1[e];
                }
                float *rp = sp + (size_t)row * DK;
                __builtin_nontemporal_store(n0, reinterpret_cast<f32x4 *>(rp + c0));
                __builtin_nontemporal_store(n1, reinterpret_cast<f32x4 *>(rp + c1));
                if (lr == 0)
                    op[row] = from_f32<TIO>(scale * (alpha * sq + delta * kq));
            }
        }
    }
}

template <int DK, typename TIO>
static hipError_t launch_decode_dk(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, float *state, void *o, int B, int H,
                                   int d_v, float scale, hipStream_t stream)
{
    constexpr int RPP = 256 / (DK / 8);
    // Rows per workgroup pass: enough passes to cover d_v = DK rows in one
    // unrolled sweep (8 at d_k = 128), capped for register use.
    constexpr int NPASS = (DK + RPP - 1) / RPP > 8 ? 8 : ((DK + RPP - 1) / RPP);
    dim3 grid((unsigned)(B * H)), block(256);
    hipLaunchKernelGGL((decode_step_kernel<DK, NPASS, TIO>), grid, block, 0, stream,
                       (const TIO *)q, (const TIO *)k, (const TIO *)v, g, beta, state,
                       (TIO *)o, H, d_v, scale);
    return hipGetLastError();
}

template <typename TIO>
hipError_t launch_decode(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, float *state, void *o, int B, int H, int d_k,
                         int d_v, float scale, hipStream_t stream)
{
    switch (d_k) {
    case 16: return launch_decode_dk<16, TIO>(q, k, v, g, beta, state, o, B, H, d_v, scale, stream);
    case 32: return launch_decode_dk<32, TIO>(q, k, v, g, beta, state, o, B, H, d_v, scale, stream);
    case 64: return launch_decode_dk<64, TIO>(q, k, v, g, beta, state, o, B, H, d_v, scale, stream);
    case 128: return launch_decode_dk<128, TIO>(q, k, v, g, beta, state, o, B, H, d_v, scale, stream);
    default: return hipErrorInvalidValue;
    }
}

template hipError_t launch_decode<float>(const void *, const void *, const void *, const float *,
                                         const float *, float *, void *, int, int, int, int,
                                         float, hipStream_t);
template hipError_t launch_decode<bf16>(const void *, const void *, const void *, const float *,
                                        const float *, float *, void *, int, int, int, int,
                                        float, hipStream_t);

}  // namespace gdn
