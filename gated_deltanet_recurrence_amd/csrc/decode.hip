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
// Grouped heads: q and k have H_k heads, everything else H; value head h
// reads query/key head h / (H / H_k) (the repeat_interleave head expansion of
// the "Gated DeltaNet body" layer code, "5. Linear Attention").
//
// Per-channel decay (PERCH; "6.6 Gated DeltaNet" section 6.6.7): g is
// [B][H][d_k] and column j of the state decays by exp(g[j]) before the
// retrieval; each lane decays its own 8 columns.
//
// Work mapping: a row of d_k floats is owned by G = d_k/8 consecutive lanes;
// lane j of the group holds columns [4j, 4j+4) and [d_k/2 + 4j, d_k/2 + 4j + 4),
// so each 16-byte load instruction of a group covers one contiguous half row
// (256 B at d_k = 128) and a wave's load covers whole cache lines. Each lane
// group handles exactly one row, and a 512-thread workgroup 512/G rows of one
// (batch, head) (32 at d_k = 128, so four workgroups per 128-row head): many
// small workgroups keep more 16-byte requests in flight per CU than a few
// that walk many rows each. The state row is requested before anything else,
// non-temporally (it is touched once); q, k, v, g and beta follow, shared by
// the head's workgroups through the cache.
#include "common.h"
#include "launch.h"

namespace gdn {

constexpr int DEC_NT = 512;

template <int DK, typename TIO, bool PERCH>
__global__ void __launch_bounds__(DEC_NT)
decode_step_kernel(const TIO *__restrict__ q, const TIO *__restrict__ k,
                   const TIO *__restrict__ v, const float *__restrict__ g,
                   const float *__restrict__ beta, float *__restrict__ state,
                   TIO *__restrict__ o, int grp, int d_v, int wg_per_head, float scale)
{
    constexpr int G = DK / 8;                 // lanes per state row
    constexpr int RPW = DEC_NT / G;           // rows per workgroup
    const int bh = blockIdx.x / wg_per_head;  // b * H + h
    const int row = (blockIdx.x - bh * wg_per_head) * RPW + (int)threadIdx.x / G;
    if (row >= d_v) return;                   // whole row groups leave together
    const int lr = threadIdx.x % G;           // lane within its row group
    const int c0 = 4 * lr, c1 = DK / 2 + 4 * lr;

    float *rp = state + ((size_t)bh * d_v + row) * DK;
    f32x4 s0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(rp + c0));
    f32x4 s1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(rp + c1));
    __builtin_amdgcn_sched_barrier(0);        // the state request goes out first

    // grp = H / H_k value heads per query/key head; (b H + h) / grp = b H_k + h / grp
    // is the query/key row of value head h
    const int kbh = bh / grp;
    const TIO *qp = q + (size_t)kbh * DK;
    const TIO *kp = k + (size_t)kbh * DK;
    const f32x4 k0 = load4(kp + c0), k1 = load4(kp + c1);
    const f32x4 q0 = load4(qp + c0), q1 = load4(qp + c1);
    const float vv = to_f32(v[(size_t)bh * d_v + row]);
    const float b = beta[bh];
    float alpha = 1.0f;                        // scalar gate; folded into s with PERCH
    if constexpr (PERCH) {
        const f32x4 g0 = load4(g + (size_t)bh * DK + c0), g1 = load4(g + (size_t)bh * DK + c1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s0[e] *= __expf(g0[e]);
            s1[e] *= __expf(g1[e]);
        }
    } else {
        alpha = __expf(g[bh]);
    }

    float kq = k0[0] * q0[0] + k0[1] * q0[1] + k0[2] * q0[2] + k0[3] * q0[3]
             + k1[0] * q1[0] + k1[1] * q1[1] + k1[2] * q1[2] + k1[3] * q1[3];
    float sk = s0[0] * k0[0] + s0[1] * k0[1] + s0[2] * k0[2] + s0[3] * k0[3]
             + s1[0] * k1[0] + s1[1] * k1[1] + s1[2] * k1[2] + s1[3] * k1[3];
    float sq = s0[0] * q0[0] + s0[1] * q0[1] + s0[2] * q0[2] + s0[3] * q0[3]
             + s1[0] * q1[0] + s1[1] * q1[1] + s1[2] * q1[2] + s1[3] * q1[3];
    kq = group_sum<G>(kq);
    sk = group_sum<G>(sk);
    sq = group_sum<G>(sq);
    const float delta = b * (vv - alpha * sk);
    f32x4 n0, n1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        n0[e] = alpha * s0[e] + delta * k0[e];
        n1[e] = alpha * s1[e] + delta * k1[e];
    }
    __builtin_nontemporal_store(n0, reinterpret_cast<f32x4 *>(rp + c0));
    __builtin_nontemporal_store(n1, reinterpret_cast<f32x4 *>(rp + c1));
    if (lr == 0) o[(size_t)bh * d_v + row] = from_f32<TIO>(scale * (alpha * sq + delta * kq));
}

template <int DK, typename TIO>
static hipError_t launch_decode_dk(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, float *state, void *o, int B, int H,
                                   int Hk, int d_v, float scale, bool per_channel,
                                   hipStream_t stream)
{
    constexpr int RPW = DEC_NT / (DK / 8);
    const int wg_per_head = (d_v + RPW - 1) / RPW;
    dim3 grid((unsigned)((long)B * H * wg_per_head)), block(DEC_NT);
    auto kern = per_channel ? decode_step_kernel<DK, TIO, true> : decode_step_kernel<DK, TIO, false>;
    hipLaunchKernelGGL(kern, grid, block, 0, stream,
                       (const TIO *)q, (const TIO *)k, (const TIO *)v, g, beta, state,
                       (TIO *)o, H / Hk, d_v, wg_per_head, scale);
    return hipGetLastError();
}

template <typename TIO>
hipError_t launch_decode(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, float *state, void *o, int B, int H, int Hk,
                         int d_k, int d_v, float scale, bool per_channel, hipStream_t stream)
{
    switch (d_k) {
    case 16: return launch_decode_dk<16, TIO>(q, k, v, g, beta, state, o, B, H, Hk, d_v, scale, per_channel, stream);
    case 32: return launch_decode_dk<32, TIO>(q, k, v, g, beta, state, o, B, H, Hk, d_v, scale, per_channel, stream);
    case 64: return launch_decode_dk<64, TIO>(q, k, v, g, beta, state, o, B, H, Hk, d_v, scale, per_channel, stream);
    case 128: return launch_decode_dk<128, TIO>(q, k, v, g, beta, state, o, B, H, Hk, d_v, scale, per_channel, stream);
    default: return hipErrorInvalidValue;
    }
}

template hipError_t launch_decode<float>(const void *, const void *, const void *, const float *,
                                         const float *, float *, void *, int, int, int, int,
                                         int, float, bool, hipStream_t);
template hipError_t launch_decode<bf16>(const void *, const void *, const void *, const float *,
                                        const float *, float *, void *, int, int, int, int,
                                        int, float, bool, hipStream_t);

}  // namespace gdn
