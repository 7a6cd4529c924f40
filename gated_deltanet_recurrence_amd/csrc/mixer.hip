// mixer.hip - the elementwise stages around the recurrence: the prologue
// (causal conv1d + SiLU, L2-norm of q and k, gates) and the epilogue (gated
// RMSNorm). Both are HBM-bound streaming kernels.
//
// Sources:
//  "5. Linear Attention" (LinkQwen ch. 5): section "Causal Conv1d"
//   (depthwise, 4 taps, left zero padding, no bias, followed by SiLU);
//   section "Gated RMSNorm" (weight * x * rsqrt(mean(x^2) + eps) * silu(z));
//   the layer body (conv -> split q/k/v -> gates -> core -> gated norm).
//  "6.6 Gated DeltaNet (linear attention)", LLM full-stack book: section
//   6.6.3 (alpha = exp(-A * softplus(.)), beta = sigmoid(.)) and the l2norm
//   of section 6.6.4 (eps 1e-6 added to the sum of squares).
//
// Grouped heads: q and k have H_k heads, v, z, the gates and the output H
// (the conv channels are H_k d_k of q, H_k d_k of k, then H d_v of v, as the
// layer code of "5. Linear Attention" orders them); the gates are per value
// head and are computed by the v lane groups.
//
// Work mapping (both kernels): one (token, head) row of D channels is owned
// by G = D/8 lanes, 8 channels (16 B of bf16) per lane, so row reductions are
// DPP sums inside the group. In the prologue the lane groups of a workgroup
// take consecutive heads of one tensor (so a workgroup streams whole token
// rows) and each group walks a tile of TT
// consecutive tokens of one head of one tensor and keeps the three previous
// inputs of its channels in registers (the convolution window), so every
// input element is read from HBM once (plus three tokens of history per
// tile); the tile's loads are all issued before its first token is computed.
#include "common.h"
#include "launch.h"

namespace gdn {

constexpr int PRO_TT = 8;          // tokens per lane group in the prologue

// Eight consecutive elements of a storage type as loaded (16 B of bf16, 32 B
// of fp32), converted to fp32 only where they are used, so that a lane can
// keep many tokens' loads in flight in few registers.
template <typename TIO> struct Raw8;
template <> struct Raw8<bf16> {
    bf16x8 v;
    __device__ __forceinline__ void load(const bf16 *p) { v = *reinterpret_cast<const bf16x8 *>(p); }
    __device__ __forceinline__ void get(float (&x)[8]) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
    }
};
template <> struct Raw8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float *p) { a = load4(p); b = load4(p + 4); }
    __device__ __forceinline__ void get(float (&x)[8]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
    }
};

// Sequence of global token t: [start, end). cu == nullptr: rows of T tokens.
__device__ __forceinline__ void seq_bounds(const int32_t *cu, int N, long T, long t, long &start,
                                           long &end, int &n)
{
    if (!cu) {
        n = (int)(t / T);
        start = (long)n * T;
        end = start + T;
        return;
    }
    // largest n with cu[n] <= t (offsets clamped into [0, T], non-decreasing)
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        long c = cu[mid];
        if (c <= t) lo = mid; else hi = mid - 1;
    }
    n = lo;
    start = cu[lo];
    end = cu[lo + 1];
    if (start < 0) start = 0;
    if (end > T) end = T;
}

template <int D, typename TIO>
__global__ void __launch_bounds__(256)
prologue_conv_kernel(const TIO *__restrict__ x_q, const TIO *__restrict__ x_k,
                     const TIO *__restrict__ x_v, const TIO *__restrict__ conv_w,
                     TIO *__restrict__ y_q, TIO *__restrict__ y_k, TIO *__restrict__ y_v,
                     const TIO *__restrict__ a, const TIO *__restrict__ b,
                     const float *__restrict__ A, const float *__restrict__ dt_bias,
                     float *__restrict__ g, float *__restrict__ beta,
                     const int32_t *__restrict__ cu, long total, long T, int N, int H,
                     int Hk, int d_k, int which0)
{
    constexpr int G = D / 8;
    constexpr int GPB = 256 / G;                  // lane groups per block
    const int which = which0 + (int)blockIdx.z;   // 0 = q, 1 = k, 2 = v
    const int Ht0 = which < 2 ? Hk : H;
    // the lane groups of a workgroup take consecutive heads of one token tile,
    // so that together they stream whole token rows
    const int h = (int)blockIdx.y * GPB + (int)threadIdx.x / G;   // head of this tensor
    if (h >= Ht0) return;                         // whole lane groups
    const int Ht = Ht0;                           // heads of this tensor
    const int lr = threadIdx.x % G;
    // tiles dealt so that a tile and the one before it run on the same XCD
    // (workgroups go to the 8 XCDs in turn): the previous tile's last three
    // tokens, this tile's convolution history, are then read from that XCD's L2
    const long nb = (long)gridDim.x, full = nb / 8 * 8, bx = (long)blockIdx.x;
    const long tile = bx < full ? (bx % 8) * (nb / 8) + bx / 8 : bx;
    const long t0 = tile * PRO_TT;
    const long t1 = t0 + PRO_TT < total ? t0 + PRO_TT : total;

    const TIO *x = which == 0 ? x_q : (which == 1 ? x_k : x_v);
    TIO *y = which == 0 ? y_q : (which == 1 ? y_k : y_v);
    const int c = 8 * lr;
    // conv channel of (tensor, head, c): q channels, then k, then v
    const long ch = (long)which * Hk * d_k + (long)h * D + c;
    // the 4 taps of this lane's 8 channels are 32 consecutive weights: four
    // 8-element loads, kept as loaded
    float w[4][8];                                // w[u][8 r + j]: channel 2 u + r, tap j
    {
        Raw8<TIO> wr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) wr[i].load(conv_w + ch * 4 + 8 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i) wr[i].get(w[i]);
    }

    long start, end;
    int n;
    seq_bounds(cu, N, T, t0, start, end, n);

    auto row = [&](long t) { return ((size_t)t * Ht + h) * D + c; };
    // the three inputs before the tile (taken as zero before the sequence
    // start), then the tile's inputs: all requested, without branches (rows
    // out of range are read at a valid row and not used), before any is used
    Raw8<TIO> hr[3];
    bool hok[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        hok[j] = t0 - 1 - j >= start;
        hr[j].load(x + row(hok[j] ? t0 - 1 - j : t0));
    }
    Raw8<TIO> xr[PRO_TT];
#pragma unroll
    for (int i = 0; i < PRO_TT; ++i) xr[i].load(x + row(t0 + i < t1 ? t0 + i : t1 - 1));

    if (which == 2) {
        // the gates of the tile's (token, value head) pairs, spread over the
        // threads of the lane groups that have a head (the first nh groups),
        // their loads issued together behind the tile's
        const int hb = (int)blockIdx.y * GPB;
        const int nh = H - hb < GPB ? H - hb : GPB;
        for (int e = (int)threadIdx.x; e < PRO_TT * nh; e += nh * G) {
            const long t = t0 + e / nh;
            const int hh = hb + e % nh;
            if (t < t1) {
                const size_t i = (size_t)t * H + hh;
                const float bias = dt_bias ? dt_bias[hh] : 0.f;
                g[i] = -A[hh] * softplus_f32(to_f32(a[i]) + bias);
                beta[i] = 1.0f / (1.0f + expf(-to_f32(b[i])));
            }
        }
    }
    float x1[8], x2[8], x3[8];                    // inputs at t-1, t-2, t-3
    hr[0].get(x1);
    hr[1].get(x2);
    hr[2].get(x3);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x1[e] = hok[0] ? x1[e] : 0.f;
        x2[e] = hok[1] ? x2[e] : 0.f;
        x3[e] = hok[2] ? x3[e] : 0.f;
    }

#pragma unroll
    for (int i = 0; i < PRO_TT; ++i) {
        const long t = t0 + i;
        if (t >= t1) break;                       // uniform across the lane group
        while (t >= end && n < N - 1) {           // crossed into the next sequence
            ++n;
            start = end;
            end = cu ? (long)cu[n + 1] : start + T;
            if (end > T && cu) end = T;
#pragma unroll
            for (int e = 0; e < 8; ++e) { x1[e] = 0.f; x2[e] = 0.f; x3[e] = 0.f; }
        }
        float xt[8], out[8];
        xr[i].get(xt);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float *we = &w[e >> 1][4 * (e & 1)];      // taps 0..3 of channel e
            const float pre = we[3] * xt[e] + we[2] * x1[e] + we[1] * x2[e] + we[0] * x3[e];
            out[e] = silu_f32(pre);
            ss += out[e] * out[e];
        }
        if (which < 2) {                          // L2-norm of q and k rows
            ss = group_sum<G>(ss);
            const float inv = rsqrt_f32(ss + 1e-6f);
#pragma unroll
            for (int e = 0; e < 8; ++e) out[e] *= inv;
        }
        store8(y + row(t), out);
#pragma unroll
        for (int e = 0; e < 8; ++e) { x3[e] = x2[e]; x2[e] = x1[e]; x1[e] = xt[e]; }
    }
}

template <int D, typename TIO>
__global__ void __launch_bounds__(256)
epilogue_kernel(const TIO *y, const TIO *__restrict__ z, const float *__restrict__ w,
                TIO *out, long rows, float eps)
{
    constexpr int G = D / 8;
    constexpr int GPB = 256 / G;
    const int lr = threadIdx.x % G;
    const int c = 8 * lr;
    for (long r = (long)blockIdx.x * GPB + threadIdx.x / G; r < rows;
         r += (long)gridDim.x * GPB) {
        float yv[8], zv[8], ov[8], wv[8];
        load8(y + (size_t)r * D + c, yv);
        load8(z + (size_t)r * D + c, zv);
        // the weights after the row's loads, so that their latencies overlap
        // (a workgroup normally takes one row per lane group)
        if (w) load8(w + c, wv);
        else {
#pragma unroll
            for (int e = 0; e < 8; ++e) wv[e] = 1.0f;
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += yv[e] * yv[e];
        ss = group_sum<G>(ss);
        const float inv = rsqrt_f32(ss * (1.0f / D) + eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) ov[e] = wv[e] * (yv[e] * inv) * silu_f32(zv[e]);
        store8(out + (size_t)r * D + c, ov);
    }
}

template <int D, typename TIO>
static hipError_t launch_conv(const void *xq, const void *xk, const void *xv, const void *w,
                              void *yq, void *yk, void *yv, const void *a, const void *b,
                              const float *A, const float *dtb, float *g, float *beta,
                              const int32_t *cu, long total, long T, int N, int H, int Hk,
                              int d_k, int which0, int nwhich, hipStream_t stream)
{
    constexpr int GPB = 256 / (D / 8);
    const long tiles = (total + PRO_TT - 1) / PRO_TT;
    // heads of the widest tensor in the launch (lane groups past a tensor's
    // heads return at once)
    const int heads = which0 + nwhich > 2 ? (H > Hk ? H : Hk) : Hk;
    dim3 grid((unsigned)tiles, (unsigned)((heads + GPB - 1) / GPB), (unsigned)nwhich), block(256);
    hipLaunchKernelGGL((prologue_conv_kernel<D, TIO>), grid, block, 0, stream,
                       (const TIO *)xq, (const TIO *)xk, (const TIO *)xv, (const TIO *)w,
                       (TIO *)yq, (TIO *)yk, (TIO *)yv, (const TIO *)a, (const TIO *)b, A, dtb,
                       g, beta, cu, total, T, N, H, Hk, d_k, which0);
    return hipGetLastError();
}

template <typename TIO>
static hipError_t conv_dispatch(int D, const void *xq, const void *xk, const void *xv,
                                const void *w, void *yq, void *yk, void *yv, const void *a,
                                const void *b, const float *A, const float *dtb, float *g,
                                float *beta, const int32_t *cu, long total, long T, int N, int H,
                                int Hk, int d_k, int which0, int nwhich, hipStream_t s)
{
    switch (D) {
    case 16: return launch_conv<16, TIO>(xq, xk, xv, w, yq, yk, yv, a, b, A, dtb, g, beta, cu, total, T, N, H, Hk, d_k, which0, nwhich, s);
    case 32: return launch_conv<32, TIO>(xq, xk, xv, w, yq, yk, yv, a, b, A, dtb, g, beta, cu, total, T, N, H, Hk, d_k, which0, nwhich, s);
    case 64: return launch_conv<64, TIO>(xq, xk, xv, w, yq, yk, yv, a, b, A, dtb, g, beta, cu, total, T, N, H, Hk, d_k, which0, nwhich, s);
    case 128: return launch_conv<128, TIO>(xq, xk, xv, w, yq, yk, yv, a, b, A, dtb, g, beta, cu, total, T, N, H, Hk, d_k, which0, nwhich, s);
    case 256: return launch_conv<256, TIO>(xq, xk, xv, w, yq, yk, yv, a, b, A, dtb, g, beta, cu, total, T, N, H, Hk, d_k, which0, nwhich, s);
    default: return hipErrorInvalidValue;
    }
}

template <typename TIO>
hipError_t launch_prologue(const void *q_raw, const void *k_raw, const void *v_raw,
                           const void *conv_w, const void *a, const void *b, const float *A,
                           const float *dt_bias, const int32_t *cu, void *q, void *k, void *v,
                           float *g, float *beta, int B, int T, int H, int Hk, int d_k,
                           int d_v, int N, hipStream_t stream)
{
    const long total = (long)B * T;
    if (total == 0) return hipSuccess;
    // one launch for q, k and v when their head sizes agree (no gap between
    // two launches); else q and k share a launch and v has its own
    if (d_k == d_v)
        return conv_dispatch<TIO>(d_k, q_raw, k_raw, v_raw, conv_w, q, k, v, a, b, A, dt_bias,
                                  g, beta, cu, total, (long)T, N, H, Hk, d_k, 0, 3, stream);
    hipError_t e = conv_dispatch<TIO>(d_k, q_raw, k_raw, v_raw, conv_w, q, k, v, a, b, A, dt_bias,
                                      g, beta, cu, total, (long)T, N, H, Hk, d_k, 0, 2, stream);
    if (e != hipSuccess) return e;
    return conv_dispatch<TIO>(d_v, q_raw, k_raw, v_raw, conv_w, q, k, v, a, b, A, dt_bias, g,
                              beta, cu, total, (long)T, N, H, Hk, d_k, 2, 1, stream);
}

template <typename TIO>
hipError_t launch_epilogue(const void *y, const void *z, const float *w, void *out, long rows,
                           int d_v, float eps, hipStream_t stream)
{
    if (rows == 0) return hipSuccess;
    auto go = [&](auto kern, int gpb) {
        long blocks = (rows + gpb - 1) / gpb;
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, stream, (const TIO *)y,
                           (const TIO *)z, w, (TIO *)out, rows, eps);
        return hipGetLastError();
    };
    switch (d_v) {
    case 16: return go(epilogue_kernel<16, TIO>, 128);
    case 32: return go(epilogue_kernel<32, TIO>, 64);
    case 64: return go(epilogue_kernel<64, TIO>, 32);
    case 128: return go(epilogue_kernel<128, TIO>, 16);
    case 256: return go(epilogue_kernel<256, TIO>, 8);
    default: return hipErrorInvalidValue;
    }
}

template hipError_t launch_prologue<float>(const void *, const void *, const void *, const void *,
                                           const void *, const void *, const float *,
                                           const float *, const int32_t *, void *, void *, void *,
                                           float *, float *, int, int, int, int, int, int, int,
                                           hipStream_t);
template hipError_t launch_prologue<bf16>(const void *, const void *, const void *, const void *,
                                          const void *, const void *, const float *,
                                          const float *, const int32_t *, void *, void *, void *,
                                          float *, float *, int, int, int, int, int, int, int,
                                          hipStream_t);
template hipError_t launch_epilogue<float>(const void *, const void *, const float *, void *,
                                           long, int, float, hipStream_t);
template hipError_t launch_epilogue<bf16>(const void *, const void *, const float *, void *, long,
                                          int, float, hipStream_t);

}  // namespace gdn
