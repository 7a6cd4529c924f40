// common.h - device helpers shared by the gfx950 kernels of libgdn.
//
// Storage types, 16-byte vector types, bf16 <-> fp32 conversion, and
// cross-lane reductions built on DPP (data-parallel primitives of the CDNA
// vector ALU: a lane reads a neighbour's register in the same instruction,
// without going through LDS).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---- scalar conversions ---------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// ---- 4-element loads/stores of a storage type as fp32 ---------------------
// fp32: one 16-byte access; bf16: one 8-byte access.
__device__ __forceinline__ f32x4 load4(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
}
__device__ __forceinline__ f32x4 load4(const bf16 *p) {
    bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ void store4(float *p, f32x4 v) {
    *reinterpret_cast<f32x4 *>(p) = v;
}
__device__ __forceinline__ void store4(bf16 *p, f32x4 v) {
    bf16x4 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    *reinterpret_cast<bf16x4 *>(p) = o;
}

// 8 contiguous elements as fp32 (fp32: 2 x 16 B, bf16: 16 B).
__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
    f32x4 a = load4(p), b = load4(p + 4);
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}
__device__ __forceinline__ void load8(const bf16 *p, float (&x)[8]) {
    bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
}
__device__ __forceinline__ void store8(float *p, const float (&x)[8]) {
    store4(p, f32x4{x[0], x[1], x[2], x[3]});
    store4(p + 4, f32x4{x[4], x[5], x[6], x[7]});
}
__device__ __forceinline__ void store8(bf16 *p, const float (&x)[8]) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (bf16)x[i];
    *reinterpret_cast<bf16x8 *>(p) = v;
}

// ---- DPP cross-lane sums ----------------------------------------------------
// DPP control codes (CDNA ISA): quad_perm selectors, and the row mirrors
// that reverse lanes within a half row (8 lanes) or a row (16 lanes).
enum : int {
    DPP_QUAD_XOR1 = 0xB1,      // quad_perm [1,0,3,2]
    DPP_QUAD_XOR2 = 0x4E,      // quad_perm [2,3,0,1]
    DPP_ROW_HALF_MIRROR = 0x141,
    DPP_ROW_MIRROR = 0x140,
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G in 1, 2, 4, 8, 16, 32, 64); every lane
// of a group receives the group's sum. Groups up to 16 lanes stay inside one
// DPP row; 32 and 64 finish with LDS-free bpermute shuffles.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32 || G == 64,
                  "group size");
    if constexpr (G >= 2) x += dpp_f32<DPP_QUAD_XOR1>(x);
    if constexpr (G >= 4) x += dpp_f32<DPP_QUAD_XOR2>(x);
    if constexpr (G >= 8) x += dpp_f32<DPP_ROW_HALF_MIRROR>(x);
    if constexpr (G >= 16) x += dpp_f32<DPP_ROW_MIRROR>(x);
    if constexpr (G >= 32) x += __shfl_xor(x, 16, 64);
    if constexpr (G >= 64) x += __shfl_xor(x, 32, 64);
    return x;
}

// SiLU(x) = x * sigmoid(x) with the hardware exponential and reciprocal
// (v_exp_f32, v_rcp_f32, about 1 ulp each) instead of an IEEE division: the
// elementwise stages are bound by memory, and a correctly rounded divide per
// channel costs them more than their loads. Large negative x gives
// exp(-x) = inf, rcp(inf) = 0 and -0, the limit.
__device__ __forceinline__ float silu_f32(float x) {
    return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}
// 1 / sqrt(x) for x > 0 by the hardware reciprocal square root (about 1 ulp).
__device__ __forceinline__ float rsqrt_f32(float x) { return __builtin_amdgcn_rsqf(x); }

// softplus(x) = log(1 + e^x), evaluated without overflow.
__device__ __forceinline__ float softplus_f32(float x) {
    return x > 0.0f ? x + log1pf(expf(-x)) : log1pf(expf(x));
}

}  // namespace gdn
