// gdn_api.hip - the extern "C" entry points of libgdn: argument validation,
// choice of kernel, launch on the caller's stream. No device memory is
// allocated and no state is kept between calls.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "gdn.h"
#include "common.h"
#include "launch.h"

namespace {

bool head_dim_pow2(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool mixer_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }
bool valid_dtype(int dt) { return dt == GDN_DTYPE_F32 || dt == GDN_DTYPE_BF16; }
int status_of(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

// Value heads H, query/key heads H_k: each query/key head serves H / H_k
// consecutive value heads.
bool heads_ok(int H, int Hk) { return H >= 1 && Hk >= 1 && Hk <= H && H % Hk == 0; }

// Shared validation of the prefill arguments.
int check_prefill(const void *q, const void *k, const void *v, const float *g, const float *beta,
                  const void *o, const int32_t *cu, int B, int T, int H, int Hk, int d_k,
                  int d_v, int N, int dtype)
{
    // with no tokens at all the activation pointers are never dereferenced
    const bool no_tokens = (int64_t)B * T == 0;
    if (!no_tokens && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
    if (!valid_dtype(dtype)) return GDN_ERR_DTYPE;
    if (B < 1 || T < 0 || H < 1 || N < 1 || d_k < 1 || d_v < 1) return GDN_ERR_SHAPE;
    if (!heads_ok(H, Hk)) return GDN_ERR_SHAPE;
    if (cu ? B != 1 : N != B) return GDN_ERR_SHAPE;
    if ((int64_t)B * T > (int64_t)INT32_MAX) return GDN_ERR_SHAPE;   // token index fits int32
    if (H > 65535 || N > 65535) return GDN_ERR_UNSUPPORTED;           // launch grid y / z
    if ((int64_t)H * N * 4 > (int64_t)INT32_MAX) return GDN_ERR_UNSUPPORTED;  // 1-D grid
    if (!head_dim_pow2(d_k) || d_v > 128) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

// bf16 with d_k = d_v = 128 runs on the MFMA chunk kernels
bool chunk_path(int dtype, int d_k, int d_v) {
    return dtype == GDN_DTYPE_BF16 && d_k == 128 && d_v == 128;
}

// the two-pass kernels index (chunk slot, head) items with 32-bit integers
// the prep passes' (chunk slot, head) items, slots rounded up to groups of 8,
// and a margin for their grid strides fit 32-bit indices
bool items_fit(int64_t tokens, int H, int64_t N) {
    return ((tokens / 64 + N + 1) + 7) / 8 * 8 * H + ((int64_t)1 << 20) <= (int64_t)INT32_MAX;
}

// a caller's workspace for the two-pass chunk path: 256-byte aligned, large enough
bool workspace_ok(const void *ws, size_t bytes, int B, int T, int H, int N,
                  bool per_channel = false) {
    return (reinterpret_cast<uintptr_t>(ws) & 255) == 0 &&
           bytes >= gdn::prefill_split_workspace_bytes((long)B * T, H, N, per_channel);
}

}  // namespace

// ---- scratch of gdn_prefill_noalloc -----------------------------------------
// A file-scope device array: every GPU the library runs on holds its own copy
// (zero-initialised when the code object is loaded) until the process ends.
// In host code `gdn_noalloc_scratch` names a host-side stand-in, not device
// memory: its device address is looked up once per device with
// hipGetSymbolAddress (the device current at the time) and only that address
// is handed to kernels.
static __device__ __attribute__((aligned(256))) unsigned char
    gdn_noalloc_scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int NOALLOC_MAX_DEVICES = 64;
std::atomic<void *> noalloc_addr[NOALLOC_MAX_DEVICES];

// Device address of the current device's scratch (looked up on the first call
// on that device; concurrent first calls store the same address).
hipError_t noalloc_scratch(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hipErrorInvalidDevice;
    void *p = noalloc_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(gdn_noalloc_scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        noalloc_addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}
}  // namespace

extern "C" {

int gdn_version(void) { return GDN_VERSION; }

const char *gdn_status_string(int status)
{
    switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "a required pointer is NULL";
    case GDN_ERR_SHAPE: return "invalid or inconsistent sizes";
    case GDN_ERR_DTYPE: return "unknown dtype";
    case GDN_ERR_UNSUPPORTED: return "valid arguments, but this size or mode is not implemented";
    case GDN_ERR_HIP: return "the HIP runtime reported an error at launch";
    case GDN_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case GDN_ERR_SCRATCH:
        return "the sizes need more scratch than gdn_prefill_noalloc's static buffer holds";
    default: return "unknown status";
    }
}

int gdn_check_cu_seqlens(const int32_t *cu, int N, int T)
{
    if (!cu) return GDN_ERR_NULL;
    if (N < 1 || T < 0 || cu[0] != 0 || cu[N] != T) return GDN_ERR_SHAPE;
    for (int n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n]) return GDN_ERR_SHAPE;
    return GDN_OK;
}

int gdn_prefill_recurrent(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *initial_state, float *final_state,
                          void *o, const int32_t *cu_seqlens, int B, int T, int H, int H_k,
                          int d_k, int d_v, int N, float scale, int dtype, void *stream)
{
    int st = check_prefill(q, k, v, g, beta, o, cu_seqlens, B, T, H, H_k, d_k, d_v, N, dtype);
    if (st != GDN_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = dtype == GDN_DTYPE_BF16
        ? gdn::launch_prefill_recurrent<gdn::bf16>(q, k, v, g, beta, initial_state, final_state, o,
                                                   cu_seqlens, T, H, H_k, d_k, d_v, N, scale,
                                                   false, s)
        : gdn::launch_prefill_recurrent<float>(q, k, v, g, beta, initial_state, final_state, o,
                                               cu_seqlens, T, H, H_k, d_k, d_v, N, scale, false,
                                               s);
    return status_of(e);
}

int gdn_prefill_workspace_size(int B, int T, int H, int d_k, int d_v, int N, int varlen,
                               int dtype, size_t *bytes)
{
    if (!bytes) return GDN_ERR_NULL;
    *bytes = 0;
    // the pointer checks of gdn_prefill do not apply here: pass stand-ins
    const int32_t *cu = varlen ? reinterpret_cast<const int32_t *>(bytes) : nullptr;
    const void *p = bytes;
    const int st = check_prefill(p, p, p, (const float *)p, (const float *)p, p, cu, B, T, H,
                                 H, d_k, d_v, N, dtype);
    if (st != GDN_OK) return st;
    if (chunk_path(dtype, d_k, d_v)) {
        if (!items_fit((int64_t)B * T, H, N)) return GDN_ERR_UNSUPPORTED;
        *bytes = gdn::prefill_split_workspace_bytes((long)B * T, H, N);
    }
    return GDN_OK;
}

int gdn_prefill(const void *q, const void *k, const void *v, const float *g, const float *beta,
                const float *initial_state, float *final_state, void *o,
                const int32_t *cu_seqlens, int B, int T, int H, int H_k, int d_k, int d_v,
                int N, float scale, int dtype, void *workspace, size_t workspace_bytes,
                void *stream)
{
    int st = check_prefill(q, k, v, g, beta, o, cu_seqlens, B, T, H, H_k, d_k, d_v, N, dtype);
    if (st != GDN_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (chunk_path(dtype, d_k, d_v)) {
        if (!workspace)
            return status_of(gdn::launch_prefill_fused(q, k, v, g, beta, initial_state,
                                                       final_state, o, cu_seqlens, T, H, H_k,
                                                       N, scale, s));
        if (!items_fit((int64_t)B * T, H, N)) return GDN_ERR_UNSUPPORTED;
        if (!workspace_ok(workspace, workspace_bytes, B, T, H, N)) return GDN_ERR_WORKSPACE;
        hipError_t e = gdn::launch_prefill_prepare(q, k, g, beta, cu_seqlens, T, H, H_k, N,
                                                   workspace, s);
        if (e == hipSuccess)
            e = gdn::launch_prefill_apply(q, k, v, g, initial_state, final_state, o, cu_seqlens,
                                          T, H, H_k, N, scale, workspace, s);
        return status_of(e);
    }
    return gdn_prefill_recurrent(q, k, v, g, beta, initial_state, final_state, o, cu_seqlens, B,
                                 T, H, H_k, d_k, d_v, N, scale, dtype, stream);
}

int gdn_prefill_noalloc(const void *q, const void *k, const void *v, const float *g,
                        const float *beta, const float *initial_state, float *final_state,
                        void *o, const int32_t *cu_seqlens, int B, int T, int H, int H_k,
                        int d_k, int d_v, int N, float scale, int dtype, void *stream)
{
    int st = check_prefill(q, k, v, g, beta, o, cu_seqlens, B, T, H, H_k, d_k, d_v, N, dtype);
    if (st != GDN_OK) return st;
    if (!chunk_path(dtype, d_k, d_v))          // the token-serial path needs no scratch
        return gdn_prefill_recurrent(q, k, v, g, beta, initial_state, final_state, o,
                                     cu_seqlens, B, T, H, H_k, d_k, d_v, N, scale, dtype, stream);
    if (gdn::prefill_split_workspace_bytes((long)B * T, H, N) > GDN_NOALLOC_SCRATCH_BYTES)
        return GDN_ERR_SCRATCH;
    void *ws = nullptr;
    hipError_t e = noalloc_scratch(&ws);
    if (e != hipSuccess) return GDN_ERR_HIP;
    hipStream_t s = (hipStream_t)stream;
    e = gdn::launch_prefill_prepare(q, k, g, beta, cu_seqlens, T, H, H_k, N, ws, s);
    if (e == hipSuccess)
        e = gdn::launch_prefill_apply(q, k, v, g, initial_state, final_state, o, cu_seqlens, T, H,
                                      H_k, N, scale, ws, s);
    return status_of(e);
}

int gdn_prefill_prepare(const void *q, const void *k, const float *g, const float *beta,
                        const int32_t *cu_seqlens, int B, int T, int H, int H_k, int d_k,
                        int d_v, int N, int dtype, void *workspace, size_t workspace_bytes,
                        void *stream)
{
    // v and o are not arguments of this pass: validate with stand-ins
    const void *p = workspace ? workspace : (const void *)k;
    int st = check_prefill(q, k, p, g, beta, p, cu_seqlens, B, T, H, H_k, d_k, d_v, N, dtype);
    if (st != GDN_OK) return st;
    if (!chunk_path(dtype, d_k, d_v) || !items_fit((int64_t)B * T, H, N))
        return GDN_ERR_UNSUPPORTED;
    if (!workspace) return GDN_ERR_NULL;
    if (!workspace_ok(workspace, workspace_bytes, B, T, H, N)) return GDN_ERR_WORKSPACE;
    return status_of(gdn::launch_prefill_prepare(q, k, g, beta, cu_seqlens, T, H, H_k, N,
                                                 workspace, (hipStream_t)stream));
}

int gdn_prefill_apply(const void *q, const void *k, const void *v, const float *g,
                      const float *initial_state, float *final_state, void *o,
                      const int32_t *cu_seqlens, int B, int T, int H, int H_k, int d_k,
                      int d_v, int N, float scale, int dtype, const void *workspace,
                      size_t workspace_bytes, void *stream)
{
    // beta is folded into the workspace: validate with a stand-in
    const float *pb = workspace ? (const float *)workspace : g;
    int st = check_prefill(q, k, v, g, pb, o, cu_seqlens, B, T, H, H_k, d_k, d_v, N, dtype);
    if (st != GDN_OK) return st;
    if (!chunk_path(dtype, d_k, d_v) || !items_fit((int64_t)B * T, H, N))
        return GDN_ERR_UNSUPPORTED;
    if (!workspace) return GDN_ERR_NULL;
    if (!workspace_ok(workspace, workspace_bytes, B, T, H, N)) return GDN_ERR_WORKSPACE;
    return status_of(gdn::launch_prefill_apply(q, k, v, g, initial_state, final_state, o,
                                               cu_seqlens, T, H, H_k, N, scale, workspace,
                                               (hipStream_t)stream));
}

int gdn_decode_step(const void *q, const void *k, const void *v, const float *g,
                    const float *beta, float *state, void *o, int B, int H, int H_k, int d_k,
                    int d_v, float scale, int dtype, void *stream)
{
    if (!q || !k || !v || !g || !beta || !state || !o) return GDN_ERR_NULL;
    if (!valid_dtype(dtype)) return GDN_ERR_DTYPE;
    if (B < 1 || H < 1 || d_k < 1 || d_v < 1 || !heads_ok(H, H_k)) return GDN_ERR_SHAPE;
    if ((int64_t)B * H > (int64_t)INT32_MAX) return GDN_ERR_SHAPE;
    if (!head_dim_pow2(d_k) || d_v > 4096) return GDN_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = dtype == GDN_DTYPE_BF16
        ? gdn::launch_decode<gdn::bf16>(q, k, v, g, beta, state, o, B, H, H_k, d_k, d_v, scale,
                                        false, s)
        : gdn::launch_decode<float>(q, k, v, g, beta, state, o, B, H, H_k, d_k, d_v, scale, false,
                                    s);
    return status_of(e);
}

int gdn_mixer_prologue(const void *q_raw, const void *k_raw, const void *v_raw,
                       const void *conv_w, const void *a, const void *b, const float *A,
                       const float *dt_bias, const int32_t *cu_seqlens, void *q, void *k,
                       void *v, float *g, float *beta, int B, int T, int H, int H_k, int d_k,
                       int d_v, int N, int dtype, void *stream)
{
    if (!q_raw || !k_raw || !v_raw || !conv_w || !a || !b || !A || !q || !k || !v || !g || !beta)
        return GDN_ERR_NULL;
    if (!valid_dtype(dtype)) return GDN_ERR_DTYPE;
    if (B < 1 || T < 0 || H < 1 || N < 1 || d_k < 1 || d_v < 1) return GDN_ERR_SHAPE;
    if (!heads_ok(H, H_k)) return GDN_ERR_SHAPE;
    if (cu_seqlens ? B != 1 : N != B) return GDN_ERR_SHAPE;
    if ((int64_t)B * T > (int64_t)INT32_MAX) return GDN_ERR_SHAPE;
    if (H > 65535) return GDN_ERR_UNSUPPORTED;                        // launch grid y
    if (!mixer_dim(d_k) || !mixer_dim(d_v)) return GDN_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = dtype == GDN_DTYPE_BF16
        ? gdn::launch_prologue<gdn::bf16>(q_raw, k_raw, v_raw, conv_w, a, b, A, dt_bias, cu_seqlens,
                                          q, k, v, g, beta, B, T, H, H_k, d_k, d_v, N, s)
        : gdn::launch_prologue<float>(q_raw, k_raw, v_raw, conv_w, a, b, A, dt_bias, cu_seqlens, q,
                                      k, v, g, beta, B, T, H, H_k, d_k, d_v, N, s);
    return status_of(e);
}

int gdn_mixer_epilogue(const void *y, const void *z, const float *norm_w, void *out, int rows,
                       int H, int d_v, float eps, int dtype, void *stream)
{
    if (!y || !z || !out) return GDN_ERR_NULL;
    if (!valid_dtype(dtype)) return GDN_ERR_DTYPE;
    if (rows < 0 || H < 1 || d_v < 1 || !(eps >= 0.0f)) return GDN_ERR_SHAPE;
    if (!mixer_dim(d_v)) return GDN_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    const long r = (long)rows * H;
    hipError_t e = dtype == GDN_DTYPE_BF16
        ? gdn::launch_epilogue<gdn::bf16>(y, z, norm_w, out, r, d_v, eps, s)
        : gdn::launch_epilogue<float>(y, z, norm_w, out, r, d_v, eps, s);
    return status_of(e);
}

int gdn_decode_mixer_step(const void *q_raw, const void *k_raw, const void *v_raw,
                          const void *conv_w, void *conv_state, const void *a, const void *b,
                          const float *A, const float *dt_bias, const void *z,
                          const float *norm_w, float eps, float *state, void *out, int B, int H,
                          int H_k, int d_k, int d_v, float scale, int dtype, void *stream)
{
    if (!q_raw || !k_raw || !v_raw || !conv_w || !conv_state || !a || !b || !A || !z || !state ||
        !out)
        return GDN_ERR_NULL;
    if (!valid_dtype(dtype)) return GDN_ERR_DTYPE;
    if (B < 1 || d_k < 1 || d_v < 1 || !heads_ok(H, H_k) || !(eps >= 0.0f)) return GDN_ERR_SHAPE;
    if ((int64_t)B * H > (int64_t)INT32_MAX) return GDN_ERR_SHAPE;
    if (!head_dim_pow2(d_k) || !mixer_dim(d_v)) return GDN_ERR_UNSUPPORTED;
    if ((int64_t)(H / H_k) * d_v > gdn::DECODE_MIXER_MAX_ROWS) return GDN_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = dtype == GDN_DTYPE_BF16
        ? gdn::launch_decode_mixer<gdn::bf16>(q_raw, k_raw, v_raw, conv_w, conv_state, a, b, A,
                                              dt_bias, z, norm_w, eps, state, out, B, H, H_k,
                                              d_k, d_v, scale, s)
        : gdn::launch_decode_mixer<float>(q_raw, k_raw, v_raw, conv_w, conv_state, a, b, A,
                                          dt_bias, z, norm_w, eps, state, out, B, H, H_k, d_k,
                                          d_v, scale, s);
    return status_of(e);
}

int gdn_prefill_channel_workspace_size(int B, int T, int H, int d_k, int d_v, int N, int varlen,
                                       int dtype, size_t *bytes)
{
    if (!bytes) return GDN_ERR_NULL;
    *bytes = 0;
    const int32_t *cu = varlen ? reinterpret_cast<const int32_t *>(bytes) : nullptr;
    const void *p = bytes;
    const int st = check_prefill(p, p, p, (const float *)p, (const float *)p, p, cu, B, T, H,
                                 H, d_k, d_v, N, dtype);
    if (st != GDN_OK) return st;
    if (chunk_path(dtype, d_k, d_v)) {
        if (!items_fit((int64_t)B * T, H, N)) return GDN_ERR_UNSUPPORTED;
        *bytes = gdn::prefill_split_workspace_bytes((long)B * T, H, N, true);
    }
    return GDN_OK;
}

int gdn_prefill_channel_gated(const void *q, const void *k, const void *v, const float *g,
                              const float *beta, const float *initial_state, float *final_state,
                              void *o, const int32_t *cu_seqlens, int B, int T, int H, int H_k,
                              int d_k, int d_v, int N, float scale, int dtype, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    int st = check_prefill(q, k, v, g, beta, o, cu_seqlens, B, T, H, H_k, d_k, d_v, N, dtype);
    if (st != GDN_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (workspace && chunk_path(dtype, d_k, d_v)) {
        if (!items_fit((int64_t)B * T, H, N)) return GDN_ERR_UNSUPPORTED;
        if (!workspace_ok(workspace, workspace_bytes, B, T, H, N, true)) return GDN_ERR_WORKSPACE;
        hipError_t e = gdn::launch_prefill_prepare(q, k, g, beta, cu_seqlens, T, H, H_k, N,
                                                   workspace, s, true);
        if (e == hipSuccess)
            e = gdn::launch_prefill_apply(q, k, v, g, initial_state, final_state, o, cu_seqlens,
                                          T, H, H_k, N, scale, workspace, s, 0, true);
        return status_of(e);
    }
    hipError_t e = dtype == GDN_DTYPE_BF16
        ? gdn::launch_prefill_recurrent<gdn::bf16>(q, k, v, g, beta, initial_state, final_state, o,
                                                   cu_seqlens, T, H, H_k, d_k, d_v, N, scale,
                                                   true, s)
        : gdn::launch_prefill_recurrent<float>(q, k, v, g, beta, initial_state, final_state, o,
                                               cu_seqlens, T, H, H_k, d_k, d_v, N, scale, true,
                                               s);
    return status_of(e);
}

int gdn_decode_step_channel_gated(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, float *state, void *o, int B, int H,
                                  int H_k, int d_k, int d_v, float scale, int dtype, void *stream)
{
    if (!q || !k || !v || !g || !beta || !state || !o) return GDN_ERR_NULL;
    if (!valid_dtype(dtype)) return GDN_ERR_DTYPE;
    if (B < 1 || H < 1 || d_k < 1 || d_v < 1 || !heads_ok(H, H_k)) return GDN_ERR_SHAPE;
    if ((int64_t)B * H > (int64_t)INT32_MAX) return GDN_ERR_SHAPE;
    if (!head_dim_pow2(d_k) || d_v > 4096) return GDN_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = dtype == GDN_DTYPE_BF16
        ? gdn::launch_decode<gdn::bf16>(q, k, v, g, beta, state, o, B, H, H_k, d_k, d_v, scale,
                                        true, s)
        : gdn::launch_decode<float>(q, k, v, g, beta, state, o, B, H, H_k, d_k, d_v, scale, true,
                                    s);
    return status_of(e);
}

// Shared validation of the sequence-parallel prefill's arguments: those of
// gdn_prefill, on the MFMA chunk path only, and the segment count.
static int check_seqpar(const void *q, const void *k, const void *v, const float *g,
                        const float *beta, const void *o, const int32_t *cu, int B, int T, int H,
                        int H_k, int d_k, int d_v, int N, int segments, int dtype)
{
    const int st = check_prefill(q, k, v, g, beta, o, cu, B, T, H, H_k, d_k, d_v, N, dtype);
    if (st != GDN_OK) return st;
    if (segments < 1) return GDN_ERR_SHAPE;
    if (!chunk_path(dtype, d_k, d_v)) return GDN_ERR_UNSUPPORTED;
    // segments (N * segments) index the 1-D chain grid of pass 1: 2 jobs per
    // segment, H pairs per job, 4 workgroups per pair
    if ((int64_t)N * segments > 65535) return GDN_ERR_UNSUPPORTED;
    if ((int64_t)N * segments * H * 8 > (int64_t)INT32_MAX) return GDN_ERR_UNSUPPORTED;
    if (!items_fit((int64_t)B * T, H, (int64_t)N * segments)) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

int gdn_prefill_seqpar_workspace_size(int B, int T, int H, int d_k, int d_v, int N, int varlen,
                                      int segments, int dtype, size_t *bytes)
{
    if (!bytes) return GDN_ERR_NULL;
    *bytes = 0;
    // the pointer checks of gdn_prefill_seqpar do not apply here: pass stand-ins
    const int32_t *cu = varlen ? reinterpret_cast<const int32_t *>(bytes) : nullptr;
    const void *p = bytes;
    const int st = check_seqpar(p, p, p, (const float *)p, (const float *)p, p, cu, B, T, H, H,
                                d_k, d_v, N, segments, dtype);
    if (st != GDN_OK) return st;
    *bytes = gdn::prefill_seqpar_workspace_bytes((int64_t)B * T, H, N, segments);
    return GDN_OK;
}

int gdn_prefill_seqpar(const void *q, const void *k, const void *v, const float *g,
                       const float *beta, const float *initial_state, float *final_state,
                       void *o, const int32_t *cu_seqlens, int B, int T, int H, int H_k,
                       int d_k, int d_v, int N, int segments, float scale, int dtype,
                       void *workspace, size_t workspace_bytes, void *stream)
{
    const int st = check_seqpar(q, k, v, g, beta, o, cu_seqlens, B, T, H, H_k, d_k, d_v, N,
                                segments, dtype);
    if (st != GDN_OK) return st;
    if (!workspace) return GDN_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0 ||
        workspace_bytes < gdn::prefill_seqpar_workspace_bytes((int64_t)B * T, H, N, segments))
        return GDN_ERR_WORKSPACE;
    return status_of(gdn::launch_prefill_seqpar(q, k, v, g, beta, initial_state, final_state, o,
                                                cu_seqlens, T, H, H_k, N, segments, scale,
                                                workspace, (hipStream_t)stream));
}

}  // extern "C"
