// launch.h - host-side launchers of libgdn's kernels, shared by the C-ABI
// layer (gdn_api.hip) and the files that define them. Each launcher checks
// nothing beyond what its kernels assume of the sizes, enqueues its kernels
// on `stream` and returns the launch status; the entry points in gdn_api.hip
// validate the caller's arguments first.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct SegJob;                                 // chunk_common.h

template <typename TIO>
hipError_t launch_decode(const void *, const void *, const void *, const float *, const float *,
                         float *, void *, int, int, int, int, int, float, bool, hipStream_t);
template <typename TIO>
hipError_t launch_prefill_recurrent(const void *, const void *, const void *, const float *,
                                    const float *, const float *, float *, void *,
                                    const int32_t *, int, int, int, int, int, int, float, bool,
                                    hipStream_t);

// Two-pass chunk path (prefill_split.hip). T is the packed token count when
// cu is given, else the tokens per sequence; N the sequences (or segments).
hipError_t launch_prefill_prepare(const void *q, const void *k, const float *g,
                                  const float *beta, const int32_t *cu, int T, int H, int Hk,
                                  int N, void *ws, hipStream_t stream, bool per_channel = false);
hipError_t launch_prefill_apply(const void *q, const void *k, const void *v, const float *g,
                                const float *s_init, float *s_final, void *o, const int32_t *cu,
                                int T, int H, int Hk, int N, float scale, const void *ws,
                                hipStream_t stream, int flags = 0, bool per_channel = false,
                                const SegJob *jobs = nullptr, int njobs = 0);
size_t prefill_split_workspace_bytes(long tokens, int H, int N, bool per_channel = false);
// One pass that also solves each chunk's triangular system on the way (scalar
// gates); same arguments as the apply pass, no workspace.
hipError_t launch_prefill_fused(const void *q, const void *k, const void *v, const float *g,
                                const float *beta, const float *s_init, float *s_final, void *o,
                                const int32_t *cu, int T, int H, int Hk, int N, float scale,
                                hipStream_t stream, int flags = 0, const SegJob *jobs = nullptr,
                                int njobs = 0);

// Sequence-parallel prefill (seqpar.hip): N sequences (packed by cu, or N
// rows of T tokens), the longest cut into P segments.
size_t prefill_seqpar_workspace_bytes(long tokens, int H, int N, int P);
hipError_t launch_prefill_seqpar(const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *s_init, float *s_final, void *o,
                                 const int32_t *cu, int T, int H, int Hk, int N, int P,
                                 float scale, void *ws, hipStream_t stream);

template <typename TIO>
hipError_t launch_prologue(const void *, const void *, const void *, const void *, const void *,
                           const void *, const float *, const float *, const int32_t *, void *,
                           void *, void *, float *, float *, int, int, int, int, int, int, int,
                           hipStream_t);
template <typename TIO>
hipError_t launch_decode_mixer(const void *, const void *, const void *, const void *, void *,
                               const void *, const void *, const float *, const float *,
                               const void *, const float *, float, float *, void *, int, int,
                               int, int, int, float, hipStream_t);
constexpr int DECODE_MIXER_MAX_ROWS = 4096;
template <typename TIO>
hipError_t launch_epilogue(const void *, const void *, const float *, void *, long, int, float,
                           hipStream_t);

}  // namespace gdn
