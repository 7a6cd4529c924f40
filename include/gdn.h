/*
 * gdn.h - C ABI of the MI355X (gfx950) Gated Delta Rule token-mixer library
 * (libgdn.so).
 *
 * The library computes the gated delta rule of
 *   "[LLM Algorithms-2] Gated DeltaNet: Teaching Linear Attention to
 *    Overwrite and Forget", section 4 (boxed update) and section 5:
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t
 *
 * with one state S of shape d_v x d_k per (sequence, head). The decay is
 * applied before the retrieval (section 4.3 of the same page) and the readout
 * uses the updated state.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer (memory from hipMalloc or a
 *    device allocator on the device current when the call is made). The
 *    caller owns and allocates every buffer; the library keeps no pointer
 *    after a call returns and allocates no device memory.
 *  - Activations are token-major and C-contiguous: q, k are [B][T][H_k][d_k];
 *    v, o are [B][T][H][d_v]; per-token scalars are [B][T][H].
 *  - Grouped heads: H counts the value heads (v, o, g, beta, states) and H_k
 *    the query/key heads, 1 <= H_k <= H with H divisible by H_k; value head h
 *    reads query/key head h / (H / H_k), i.e. q and k repeated along the head
 *    axis with repeat_interleave ("5. Linear Attention" chapter, "Gated
 *    DeltaNet body" layer code, the KV head expansion before the core). H_k =
 *    H is the ungrouped layer. A bad pair gives GDN_ERR_SHAPE.
 *  - States are fp32, [N][H][d_v][d_k] with d_k contiguous.
 *  - The decay gate is passed in log space: g = log(alpha), fp32 (alpha =
 *    exp(g) <= 1 for g <= 0). g must be finite; the chunkwise paths split
 *    decay factors into pieces bounded by 1, which holds for g <= 0, the
 *    pages' gate range (alpha in (0, 1]). beta is fp32, one scalar per
 *    (token, head).
 *  - dtype (gdn_dtype_t) selects the storage type of q, k, v and of the
 *    output o: GDN_DTYPE_F32 or GDN_DTYPE_BF16. All arithmetic accumulates in
 *    fp32; bf16 tensors are rounded to nearest-even on store.
 *  - stream is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work and return; results are valid once the stream
 *    has reached that point. Launch errors are reported by the call itself;
 *    faults during execution surface at the caller's next synchronisation.
 *  - Arguments are validated before anything is enqueued. On error nothing is
 *    enqueued and a negative gdn_status_t is returned; gdn_status_string()
 *    describes it. No call aborts the process or throws.
 *  - Calls on different streams may run concurrently when their output
 *    buffers are disjoint.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_VERSION 3

typedef enum {
    GDN_DTYPE_F32 = 0,
    GDN_DTYPE_BF16 = 1
} gdn_dtype_t;

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = -1,        /* a required pointer is NULL                        */
    GDN_ERR_SHAPE = -2,       /* a size is negative, zero where not allowed, or
                                 inconsistent with another argument                 */
    GDN_ERR_DTYPE = -3,       /* dtype is not a gdn_dtype_t value                   */
    GDN_ERR_UNSUPPORTED = -4, /* valid but not implemented (e.g. head dim > 128)    */
    GDN_ERR_HIP = -5,         /* the HIP runtime reported an error at launch        */
    GDN_ERR_WORKSPACE = -6,   /* workspace smaller than gdn_prefill_workspace_size()
                                 or not 256-byte aligned                            */
    GDN_ERR_SCRATCH = -7      /* gdn_prefill_noalloc: the sizes need more scratch
                                 than GDN_NOALLOC_SCRATCH_BYTES                     */
} gdn_status_t;

/* Library version (GDN_VERSION). */
int gdn_version(void);

/* Static description of a status code (never NULL). */
const char *gdn_status_string(int status);

/*
 * gdn_prefill - forward pass of the gated delta rule over whole sequences,
 * computed chunkwise ("5. Linear Attention" chapter, section "Chunk
 * implementation of the Delta Rule", stages 1-3; "Overwrite and Forget",
 * section 7): per chunk of 64 tokens the intra-chunk key Gram system is
 * solved as a unit-lower-triangular inverse and the chunk is applied to the
 * state as one update; the state is carried in fp32 from chunk to chunk.
 * The result equals the token-by-token recurrence up to rounding.
 *
 *   q, k          [B][T][H_k][d_k], dtype
 *   v             [B][T][H][d_v], dtype
 *   g, beta       [B][T][H] fp32 (g = log alpha)
 *   initial_state [N][H][d_v][d_k] fp32, or NULL for a zero initial state
 *   final_state   [N][H][d_v][d_k] fp32, or NULL to skip; may alias
 *                 initial_state (in-place continuation)
 *   o             [B][T][H][d_v], dtype; must not alias any input
 *   cu_seqlens    NULL: N must equal B and each batch row is one sequence of
 *                 T tokens. Otherwise a DEVICE int32 array of N+1 offsets
 *                 that packs N sequences along the T axis of a single batch
 *                 row: B must be 1, cu_seqlens[0] = 0, non-decreasing,
 *                 cu_seqlens[N] = T. Sequence n is tokens [cu[n], cu[n+1]);
 *                 empty sequences are allowed (their final state equals their
 *                 initial state). The offsets are read only on the device;
 *                 kernels clamp them into [0, T] and treat a decreasing pair
 *                 as an empty sequence, so malformed offsets give wrong
 *                 results but never out-of-range accesses. Check offsets on
 *                 the host with gdn_check_cu_seqlens() when in doubt.
 *   H_k           query/key heads (see the conventions above)
 *   B, T, H, N    B >= 1, T >= 0, 1 <= H <= 65535, 1 <= N <= 65535,
 *                 B*T < 2^31. When B*T = 0 the activation
 *                 pointers (q, k, v, g, beta, o) are not read and may be NULL.
 *   d_k, d_v      d_k in {16, 32, 64, 128}; 1 <= d_v <= 128 (else
 *                 GDN_ERR_UNSUPPORTED). bf16 with d_k = d_v = 128 runs the
 *                 MFMA chunk kernels; every other case runs the fp32
 *                 token-serial kernel (same result up to rounding).
 *   scale         multiplies every output (d_k^-1/2 in the usual layer)
 *   workspace     NULL, or DEVICE scratch memory owned by the caller, of at
 *                 least gdn_prefill_workspace_size() bytes, 256-byte aligned
 *                 (hipMalloc's alignment); its contents on entry do not
 *                 matter and are garbage on exit. With a workspace the MFMA
 *                 path runs in two passes: the per-chunk triangular systems
 *                 of every chunk and head are solved in parallel first, and
 *                 only the state recurrence walks the chunks in order (the
 *                 fast path). With NULL it runs as one pass whose
 *                 workgroups also solve each chunk's system, two chunks ahead
 *                 of the recurrence, on waves of their own (no scratch;
 *                 slower, since each of a head's four 32-wide d_v tiles
 *                 solves it again). Both give the same result up to rounding
 *                 order. Ignored by
 *                 the token-serial path. Calls that share a workspace must be
 *                 ordered on one stream.
 *   workspace_bytes  size of workspace; GDN_ERR_WORKSPACE if workspace is
 *                 non-NULL and too small or misaligned. The two-pass path
 *                 counts (64-token chunk slot, head) items, (B*T/64 + N + 1)
 *                 * H, in 32 bits: above 2^31 - 1 it returns
 *                 GDN_ERR_UNSUPPORTED (the workspace would exceed 12 TB).
 */
int gdn_prefill(const void *q, const void *k, const void *v,
                const float *g, const float *beta,
                const float *initial_state, float *final_state,
                void *o, const int32_t *cu_seqlens,
                int B, int T, int H, int H_k, int d_k, int d_v, int N,
                float scale, int dtype,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_prefill_noalloc - gdn_prefill for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. Same arguments, result and kernels as gdn_prefill with a
 * workspace, but no workspace argument: the scratch of the two-pass path is a
 * static device buffer of GDN_NOALLOC_SCRATCH_BYTES inside the library (one
 * per GPU, held from the library's first use of that GPU until the process
 * ends). The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine); the caller still passes every input and output.
 *
 * Limit: gdn_prefill_workspace_size() for the sizes must not exceed
 * GDN_NOALLOC_SCRATCH_BYTES (32 MiB: 5461 (64-token chunk slot, head)
 * items, e.g. B=4, T=4096, H=16), else GDN_ERR_SCRATCH and nothing is
 * enqueued. Paths that use no scratch (fp32, head dims other than 128) run
 * as in gdn_prefill.
 *
 * Every call on one GPU uses that GPU's one buffer: calls that overlap in
 * time on one GPU (different streams, or different host threads without
 * ordering) race and give wrong results. Order them on one stream. The
 * buffer's contents between calls do not matter; nothing in it must start at
 * zero.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int gdn_prefill_noalloc(const void *q, const void *k, const void *v,
                        const float *g, const float *beta,
                        const float *initial_state, float *final_state,
                        void *o, const int32_t *cu_seqlens,
                        int B, int T, int H, int H_k, int d_k, int d_v, int N,
                        float scale, int dtype, void *stream);

/*
 * gdn_prefill_workspace_size - bytes of workspace that gdn_prefill uses for
 * these sizes (same meaning as there, H the value heads; varlen != 0 when
 * cu_seqlens will be non-NULL). 0 when the path for these sizes uses none.
 * The size depends on the token count and the number of heads only, not on
 * the offsets: 6 KiB per (64-token chunk slot, head), with (B*T)/64 + N + 1
 * slots. Written to
 * *bytes; returns GDN_OK or the error gdn_prefill would return for these
 * sizes.
 */
int gdn_prefill_workspace_size(int B, int T, int H, int d_k, int d_v, int N,
                               int varlen, int dtype, size_t *bytes);

/*
 * gdn_prefill_prepare, gdn_prefill_apply - the two passes of gdn_prefill's
 * workspace path as separate calls; gdn_prefill with a workspace is exactly
 * prepare followed by apply on one stream. Arguments have the meaning they
 * have for gdn_prefill; both calls must see the same sizes, cu_seqlens, q,
 * k and g. Only the MFMA chunk path has passes (bf16, d_k = d_v = 128; else
 * GDN_ERR_UNSUPPORTED), and workspace is required (GDN_ERR_NULL).
 *
 * prepare reads k, g, beta (q is validated but not read) and writes, for
 * every 64-token chunk of every head, the chunk's T diag(beta) (T the
 * inverse of the unit-lower-triangular key Gram system: "5. Linear
 * Attention" chapter, section "Chunk implementation of the Delta Rule",
 * stage 1) into the workspace. All chunks are independent.
 *
 * apply reads q, k, v, g and the workspace, walks each sequence's chunks in
 * order carrying the state, and writes o and final_state (stages 2-3 of the
 * same section, with the decayed intra-chunk attention lower(Q K^T * Gamma)
 * formed on the way). beta enters only through the workspace.
 *
 * Splitting lets a caller overlap prepare of one batch with apply of
 * another on two streams (with two workspaces).
 */
int gdn_prefill_prepare(const void *q, const void *k, const float *g, const float *beta,
                        const int32_t *cu_seqlens,
                        int B, int T, int H, int H_k, int d_k, int d_v, int N, int dtype,
                        void *workspace, size_t workspace_bytes, void *stream);

int gdn_prefill_apply(const void *q, const void *k, const void *v, const float *g,
                      const float *initial_state, float *final_state,
                      void *o, const int32_t *cu_seqlens,
                      int B, int T, int H, int H_k, int d_k, int d_v, int N,
                      float scale, int dtype,
                      const void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_prefill_seqpar - the same forward pass as gdn_prefill, with long
 * sequences cut into segments of whole 64-token chunks whose chains run side
 * by side: for batches whose longest chains leave compute units idle (one
 * long sequence, few heads, or a packed batch where one sequence is much
 * longer than the rest). A run of tokens acts on the state as one affine map
 * S_end = S_start A + B ("Overwrite and Forget", section 7). The longest
 * sequence (M chunks) is cut into `segments` segments of L = ceil(M /
 * segments) chunks and every other sequence into segments of L chunks (its
 * last one shorter), so short sequences stay whole. A first chain pass runs
 * every sequence's first segment from its initial state (writing outputs)
 * and, side by side, computes B and A of every middle segment (zero start
 * state; v = 0 from the identity); the start states of the later segments
 * follow in order; a second chain pass runs those segments from their true
 * start states and writes their outputs and the final states. Critical path:
 * two segments' chains; extra work: two more chain walks of each middle
 * segment. The result equals gdn_prefill's up to rounding (a map carries the
 * bf16 rounding of the chunk kernels once more). segments = 1 runs each
 * sequence as one segment, like gdn_prefill's two-pass path.
 *
 *   arguments     as gdn_prefill, including cu_seqlens and N (packed
 *                 sequences: B = 1); bf16 with d_k = d_v = 128 only (else
 *                 GDN_ERR_UNSUPPORTED)
 *   segments      >= 1, segments of the longest sequence; N * segments <=
 *                 65535 and (B*T/64 + N * segments + 1) * H < 2^31 (else
 *                 GDN_ERR_UNSUPPORTED)
 *   workspace     required, gdn_prefill_seqpar_workspace_size() bytes,
 *                 256-byte aligned, caller-owned; contents on entry do not
 *                 matter. Calls that share a workspace must be ordered on one
 *                 stream.
 */
int gdn_prefill_seqpar(const void *q, const void *k, const void *v,
                       const float *g, const float *beta,
                       const float *initial_state, float *final_state, void *o,
                       const int32_t *cu_seqlens,
                       int B, int T, int H, int H_k, int d_k, int d_v, int N, int segments,
                       float scale, int dtype,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace gdn_prefill_seqpar needs (H the value heads; varlen
 * non-zero when cu_seqlens will be given, as for gdn_prefill_workspace_size). */
int gdn_prefill_seqpar_workspace_size(int B, int T, int H, int d_k, int d_v, int N, int varlen,
                                      int segments, int dtype, size_t *bytes);

/*
 * gdn_prefill_recurrent - the same forward pass as gdn_prefill, computed by
 * the token-serial recurrence in fp32 arithmetic (the "recurrent" execution
 * path of "Overwrite and Forget", section 7). Same arguments, layouts and
 * errors as gdn_prefill. gdn_prefill itself uses this path for fp32 tensors
 * and for head sizes other than d_k = d_v = 128; calling it directly gives
 * the chunkwise path an independent on-device cross-check.
 */
int gdn_prefill_recurrent(const void *q, const void *k, const void *v,
                          const float *g, const float *beta,
                          const float *initial_state, float *final_state,
                          void *o, const int32_t *cu_seqlens,
                          int B, int T, int H, int H_k, int d_k, int d_v, int N,
                          float scale, int dtype, void *stream);

/*
 * gdn_decode_step - one recurrent step for B independent sequences, updating
 * an HBM-resident state in place ("Overwrite and Forget", section 5
 * pseudo-code; "6.6 Gated DeltaNet" section 6.6.8, inference flow):
 *
 *   r = alpha S k;  delta = beta (v - r);  S <- alpha S + delta k^T;
 *   o = scale S q
 *
 * Each state row is read once and written once.
 *
 *   q, k       [B][H_k][d_k], dtype (H_k query/key heads, as above)
 *   v          [B][H][d_v], dtype
 *   g, beta    [B][H] fp32
 *   state      [B][H][d_v][d_k] fp32, read and overwritten in place
 *   o          [B][H][d_v], dtype
 *   d_k, d_v   d_k in {16, 32, 64, 128}; 1 <= d_v <= 4096
 */
int gdn_decode_step(const void *q, const void *k, const void *v,
                    const float *g, const float *beta,
                    float *state, void *o,
                    int B, int H, int H_k, int d_k, int d_v,
                    float scale, int dtype, void *stream);

/*
 * gdn_prefill_channel_gated, gdn_decode_step_channel_gated - the same
 * forward pass and decode step with one decay rate per key channel instead
 * of one per head ("6.6 Gated DeltaNet" section 6.6.7: Kimi Linear's gate,
 * alpha_t in R^d). Column j of each d_v x d_k state decays by exp(g[j])
 * before the retrieval:
 *
 *     S_t = S_{t-1} diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *
 * Arguments, layouts and errors as gdn_prefill and gdn_decode_step, except g:
 *   prefill: g [B][T][H][d_k] fp32;  decode: g [B][H][d_k] fp32.
 * With every channel of g equal, the results equal those of the per-head
 * entry points.
 *
 * Prefill paths. bf16 with d_k = d_v = 128 and a workspace (size from
 * gdn_prefill_channel_workspace_size; 256-byte aligned, caller-owned, contents
 * on entry irrelevant, GDN_ERR_WORKSPACE if too small or misaligned) runs the
 * chunkwise form in two passes: with gamma the running sum of g over a
 * 64-token chunk, the keys and queries carry the decay channel by channel
 * (K e^gamma, K e^{gamma_63 - gamma}, Q e^gamma), the in-chunk products
 * sum_c k_i[c] k_j[c] e^{gamma_i[c] - gamma_j[c]} are split at a reference
 * token per 16-token block so that they run on the matrix cores (the
 * query-key sums of a block with itself from bf16 hi + lo operand splits, so
 * that nearly cancelling sums keep their relative precision), and the
 * state decays by e^{gamma_63} per channel at each chunk end. Otherwise
 * (no workspace, fp32, other head sizes) the token-serial fp32 recurrence.
 */
int gdn_prefill_channel_workspace_size(int B, int T, int H, int d_k, int d_v, int N,
                                       int varlen, int dtype, size_t *bytes);

int gdn_prefill_channel_gated(const void *q, const void *k, const void *v,
                              const float *g, const float *beta,
                              const float *initial_state, float *final_state,
                              void *o, const int32_t *cu_seqlens,
                              int B, int T, int H, int H_k, int d_k, int d_v, int N,
                              float scale, int dtype, void *workspace,
                              size_t workspace_bytes, void *stream);

int gdn_decode_step_channel_gated(const void *q, const void *k, const void *v,
                                  const float *g, const float *beta,
                                  float *state, void *o,
                                  int B, int H, int H_k, int d_k, int d_v,
                                  float scale, int dtype, void *stream);

/*
 * gdn_mixer_prologue - everything between the input projections and the
 * recurrence ("5. Linear Attention" chapter, sections "Causal Conv1d" and
 * "Gated DeltaNet body"; "6.6 Gated DeltaNet" sections 6.6.3-6.6.4):
 *
 *   1. depthwise causal convolution with 4 taps over every channel of q, k,
 *      v (zero history before each sequence start, no bias), then SiLU;
 *   2. L2 normalisation of q and k per (token, head):
 *      x / sqrt(sum x^2 + 1e-6);
 *   3. gates: g = -A[h] * softplus(a + dt_bias[h]),  beta = sigmoid(b).
 *
 *   q_raw, k_raw   [B][T][H_k][d_k], dtype      (projection outputs)
 *   v_raw          [B][T][H][d_v], dtype
 *   conv_w         [2*H_k*d_k + H*d_v][4], dtype; channel order: all q
 *                  channels (head-major), then k, then v; tap 3 multiplies
 *                  the current token, tap 0 the token three steps back
 *   a, b           [B][T][H], dtype (per value head)
 *   A              [H] fp32 (positive decay rates)
 *   dt_bias        [H] fp32, or NULL for zero
 *   cu_seqlens     as for gdn_prefill (NULL: each batch row is a sequence)
 *   q, k, v        outputs, same shapes and dtype as the raw inputs; must not
 *                  alias them
 *   g, beta        outputs [B][T][H] fp32
 *   H, H_k         value and query/key heads as above, H <= 65535
 *   d_k, d_v       each in {16, 32, 64, 128, 256} (else GDN_ERR_UNSUPPORTED)
 */
int gdn_mixer_prologue(const void *q_raw, const void *k_raw, const void *v_raw,
                       const void *conv_w, const void *a, const void *b,
                       const float *A, const float *dt_bias,
                       const int32_t *cu_seqlens,
                       void *q, void *k, void *v, float *g, float *beta,
                       int B, int T, int H, int H_k, int d_k, int d_v, int N,
                       int dtype, void *stream);

/*
 * gdn_mixer_epilogue - gated RMSNorm of the recurrence output ("5. Linear
 * Attention" chapter, section "Gated RMSNorm"; "6.6 Gated DeltaNet" section
 * 6.6.2, output gate), per (token, head) row of d_v values:
 *
 *   out = norm_w * y / sqrt(mean(y^2) + eps) * silu(z)
 *
 *   y, z, out   [rows][H][d_v], dtype (rows = B*T); out may alias y
 *   norm_w      [d_v] fp32, or NULL for ones
 *   d_v         in {16, 32, 64, 128, 256} (else GDN_ERR_UNSUPPORTED)
 */
int gdn_mixer_epilogue(const void *y, const void *z, const float *norm_w, void *out,
                       int rows, int H, int d_v, float eps, int dtype, void *stream);

/*
 * gdn_decode_mixer_step - one token of the whole token mixer for B
 * sequences, fused into one launch ("6.6 Gated DeltaNet" section 6.6.8,
 * inference flow; the conv cache is the convolution state a deployment keeps
 * besides the matrix state, "Overwrite and Forget" section 13.4):
 *
 *   1. per conv channel, the causal 4-tap convolution of the three cached
 *      inputs and the new one, then SiLU (as gdn_mixer_prologue over a
 *      sequence); the cache is shifted by one token in place;
 *   2. L2-norm of q and k; g = -A softplus(a + dt_bias), beta = sigmoid(b);
 *   3. the gated delta rule step of gdn_decode_step on the state (in place),
 *      value head h reading query/key head h / (H / H_k);
 *   4. out = norm_w * y / sqrt(mean(y^2) + eps) * silu(z) per (sequence,
 *      value head), y the step's output.
 *
 * Running T steps from a zero cache and a zero state gives the same outputs as
 * gdn_mixer_prologue -> gdn_prefill -> gdn_mixer_epilogue over those T tokens
 * (up to rounding: intermediates stay fp32 here).
 *
 *   q_raw, k_raw  [B][H_k][d_k], dtype     the token's projections
 *   v_raw, z      [B][H][d_v], dtype
 *   conv_w        [2*H_k*d_k + H*d_v][4], dtype (channel order q, k, v; tap 3
 *                 multiplies the new token)
 *   conv_state    [B][3][2*H_k*d_k + H*d_v], dtype, read and updated in place:
 *                 row 0 = the input three tokens back, row 2 = the previous
 *                 token; all zeros for a sequence that has not started
 *   a, b          [B][H], dtype;  A [H] fp32;  dt_bias [H] fp32 or NULL (zero)
 *   norm_w        [d_v] fp32 or NULL (ones);  eps >= 0
 *   state         [B][H][d_v][d_k] fp32, read and updated in place
 *   out           [B][H][d_v], dtype; may alias z, no other argument
 *   d_k, d_v      d_k in {16, 32, 64, 128}; d_v in {16, 32, 64, 128, 256};
 *                 (H / H_k) * d_v <= 4096 (else GDN_ERR_UNSUPPORTED)
 */
int gdn_decode_mixer_step(const void *q_raw, const void *k_raw, const void *v_raw,
                          const void *conv_w, void *conv_state,
                          const void *a, const void *b, const float *A, const float *dt_bias,
                          const void *z, const float *norm_w, float eps,
                          float *state, void *out,
                          int B, int H, int H_k, int d_k, int d_v,
                          float scale, int dtype, void *stream);

/*
 * gdn_check_cu_seqlens - host-side validation of packed-sequence offsets.
 * cu is a HOST array of N+1 entries. Returns GDN_OK when cu[0] = 0, the
 * offsets are non-decreasing and cu[N] = T; GDN_ERR_SHAPE otherwise;
 * GDN_ERR_NULL for a NULL pointer.
 */
int gdn_check_cu_seqlens(const int32_t *cu, int N, int T);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
