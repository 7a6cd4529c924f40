/*
 * gdn_oracle.c - plain fp64 CPU oracle of the Gated Delta Rule token mixer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or constant with the HIP path and must never stand in for it.
 *
 * Everything is computed in double precision, token by token, in the order the
 * pages state the method. No blocking, no chunking, no reordering.
 *
 * Sources (web pages; section names as printed on them):
 *  [OF]  "[LLM Algorithms-2] Gated DeltaNet: Teaching Linear Attention to
 *        Overwrite and Forget" - section 4 (boxed gated update), 4.3 (the
 *        retrieval reads the already-decayed state), 5 (retain/erase/write
 *        pseudo-code), 1 (S is d_v x d_k and the readout is S q).
 *  [FB]  "6.6 Gated DeltaNet (linear attention)", LLM full-stack book -
 *        6.6.3 (decay gate exp(-A*softplus(.)), sigmoid update gate),
 *        6.6.4 (token loop: decay, retrieve, delta, rank-1 write, read the
 *        updated state; l2norm with eps 1e-6 under the square root; q scaled
 *        by d_k^-1/2).
 *  [LQ]  "5. Linear Attention" (LinkQwen ch. 5) - "Causal Conv1d" (depthwise,
 *        kernel 4, left zero padding, no bias, then SiLU), "Gated RMSNorm"
 *        (weight * x*rsqrt(mean(x^2)+eps) * silu(z)), "Gated DeltaNet body"
 *        (order: conv+SiLU, split q/k/v, gates, core, gated norm).
 *
 * Readings where the pages disagree (all listed in the design notes):
 *  - decay is applied before the retrieval ([OF] 4.3, [FB] 6.6.4 code);
 *  - the state is stored [d_v][d_k], d_k contiguous ([OF] 1);
 *  - beta is one scalar per (token, head); g = log(alpha) is the gate input;
 *  - the output scale is an explicit argument.
 *
 * Layouts (row-major, token-major activations):
 *   q, k   [T_total][H][d_k]        (a batch of B sequences of length T is
 *   v      [T_total][H][d_v]         T_total = B*T with cu = {0, T, 2T, ...})
 *   g,beta [T_total][H]
 *   S0,S1  [N][H][d_v][d_k]
 *   o      [T_total][H][d_v]
 *
 * Returns 0 on success, -1 on a bad argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_version(void) { return 1; }

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * One (sequence, head) chain of the gated delta rule, [OF] sections 4-5 and
 * [FB] 6.6.4, for tokens [bos, eos):
 *
 *   S <- alpha_t * S                       (forget: decay the whole state)
 *   r <- S k_t                             (what the decayed state holds at k_t)
 *   d <- beta_t * (v_t - r)                (error, scaled by the update gate)
 *   S <- S + d k_t^T                       (rank-1 write along k_t)
 *   o_t <- scale * S q_t                   (read the UPDATED state)
 *
 * which equals S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
 */
static void chain(const double *q, const double *k, const double *v,
                  const double *g, const double *beta, double *S, double *o,
                  int64_t bos, int64_t eos, int h, int H, int dk, int dv,
                  double scale, double *r)
{
    for (int64_t t = bos; t < eos; ++t) {
        const double *qt = q + (t * H + h) * (int64_t)dk;
        const double *kt = k + (t * H + h) * (int64_t)dk;
        const double *vt = v + (t * H + h) * (int64_t)dv;
        const double alpha = exp(g[t * H + h]);
        const double b = beta[t * H + h];

        for (int64_t i = 0; i < (int64_t)dv * dk; ++i)
            S[i] *= alpha;

        for (int i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j)
                acc += S[(int64_t)i * dk + j] * kt[j];
            r[i] = acc;
        }
        for (int i = 0; i < dv; ++i) {
            const double d = b * (vt[i] - r[i]);
            for (int j = 0; j < dk; ++j)
                S[(int64_t)i * dk + j] += d * kt[j];
        }
        double *ot = o + (t * H + h) * (int64_t)dv;
        for (int i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j)
                acc += S[(int64_t)i * dk + j] * qt[j];
            ot[i] = scale * acc;
        }
    }
}

/*
 * Full recurrence over N independent sequences delimited by cu (int64, N+1
 * entries, cu[0]=0, non-decreasing). S0 may be NULL (zero initial state);
 * S1 may be NULL (final state not returned). nthreads <= 0 uses the OpenMP
 * default.
 */
int oracle_gdn_recurrent(const double *q, const double *k, const double *v,
                         const double *g, const double *beta,
                         const double *S0, double *S1, double *o,
                         const int64_t *cu, int N, int H, int dk, int dv,
                         double scale, int nthreads)
{
    if (!q || !k || !v || !g || !beta || !o || !cu || N < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    for (int n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n] || cu[n] < 0)
            return -1;
    const int64_t pairs = (int64_t)N * H;
    const int64_t ssz = (int64_t)dv * dk;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t p = 0; p < pairs; ++p) {
        const int n = (int)(p / H), h = (int)(p % H);
        double *S = (double *)malloc(sizeof(double) * (size_t)ssz);
        double *r = (double *)malloc(sizeof(double) * (size_t)dv);
        if (S0)
            memcpy(S, S0 + p * ssz, sizeof(double) * (size_t)ssz);
        else
            memset(S, 0, sizeof(double) * (size_t)ssz);
        chain(q, k, v, g, beta, S, o, cu[n], cu[n + 1], h, H, dk, dv, scale, r);
        if (S1)
            memcpy(S1 + p * ssz, S, sizeof(double) * (size_t)ssz);
        free(S);
        free(r);
    }
    return 0;
}

/* SiLU(x) = x * sigmoid(x), [FB] 6.6.2. */
static double silu(double x) { return x / (1.0 + exp(-x)); }

/* softplus(x) = log(1 + e^x), [FB] 6.6.3; written so that it does not overflow. */
static double softplus(double x) { return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x)); }

/*
 * Depthwise causal convolution, kernel width K, followed by SiLU ([LQ]
 * "Causal Conv1d"): each channel c of each sequence is convolved on its own;
 * the window for token t is x[t-K+1 .. t], positions before the sequence
 * start read as zero, tap K-1 multiplies the current token, there is no bias.
 *   x, y [T_total][C]; w [C][K]; cu as above.
 */
int oracle_causal_conv_silu(const double *x, const double *w, double *y,
                            const int64_t *cu, int N, int C, int K, int nthreads)
{
    if (!x || !w || !y || !cu || N < 0 || C <= 0 || K <= 0)
        return -1;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int n = 0; n < N; ++n) {
        for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
            for (int c = 0; c < C; ++c) {
                double acc = 0.0;
                for (int j = 0; j < K; ++j) {
                    const int64_t s = t - (K - 1) + j;
                    if (s >= cu[n])
                        acc += w[(int64_t)c * K + j] * x[s * C + c];
                }
                y[t * C + c] = silu(acc);
            }
        }
    }
    return 0;
}

/* x <- x * (sum x^2 + eps)^-1/2 over each row of length d ([FB] 6.6.4 l2norm). */
int oracle_l2norm_rows(double *x, int64_t rows, int d, double eps)
{
    if (!x || rows < 0 || d <= 0)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int j = 0; j < d; ++j)
            ss += x[r * d + j] * x[r * d + j];
        const double inv = 1.0 / sqrt(ss + eps);
        for (int j = 0; j < d; ++j)
            x[r * d + j] *= inv;
    }
    return 0;
}

/*
 * Gates ([FB] 6.6.3; [LQ] "Gated DeltaNet body"):
 *   g    = log(alpha) = -A[h] * softplus(a + dt_bias[h])   (dt_bias may be NULL = 0)
 *   beta = sigmoid(b)
 * a, b, g, beta are [rows][H].
 */
int oracle_gates(const double *a, const double *b, const double *A, const double *dt_bias,
                 double *g, double *beta, int64_t rows, int H)
{
    if (!a || !b || !A || !g || !beta || rows < 0 || H <= 0)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        for (int h = 0; h < H; ++h) {
            const int64_t i = r * H + h;
            const double bias = dt_bias ? dt_bias[h] : 0.0;
            g[i] = -A[h] * softplus(a[i] + bias);
            beta[i] = 1.0 / (1.0 + exp(-b[i]));
        }
    }
    return 0;
}

/*
 * Gated RMSNorm ([LQ] "Gated RMSNorm"; [FB] 6.6.2 output gate) over each row
 * of length d:  out = w * y / sqrt(mean(y^2) + eps) * silu(z).
 * w may be NULL (all ones).
 */
int oracle_gated_rmsnorm(const double *y, const double *z, const double *w, double *out,
                         int64_t rows, int d, double eps)
{
    if (!y || !z || !out || rows < 0 || d <= 0)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int j = 0; j < d; ++j)
            ss += y[r * d + j] * y[r * d + j];
        const double inv = 1.0 / sqrt(ss / d + eps);
        for (int j = 0; j < d; ++j) {
            const double wj = w ? w[j] : 1.0;
            out[r * d + j] = wj * (y[r * d + j] * inv) * silu(z[r * d + j]);
        }
    }
    return 0;
}

/*
 * Per-channel decay ("6.6 Gated DeltaNet", section 6.6.7: Kimi Linear makes
 * the decay gate a vector alpha_t in R^d, one rate per feature channel of the
 * key space, instead of one scalar per head). With the state stored d_v x d_k
 * the decay scales column j of S by alpha_t[j]; the retrieval reads the
 * decayed state, as for the scalar gate:
 *
 *   S <- S diag(alpha_t);  r <- S k_t;  d <- beta_t (v_t - r);
 *   S <- S + d k_t^T;      o_t <- scale * S q_t
 *
 * i.e. S_t = S_{t-1} diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
 * g holds log(alpha) per channel: [T_total][H][dk]. Other arguments as in
 * oracle_gdn_recurrent.
 */
static void chain_channel(const double *q, const double *k, const double *v,
                          const double *g, const double *beta, double *S, double *o,
                          int64_t bos, int64_t eos, int h, int H, int dk, int dv,
                          double scale, double *r)
{
    for (int64_t t = bos; t < eos; ++t) {
        const double *qt = q + (t * H + h) * (int64_t)dk;
        const double *kt = k + (t * H + h) * (int64_t)dk;
        const double *vt = v + (t * H + h) * (int64_t)dv;
        const double *gt = g + (t * H + h) * (int64_t)dk;
        const double b = beta[t * H + h];

        for (int i = 0; i < dv; ++i)
            for (int j = 0; j < dk; ++j)
                S[(int64_t)i * dk + j] *= exp(gt[j]);

        for (int i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j)
                acc += S[(int64_t)i * dk + j] * kt[j];
            r[i] = acc;
        }
        for (int i = 0; i < dv; ++i) {
            const double d = b * (vt[i] - r[i]);
            for (int j = 0; j < dk; ++j)
                S[(int64_t)i * dk + j] += d * kt[j];
        }
        double *ot = o + (t * H + h) * (int64_t)dv;
        for (int i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j)
                acc += S[(int64_t)i * dk + j] * qt[j];
            ot[i] = scale * acc;
        }
    }
}

int oracle_gdn_recurrent_channel(const double *q, const double *k, const double *v,
                                 const double *g, const double *beta,
                                 const double *S0, double *S1, double *o,
                                 const int64_t *cu, int N, int H, int dk, int dv,
                                 double scale, int nthreads)
{
    if (!q || !k || !v || !g || !beta || !o || !cu || N < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    for (int n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n] || cu[n] < 0)
            return -1;
    const int64_t pairs = (int64_t)N * H;
    const int64_t ssz = (int64_t)dv * dk;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t p = 0; p < pairs; ++p) {
        const int n = (int)(p / H), h = (int)(p % H);
        double *S = (double *)malloc(sizeof(double) * (size_t)ssz);
        double *r = (double *)malloc(sizeof(double) * (size_t)dv);
        if (S0)
            memcpy(S, S0 + p * ssz, sizeof(double) * (size_t)ssz);
        else
            memset(S, 0, sizeof(double) * (size_t)ssz);
        chain_channel(q, k, v, g, beta, S, o, cu[n], cu[n + 1], h, H, dk, dv, scale, r);
        if (S1)
            memcpy(S1 + p * ssz, S, sizeof(double) * (size_t)ssz);
        free(S);
        free(r);
    }
    return 0;
}
