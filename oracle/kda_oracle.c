/*
 * kda_oracle.c -- plain fp64 CPU oracle for the Kimi Delta Attention (KDA)
 * forward pass.  TEST INFRASTRUCTURE ONLY: nothing on the product path may
 * link, load or call this file.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header or table
 * with the HIP library.
 *
 * What it computes (one token at a time, no chunking, no blocking):
 *
 *   The pages describe KDA as a delta-rule linear attention that keeps a
 *   fixed-size state matrix, forgets through a gate, and refines Gated
 *   DeltaNet with a finer per-channel gate ("What is Kimi Delta Attention
 *   (KDA)", Moonshot AI Open-Sources FlashKDA, kongchang.com/en; "¿Qué es la
 *   atención Kimi Delta y por qué es importante?", 7minutos.es).  Written out
 *   as the gated delta rule with a per-channel decay:
 *
 *     S_t = (I - b_t k_t k_t^T) Diag(exp(a_t)) S_{t-1} + b_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 *   with S a K x V matrix per (sequence, head).  The forward call's inputs are
 *   listed on "Debajo del capó: CUTLASS en Hopper" (7minutos.es): q,k,g [.,K],
 *   v [.,V], beta logits, scale, A_log (per head), dt_bias, lower_bound in
 *   [-5,0], optional initial/final states, optional int64 cu_seqlens.  The
 *   flags on "作为 FLA 后端的用法" (zuobiaodaohang) say the q/k L2 norm, the
 *   beta sigmoid and the gate activation all run inside the kernel, so the
 *   oracle applies them itself:
 *
 *     k_t <- k_t / sqrt(|k_t|^2 + eps), q_t likewise, eps = 1e-6
 *     b_t  = 1 / (1 + exp(-beta_t))
 *     a_t[d] = max(lower_bound, -exp(A_log[h]) * softplus(g_t[d] + dt_bias[h,d]))
 *
 *   The gate formula is not printed on the pages; this is the plain reading of
 *   the parameter names (a positive rate exp(A_log) times a positive step
 *   softplus(g + dt_bias), negated) clamped to [lower_bound, 0] ("safe gate").
 *   It lives in one function, kda_gate(), so another reading is one edit.
 *
 *   Per token the state is first decayed, then receives the delta-rule write,
 *   then the output reads the updated state:
 *     S <- Diag(exp(a)) S;  u = b (v - S^T k);  S <- S + k u^T;  o = scale S^T q
 *   which is algebraically the recurrence above.
 *
 * Precision: every input is decoded exactly (bf16 bits << 16 -> float ->
 * double) and all arithmetic is fp64.  Build without -ffast-math.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDA_ORACLE_EPS 1e-6

static double bf16_to_f64(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* softplus(x) = log(1 + e^x), in the overflow-free form max(x,0) + log1p(e^-|x|). */
double kda_softplus(double x)
{
    if (isnan(x)) return x;
    if (isinf(x)) return x > 0 ? x : 0.0;
    return (x > 0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

/* Per-channel log-decay a = max(lb, -exp(A_log) * softplus(g + dt_bias)). */
double kda_gate(double g, double A_log, double dt_bias, double lower_bound)
{
    double a = -exp(A_log) * kda_softplus(g + dt_bias);
    if (isnan(a)) return a;
    return a > lower_bound ? a : lower_bound;
}

/* b = sigmoid(beta); exact 0 and 1 at beta = -inf and +inf. */
double kda_sigmoid(double x)
{
    return 1.0 / (1.0 + exp(-x));
}

/*
 * Full forward.  Layouts are row-major and contiguous:
 *   q, k, g : [B, T, H, K] bf16 bits      v : [B, T, H, V] bf16 bits
 *   beta    : [B, T, H]    bf16 bits      A_log : [H] fp32, dt_bias : [H, K] fp32
 *   cu_seqlens : host int64 [N + 1] or NULL.  With it, B must be 1 and
 *                sequence n owns rows [cu[n], cu[n+1]); without it N = B and
 *                batch row n is one sequence of T tokens.
 *   initial_state : [N, H, K, V] fp64 or NULL (zeros)
 *   final_state   : [N, H, K, V] fp64 or NULL (not written)
 *   out           : [B, T, H, V] fp64
 * Returns 0 on success, a negative value on a bad argument.
 */
int kda_oracle_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   const uint16_t *g, const uint16_t *beta,
                   int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                   const int64_t *cu_seqlens, int64_t N,
                   double scale, const float *A_log, const float *dt_bias,
                   double lower_bound,
                   const double *initial_state, double *final_state,
                   double *out, int num_threads)
{
    if (!q || !k || !v || !g || !beta || !A_log || !dt_bias || !out) return -1;
    if (B < 1 || T < 0 || H < 1 || K < 1 || V < 1) return -2;
    if (cu_seqlens) {
        if (B != 1 || N < 1 || cu_seqlens[0] != 0 || cu_seqlens[N] != T) return -3;
        for (int64_t n = 0; n < N; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return -3;
    } else {
        N = B;
    }
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif
    const int64_t units = N * H;
    int err = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t unit = 0; unit < units; ++unit) {
        const int64_t n = unit / H, h = unit % H;
        /* token range of sequence n, as absolute rows of the [B*T] token axis */
        int64_t row0, row1;
        if (cu_seqlens) { row0 = cu_seqlens[n]; row1 = cu_seqlens[n + 1]; }
        else { row0 = n * T; row1 = n * T + T; }

        double *S = (double *)malloc(sizeof(double) * (size_t)(K * V));
        double *kh = (double *)malloc(sizeof(double) * (size_t)K);
        double *qh = (double *)malloc(sizeof(double) * (size_t)K);
        double *dec = (double *)malloc(sizeof(double) * (size_t)K);
        double *u = (double *)malloc(sizeof(double) * (size_t)V);
        if (!S || !kh || !qh || !dec || !u) {
#pragma omp atomic write
            err = -4;
            free(S); free(kh); free(qh); free(dec); free(u);
            continue;
        }
        const size_t sidx = (size_t)((n * H + h) * K * V);
        for (int64_t i = 0; i < K * V; ++i)
            S[i] = initial_state ? initial_state[sidx + (size_t)i] : 0.0;

        const double A = (double)A_log[h];
        for (int64_t row = row0; row < row1; ++row) {
            const size_t qk_off = (size_t)((row * H + h) * K);
            const size_t v_off = (size_t)((row * H + h) * V);
            /* L2 normalisation of q and k */
            double sq = 0.0, sk = 0.0;
            for (int64_t d = 0; d < K; ++d) {
                qh[d] = bf16_to_f64(q[qk_off + d]);
                kh[d] = bf16_to_f64(k[qk_off + d]);
                sq += qh[d] * qh[d];
                sk += kh[d] * kh[d];
            }
            const double rq = 1.0 / sqrt(sq + KDA_ORACLE_EPS);
            const double rk = 1.0 / sqrt(sk + KDA_ORACLE_EPS);
            for (int64_t d = 0; d < K; ++d) { qh[d] *= rq; kh[d] *= rk; }

            const double b = kda_sigmoid(bf16_to_f64(beta[(size_t)(row * H + h)]));
            for (int64_t d = 0; d < K; ++d)
                dec[d] = exp(kda_gate(bf16_to_f64(g[qk_off + d]), A,
                                      (double)dt_bias[h * K + d], lower_bound));

            /* decay: S <- Diag(exp(a)) S */
            for (int64_t d = 0; d < K; ++d)
                for (int64_t j = 0; j < V; ++j) S[d * V + j] *= dec[d];
            /* delta write: u = b (v - S^T k), S <- S + k u^T */
            for (int64_t j = 0; j < V; ++j) u[j] = 0.0;
            for (int64_t d = 0; d < K; ++d)
                for (int64_t j = 0; j < V; ++j) u[j] += S[d * V + j] * kh[d];
            for (int64_t j = 0; j < V; ++j) u[j] = b * (bf16_to_f64(v[v_off + j]) - u[j]);
            for (int64_t d = 0; d < K; ++d)
                for (int64_t j = 0; j < V; ++j) S[d * V + j] += kh[d] * u[j];
            /* output from the updated state: o = scale S^T q */
            for (int64_t j = 0; j < V; ++j) u[j] = 0.0;
            for (int64_t d = 0; d < K; ++d)
                for (int64_t j = 0; j < V; ++j) u[j] += S[d * V + j] * qh[d];
            for (int64_t j = 0; j < V; ++j) out[v_off + j] = scale * u[j];
        }
        if (final_state)
            for (int64_t i = 0; i < K * V; ++i) final_state[sidx + (size_t)i] = S[i];
        free(S); free(kh); free(qh); free(dec); free(u);
    }
    return err;
}
