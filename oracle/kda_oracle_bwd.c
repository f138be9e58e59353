/*
 * kda_oracle_bwd.c -- plain fp64 CPU oracle for the gradient (vector-Jacobian
 * product) of the Kimi Delta Attention (KDA) forward pass.  TEST
 * INFRASTRUCTURE ONLY: nothing on the product path may link, load or call this
 * file; it shares no code with the HIP library.  It is compiled into the same
 * library as kda_oracle.c and uses that file's gate, softplus and sigmoid.
 *
 * The forward it differentiates is the token recurrence of kda_oracle.c (the
 * gated delta rule with a per-channel decay, as the pages describe KDA: "What
 * is Kimi Delta Attention (KDA)", kongchang.com/en; the in-kernel norms, sigmoid
 * and gate of the backend call, "作为 FLA 后端的用法", zuobiaodaohang.com), per
 * sequence and head, with S a K x V state:
 *
 *   qh = q / sqrt(|q|^2 + eps),  kh = k / sqrt(|k|^2 + eps)
 *   b  = sigmoid(beta)
 *   z_d = -exp(A_log) softplus(g_d + dt_bias_d),  a_d = max(lb, z_d)
 *   S' = Diag(exp(a)) S_prev
 *   r  = v - S'^T kh,  u = b r
 *   S  = S' + kh u^T
 *   o  = scale S^T qh
 *
 * The pages ship a forward pass only ("性能与注意事项": no backward).  This file
 * is the derivative of that recurrence, written out by the chain rule and run
 * backwards over the tokens.  With G the gradient of the loss with respect to
 * the state after token t (dS_T, or zero, at the end):
 *
 *   G   += scale qh do^T                     dqh = scale S do
 *   dkh  = G u,  du = G^T kh                 (from S = S' + kh u^T)
 *   dv   = b du,  db = du . r,  dkh -= b S' du,  dS' = G - b kh du^T
 *   da_d = sum_j dS'[d,j] S'[d,j]            (S'[d,:] = exp(a_d) S_prev[d,:])
 *   G    = Diag(exp(a)) dS'                  (the gradient of S_prev)
 *
 * and then the input activations:
 *
 *   dq = rq dqh - rq^3 (q . dqh) q   (rq = (|q|^2 + eps)^-1/2; k likewise)
 *   dbeta = db b (1 - b)
 *   where z_d > lb:  dg_d = ddt_bias_d-share = -exp(A_log) sigmoid(g_d + dt_bias_d) da_d,
 *                    dA_log += z_d da_d;
 *   where z_d <= lb (clamped): no gradient flows to g, dt_bias or A_log.
 *
 * The clamp's kink (z_d == lb exactly) takes the clamped side: a reading of
 * ours, since max() has no derivative there.  dA_log and dt_bias are shared by
 * every sequence, so their gradients are summed over sequences and tokens.
 * The states the reverse pass needs are recomputed from checkpoints taken
 * every 64 tokens on a forward pass.  Everything is fp64, without fast-math.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDA_ORACLE_BWD_EPS 1e-6
#define KDA_ORACLE_CKPT 64

/* the gate and activations of kda_oracle.c */
double kda_softplus(double x);
double kda_sigmoid(double x);
double kda_gate(double g, double A_log, double dt_bias, double lower_bound);

/* one token's activations: normalised q and k (with their reciprocal norms),
 * b, the unclamped and clamped log-decays, and the decays */
typedef struct {
    double rq, rk, b;
} tok_t;

static void token_acts(const double *q, const double *k, double beta, const double *g, double A,
                       const double *dtb, double lb, int64_t K, double *qh, double *kh, double *z, double *a,
                       double *dec, tok_t *t)
{
    double sq = 0.0, sk = 0.0;
    for (int64_t d = 0; d < K; ++d) { sq += q[d] * q[d]; sk += k[d] * k[d]; }
    t->rq = 1.0 / sqrt(sq + KDA_ORACLE_BWD_EPS);
    t->rk = 1.0 / sqrt(sk + KDA_ORACLE_BWD_EPS);
    for (int64_t d = 0; d < K; ++d) { qh[d] = q[d] * t->rq; kh[d] = k[d] * t->rk; }
    t->b = kda_sigmoid(beta);
    for (int64_t d = 0; d < K; ++d) {
        z[d] = -exp(A) * kda_softplus(g[d] + dtb[d]);
        a[d] = kda_gate(g[d], A, dtb[d], lb);
        dec[d] = exp(a[d]);
    }
}

/* one token of the forward recurrence on S (in place); r and u are outputs */
static void token_step(double *S, const double *kh, const double *v, const double *dec, double b, int64_t K,
                       int64_t V, double *r, double *u)
{
    for (int64_t d = 0; d < K; ++d)
        for (int64_t j = 0; j < V; ++j) S[d * V + j] *= dec[d];
    for (int64_t j = 0; j < V; ++j) r[j] = 0.0;
    for (int64_t d = 0; d < K; ++d)
        for (int64_t j = 0; j < V; ++j) r[j] += S[d * V + j] * kh[d];
    for (int64_t j = 0; j < V; ++j) { r[j] = v[j] - r[j]; u[j] = b * r[j]; }
    for (int64_t d = 0; d < K; ++d)
        for (int64_t j = 0; j < V; ++j) S[d * V + j] += kh[d] * u[j];
}

static int seq_rows(const int64_t *cu, int64_t n, int64_t T, int64_t *row0, int64_t *row1)
{
    if (cu) { *row0 = cu[n]; *row1 = cu[n + 1]; }
    else { *row0 = n * T; *row1 = n * T + T; }
    return 0;
}

static int check_args(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, const int64_t *cu, int64_t *N)
{
    if (B < 1 || T < 0 || H < 1 || K < 1 || V < 1) return -2;
    if (cu) {
        if (B != 1 || *N < 1 || cu[0] != 0 || cu[*N] != T) return -3;
        for (int64_t n = 0; n < *N; ++n)
            if (cu[n + 1] < cu[n]) return -3;
    } else {
        *N = B;
    }
    return 0;
}

/*
 * The forward recurrence on fp64 inputs (the same arithmetic as kda_oracle_fwd
 * in kda_oracle.c, whose inputs are bf16 bits): needed so that the gradient can
 * be checked against finite differences of continuous inputs.  Layouts as in
 * kda_oracle_fwd; q, k, g [B,T,H,K], v [B,T,H,V], beta [B,T,H] fp64.
 */
int kda_oracle_fwd_f64(const double *q, const double *k, const double *v, const double *g, const double *beta,
                       int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, const int64_t *cu_seqlens, int64_t N,
                       double scale, const double *A_log, const double *dt_bias, double lower_bound,
                       const double *initial_state, double *final_state, double *out, int num_threads)
{
    if (!q || !k || !v || !g || !beta || !A_log || !dt_bias || !out) return -1;
    const int rc = check_args(B, T, H, K, V, cu_seqlens, &N);
    if (rc) return rc;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t unit = 0; unit < N * H; ++unit) {
        const int64_t n = unit / H, h = unit % H;
        int64_t row0, row1;
        seq_rows(cu_seqlens, n, T, &row0, &row1);
        double *S = malloc(sizeof(double) * (size_t)(K * V));
        double *buf = malloc(sizeof(double) * (size_t)(5 * K + 2 * V));
        if (!S || !buf) {
#pragma omp atomic write
            err = -4;
            free(S); free(buf);
            continue;
        }
        double *qh = buf, *kh = qh + K, *z = kh + K, *a = z + K, *dec = a + K, *r = dec + K, *u = r + V;
        const size_t sidx = (size_t)((n * H + h) * K * V);
        for (int64_t i = 0; i < K * V; ++i) S[i] = initial_state ? initial_state[sidx + (size_t)i] : 0.0;
        for (int64_t row = row0; row < row1; ++row) {
            const size_t qk = (size_t)((row * H + h) * K), vo = (size_t)((row * H + h) * V);
            tok_t t;
            token_acts(q + qk, k + qk, beta[row * H + h], g + qk, A_log[h], dt_bias + h * K, lower_bound, K,
                       qh, kh, z, a, dec, &t);
            token_step(S, kh, v + vo, dec, t.b, K, V, r, u);
            for (int64_t j = 0; j < V; ++j) {
                double s = 0.0;
                for (int64_t d = 0; d < K; ++d) s += S[d * V + j] * qh[d];
                out[vo + (size_t)j] = scale * s;
            }
        }
        if (final_state)
            for (int64_t i = 0; i < K * V; ++i) final_state[sidx + (size_t)i] = S[i];
        free(S); free(buf);
    }
    return err;
}

/*
 * The gradient.  Inputs as kda_oracle_fwd_f64, plus
 *   d_out   : [B,T,H,V] fp64, the loss gradient of every output (required)
 *   d_final : [N,H,K,V] fp64, the loss gradient of the final state, or NULL (zeros)
 * Outputs (all fp64, overwritten):
 *   dq, dk, dg : [B,T,H,K]    dv : [B,T,H,V]    dbeta : [B,T,H]
 *   d_initial  : [N,H,K,V] (may be NULL)    dA_log : [H]    ddt_bias : [H,K]
 * Returns 0 on success, a negative value on a bad argument or allocation failure.
 */
int kda_oracle_bwd_f64(const double *q, const double *k, const double *v, const double *g, const double *beta,
                       int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, const int64_t *cu_seqlens, int64_t N,
                       double scale, const double *A_log, const double *dt_bias, double lower_bound,
                       const double *initial_state, const double *d_out, const double *d_final, double *dq, double *dk,
                       double *dv, double *dg, double *dbeta, double *d_initial, double *dA_log, double *ddt_bias,
                       int num_threads)
{
    if (!q || !k || !v || !g || !beta || !A_log || !dt_bias || !d_out || !dq || !dk || !dv || !dg || !dbeta ||
        !dA_log || !ddt_bias)
        return -1;
    const int rc = check_args(B, T, H, K, V, cu_seqlens, &N);
    if (rc) return rc;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif
    memset(dq, 0, sizeof(double) * (size_t)(B * T * H * K));
    memset(dk, 0, sizeof(double) * (size_t)(B * T * H * K));
    memset(dg, 0, sizeof(double) * (size_t)(B * T * H * K));
    memset(dv, 0, sizeof(double) * (size_t)(B * T * H * V));
    memset(dbeta, 0, sizeof(double) * (size_t)(B * T * H));
    /* per-(sequence, head) partial sums of the shared parameters' gradients */
    double *pA = calloc((size_t)(N * H), sizeof(double));
    double *pdt = calloc((size_t)(N * H * K), sizeof(double));
    if (!pA || !pdt) { free(pA); free(pdt); return -4; }
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t unit = 0; unit < N * H; ++unit) {
        const int64_t n = unit / H, h = unit % H;
        int64_t row0, row1;
        seq_rows(cu_seqlens, n, T, &row0, &row1);
        const int64_t L = row1 - row0;
        const int64_t nb = (L + KDA_ORACLE_CKPT - 1) / KDA_ORACLE_CKPT;
        const size_t KV = (size_t)(K * V);
        double *ck = malloc(sizeof(double) * KV * (size_t)(nb > 0 ? nb : 1));        /* state entering each block */
        double *blk = malloc(sizeof(double) * KV * (size_t)KDA_ORACLE_CKPT);        /* states after each token */
        double *G = malloc(sizeof(double) * KV);
        double *Sp = malloc(sizeof(double) * KV);                                   /* S' of the current token */
        double *buf = malloc(sizeof(double) * (size_t)(8 * K + 3 * V));
        if (!ck || !blk || !G || !Sp || !buf) {
#pragma omp atomic write
            err = -4;
            free(ck); free(blk); free(G); free(Sp); free(buf);
            continue;
        }
        double *qh = buf, *kh = qh + K, *z = kh + K, *a = z + K, *dec = a + K, *dqh = dec + K, *dkh = dqh + K;
        double *tmp = dkh + K, *r = tmp + K, *u = r + V, *du = u + V;
        const size_t sidx = (size_t)((n * H + h) * K * V);
        const double A = A_log[h];
        const double *dtb = dt_bias + h * K;

        /* forward pass: the state entering every block of KDA_ORACLE_CKPT tokens */
        double *S = blk;  /* scratch for the running state */
        for (size_t i = 0; i < KV; ++i) S[i] = initial_state ? initial_state[sidx + i] : 0.0;
        for (int64_t bi = 0; bi < nb; ++bi) {
            memcpy(ck + (size_t)bi * KV, S, sizeof(double) * KV);
            const int64_t r0 = row0 + bi * KDA_ORACLE_CKPT;
            const int64_t r1 = r0 + KDA_ORACLE_CKPT < row1 ? r0 + KDA_ORACLE_CKPT : row1;
            for (int64_t row = r0; row < r1; ++row) {
                const size_t qk = (size_t)((row * H + h) * K), vo = (size_t)((row * H + h) * V);
                tok_t t;
                token_acts(q + qk, k + qk, beta[row * H + h], g + qk, A, dtb, lower_bound, K, qh, kh, z, a, dec, &t);
                token_step(S, kh, v + vo, dec, t.b, K, V, r, u);
            }
        }

        /* reverse pass */
        for (size_t i = 0; i < KV; ++i) G[i] = d_final ? d_final[sidx + i] : 0.0;
        for (int64_t bi = nb - 1; bi >= 0; --bi) {
            const int64_t r0 = row0 + bi * KDA_ORACLE_CKPT;
            const int64_t r1 = r0 + KDA_ORACLE_CKPT < row1 ? r0 + KDA_ORACLE_CKPT : row1;
            /* recompute the block's states after each token */
            memcpy(Sp, ck + (size_t)bi * KV, sizeof(double) * KV);
            for (int64_t row = r0; row < r1; ++row) {
                const size_t qk = (size_t)((row * H + h) * K), vo = (size_t)((row * H + h) * V);
                tok_t t;
                token_acts(q + qk, k + qk, beta[row * H + h], g + qk, A, dtb, lower_bound, K, qh, kh, z, a, dec, &t);
                token_step(Sp, kh, v + vo, dec, t.b, K, V, r, u);
                memcpy(blk + (size_t)(row - r0) * KV, Sp, sizeof(double) * KV);
            }
            for (int64_t row = r1 - 1; row >= r0; --row) {
                const size_t qk = (size_t)((row * H + h) * K), vo = (size_t)((row * H + h) * V);
                const double *Sprev = row > r0 ? blk + (size_t)(row - r0 - 1) * KV : ck + (size_t)bi * KV;
                const double *Snow = blk + (size_t)(row - r0) * KV;
                const double *dov = d_out + vo;
                tok_t t;
                token_acts(q + qk, k + qk, beta[row * H + h], g + qk, A, dtb, lower_bound, K, qh, kh, z, a, dec, &t);
                /* S' = Diag(dec) S_prev, r = v - S'^T kh, u = b r */
                for (int64_t d = 0; d < K; ++d)
                    for (int64_t j = 0; j < V; ++j) Sp[d * V + j] = dec[d] * Sprev[d * V + j];
                for (int64_t j = 0; j < V; ++j) {
                    double s = 0.0;
                    for (int64_t d = 0; d < K; ++d) s += Sp[d * V + j] * kh[d];
                    r[j] = v[vo + (size_t)j] - s;
                    u[j] = t.b * r[j];
                }
                /* o = scale S^T qh */
                for (int64_t d = 0; d < K; ++d) {
                    double s = 0.0;
                    for (int64_t j = 0; j < V; ++j) {
                        G[d * V + j] += scale * qh[d] * dov[j];
                        s += Snow[d * V + j] * dov[j];
                    }
                    dqh[d] = scale * s;
                }
                /* S = S' + kh u^T */
                for (int64_t d = 0; d < K; ++d) {
                    double s = 0.0;
                    for (int64_t j = 0; j < V; ++j) s += G[d * V + j] * u[j];
                    dkh[d] = s;
                }
                for (int64_t j = 0; j < V; ++j) {
                    double s = 0.0;
                    for (int64_t d = 0; d < K; ++d) s += G[d * V + j] * kh[d];
                    du[j] = s;
                }
                /* u = b (v - S'^T kh) */
                double db = 0.0;
                for (int64_t j = 0; j < V; ++j) {
                    dv[vo + (size_t)j] = t.b * du[j];
                    db += du[j] * r[j];
                }
                for (int64_t d = 0; d < K; ++d) {
                    double s = 0.0;
                    for (int64_t j = 0; j < V; ++j) s += Sp[d * V + j] * du[j];
                    dkh[d] -= t.b * s;
                }
                /* dS' = G - b kh du^T; da = rowwise <dS', S'>; G <- Diag(dec) dS' */
                double dz_sum = 0.0;
                for (int64_t d = 0; d < K; ++d) {
                    double da = 0.0;
                    for (int64_t j = 0; j < V; ++j) {
                        const double gs = G[d * V + j] - t.b * kh[d] * du[j];
                        da += gs * Sp[d * V + j];
                        G[d * V + j] = dec[d] * gs;
                    }
                    tmp[d] = da;
                }
                /* the input activations */
                double qd = 0.0, kd = 0.0;
                for (int64_t d = 0; d < K; ++d) { qd += q[qk + d] * dqh[d]; kd += k[qk + d] * dkh[d]; }
                const double rq3 = t.rq * t.rq * t.rq, rk3 = t.rk * t.rk * t.rk;
                for (int64_t d = 0; d < K; ++d) {
                    dq[qk + d] = t.rq * dqh[d] - rq3 * qd * q[qk + d];
                    dk[qk + d] = t.rk * dkh[d] - rk3 * kd * k[qk + d];
                }
                dbeta[row * H + h] = db * t.b * (1.0 - t.b);
                for (int64_t d = 0; d < K; ++d) {
                    if (z[d] > lower_bound) {
                        const double dx = -exp(A) * kda_sigmoid(g[qk + d] + dtb[d]) * tmp[d];
                        dg[qk + d] = dx;
                        pdt[(size_t)(unit * K + d)] += dx;
                        dz_sum += z[d] * tmp[d];
                    } else {
                        dg[qk + d] = 0.0;
                    }
                }
                pA[unit] += dz_sum;
            }
        }
        if (d_initial)
            for (size_t i = 0; i < KV; ++i) d_initial[sidx + i] = G[i];
        free(ck); free(blk); free(G); free(Sp); free(buf);
    }
    for (int64_t h = 0; h < H; ++h) {
        double s = 0.0;
        for (int64_t n = 0; n < N; ++n) s += pA[n * H + h];
        dA_log[h] = s;
        for (int64_t d = 0; d < K; ++d) {
            double t = 0.0;
            for (int64_t n = 0; n < N; ++n) t += pdt[(size_t)((n * H + h) * K + d)];
            ddt_bias[h * K + d] = t;
        }
    }
    free(pA); free(pdt);
    return err;
}
