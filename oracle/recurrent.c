/*
 * Oracle (test infrastructure only; never part of the product path).
 *
 * Plain fp64 per-token evaluation of the gated delta rule, written from the
 * update rule on the page "PyPTO-Gym 的 chunk_kda 算子实战" (section 算子定位与算法背景):
 * for every token, first decay the state by exp(g), then apply the delta
 * correction with weight beta, then read the output from the updated state:
 *
 *     S <- diag(exp(g_t)) S                      S is K x V, g_t in R^K (or a scalar)
 *     S <- S + beta_t * k_t (v_t - S^T k_t)^T     the read uses the decayed S
 *     o_t <- scale * S^T q_t                      read after the update
 *
 * The interface follows that page's I/O table (section 算子签名与 I/O 规格), with
 * H value heads sharing Hk query/key heads (value head h reads key head h / (H / Hk);
 * Hk == H is the plain case):
 *   q, k      [B*T, Hk, K]  bf16 (passed as raw uint16 bit patterns)
 *   v         [B*T, H, V]   bf16
 *   g         [B*T, H, K] fp32 (per-dimension gate) or [B*T, H] fp32 (per-head gate)
 *   beta      [B*T, H]      fp32
 *   s0        [N, H, V, K]  fp64 or NULL (zeros); the page's state layout is the
 *             transpose of the internal K x V matrix
 * With qk_l2norm (the page's use_qk_l2norm_in_kernel switch, section 测试与验证体系),
 * q_t and k_t are first replaced by x / sqrt(sum_d x_d^2 + 1e-6).
 *   cu        [N+1]         int32 sequence offsets into the packed token axis, or
 *             NULL, in which case the N = B sequences have T tokens each
 *   o         [B*T, H, V]   fp64 output
 *   s_out     [N, H, V, K]  fp64 final state (may be NULL)
 *
 * Every (sequence, head) pair is an independent chain; chains are spread over
 * OpenMP threads with a static schedule. Inputs are widened to fp64 exactly.
 * Returns 0 on success, a negative value on bad arguments.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_to_f64(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_recurrent_fwd(int B, int T, int Hk, int H, int K, int V, int N, int gate_per_dim,
                         int qk_l2norm, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const float* g, const float* beta, const double* s0,
                         const int32_t* cu, double scale, double* o, double* s_out,
                         int nthreads) {
    if (B <= 0 || T < 0 || H <= 0 || Hk <= 0 || H % Hk != 0 || K <= 0 || V <= 0 || N <= 0) return -1;
    if (!q || !k || !v || !g || !beta || !o) return -2;
    if (cu == NULL && N != B) return -3;
    const long long total = (long long)B * T;
    if (cu != NULL) {
        if (B != 1) return -4;
        if (cu[0] != 0 || cu[N] != total) return -5;
        for (int n = 0; n < N; ++n)
            if (cu[n + 1] < cu[n]) return -6;
    }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const long long chains = (long long)N * H;
    int err = 0;
#pragma omp parallel for schedule(static)
    for (long long c = 0; c < chains; ++c) {
        const int n = (int)(c / H), h = (int)(c % H);
        const long long bos = cu ? cu[n] : (long long)n * T;
        const long long eos = cu ? cu[n + 1] : (long long)(n + 1) * T;
        double* S = (double*)malloc(sizeof(double) * (size_t)K * V);     /* S[kk*V + vv] */
        double* kt = (double*)malloc(sizeof(double) * (size_t)K);
        double* qt = (double*)malloc(sizeof(double) * (size_t)K);
        double* dl = (double*)malloc(sizeof(double) * (size_t)V);
        if (!S || !kt || !qt || !dl) {
#pragma omp atomic write
            err = 1;
            free(S); free(kt); free(qt); free(dl);
            continue;
        }
        /* internal state is the transpose of the [V, K] interface layout */
        for (int kk = 0; kk < K; ++kk)
            for (int vv = 0; vv < V; ++vv)
                S[(size_t)kk * V + vv] =
                    s0 ? s0[(((size_t)n * H + h) * V + vv) * K + kk] : 0.0;
        for (long long t = bos; t < eos; ++t) {
            const size_t row = (size_t)t * H + h;
            const size_t krow = (size_t)t * Hk + h / (H / Hk);
            /* 1. decay each row of S by exp(g) */
            for (int kk = 0; kk < K; ++kk) {
                const double gv = gate_per_dim ? (double)g[row * K + kk] : (double)g[row];
                const double d = exp(gv);
                for (int vv = 0; vv < V; ++vv) S[(size_t)kk * V + vv] *= d;
            }
            /* 2. delta correction: S += beta k (v - S^T k)^T */
            for (int kk = 0; kk < K; ++kk) {
                kt[kk] = bf16_to_f64(k[krow * K + kk]);
                qt[kk] = bf16_to_f64(q[krow * K + kk]);
            }
            if (qk_l2norm) {
                double sk = 0.0, sq = 0.0;
                for (int kk = 0; kk < K; ++kk) {
                    sk += kt[kk] * kt[kk];
                    sq += qt[kk] * qt[kk];
                }
                const double fk = 1.0 / sqrt(sk + 1e-6), fq = 1.0 / sqrt(sq + 1e-6);
                for (int kk = 0; kk < K; ++kk) {
                    kt[kk] *= fk;
                    qt[kk] *= fq;
                }
            }
            const double b = (double)beta[row];
            for (int vv = 0; vv < V; ++vv) {
                double pred = 0.0;
                for (int kk = 0; kk < K; ++kk) pred += S[(size_t)kk * V + vv] * kt[kk];
                dl[vv] = b * (bf16_to_f64(v[row * V + vv]) - pred);
            }
            for (int kk = 0; kk < K; ++kk)
                for (int vv = 0; vv < V; ++vv) S[(size_t)kk * V + vv] += kt[kk] * dl[vv];
            /* 3. output from the updated state */
            for (int vv = 0; vv < V; ++vv) {
                double acc = 0.0;
                for (int kk = 0; kk < K; ++kk) acc += S[(size_t)kk * V + vv] * qt[kk];
                o[row * V + vv] = scale * acc;
            }
        }
        if (s_out)
            for (int kk = 0; kk < K; ++kk)
                for (int vv = 0; vv < V; ++vv)
                    s_out[(((size_t)n * H + h) * V + vv) * K + kk] = S[(size_t)kk * V + vv];
        free(S); free(kt); free(qt); free(dl);
    }
    return err ? -7 : 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
