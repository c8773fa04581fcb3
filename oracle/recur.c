/*
 * Oracle: token-by-token gated delta rule in fp64 (TEST INFRASTRUCTURE ONLY).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this file's library. It shares no code with the HIP path.
 *
 * What it computes (state kept as a K x V matrix, the orientation the
 * hyper-parallel "Diff Coverage" page of 2026-09-10 uses for its recurrent
 * state in torch_chunk_gated_delta_rule and _gdn_state_p2p_summary):
 *
 *   for every sequence n and head h, S = S0[n,h] (or zero), then per token t
 *     q^, k^  = q_t, k_t                       (bf16 widened exactly)
 *     if L2NORM: x^ = x / sqrt(sum(x*x) + 1e-6)  (the _l2norm helper, same page)
 *     b       = beta_t, or 1/(1+exp(-beta_t)) if BETA_SIGMOID
 *     decay   GDN: S <- exp(g_t) S
 *             KDA: S[d,:] <- 2^(g_t[d]) S[d,:]   (per key channel, log2 gate)
 *     S       <- S + b k^ (v_t - S^T k^)^T       (delta rule)
 *     o_t     = scale * S^T q^
 *   final_state[n,h] = S
 *
 * This is the recurrence S_t = e^{g_t} S_{t-1}(I - b k k^T) + b v k^T,
 * o_t = scale S_t q_t written in the K x V orientation. The chunked form on
 * the same page is an algebraic rewrite of it (checked by the tests).
 *
 * Sequences: dense (cu == NULL) sequence n is batch row n, tokens
 * [n*T, n*T+T); packed (cu != NULL, B == 1) sequence n is tokens
 * [cu[n], cu[n+1]).
 *
 * Pins: see tests/test_oracle_pins.py (chunk-form equivalence, beta=0 closed
 * form, retrieval, reset, affinity in S0, per-document independence, KDA/GDN
 * reduction, the hand-derived fixtures under tests/golden/).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_L2NORM 1u
#define ORACLE_BETA_SIGMOID 2u

static double bf16_to_f64(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static void load_row(const uint16_t* src, int n, int l2norm, double* dst) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) {
        dst[i] = bf16_to_f64(src[i]);
        ss += dst[i] * dst[i];
    }
    if (l2norm) {
        double r = 1.0 / sqrt(ss + 1e-6);
        for (int i = 0; i < n; ++i) dst[i] *= r;
    }
}

/*
 * Runs the recurrence for the listed (sequence, head) units.
 *   units: int32 pairs (n, h); NULL means every unit, n-major.
 *   o: fp64 [B*T, H, V] (token-major); only the rows of the listed units are written.
 *   final_state: fp64 [N, H, K, V] or NULL.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_recur(int kda, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                 const float* g, const uint16_t* beta, const float* initial_state,
                 const int32_t* cu, int N, int B, int T, int H, int K, int V,
                 double scale, unsigned flags, const int32_t* units, int n_units,
                 double* o, double* final_state) {
    if (K <= 0 || V <= 0 || H <= 0 || N <= 0) return -1;
    if (cu == NULL && N != B) return -1;
    int total_units = units ? n_units : N * H;
    int l2 = (flags & ORACLE_L2NORM) != 0;
    int sig = (flags & ORACLE_BETA_SIGMOID) != 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < total_units; ++u) {
        int n = units ? units[2 * u] : u / H;
        int h = units ? units[2 * u + 1] : u % H;
        long t0 = cu ? cu[n] : (long)n * T;
        long t1 = cu ? cu[n + 1] : (long)n * T + T;
        double* S = (double*)malloc(sizeof(double) * (size_t)K * V);
        double* qh = (double*)malloc(sizeof(double) * (size_t)K);
        double* kh = (double*)malloc(sizeof(double) * (size_t)K);
        double* vt = (double*)malloc(sizeof(double) * (size_t)V);
        double* pred = (double*)malloc(sizeof(double) * (size_t)V);
        for (long i = 0; i < (long)K * V; ++i)
            S[i] = initial_state ? (double)initial_state[((size_t)n * H + h) * K * V + i] : 0.0;

        for (long t = t0; t < t1; ++t) {
            size_t th = (size_t)t * H + h;
            load_row(q + th * K, K, l2, qh);
            load_row(k + th * K, K, l2, kh);
            for (int j = 0; j < V; ++j) vt[j] = bf16_to_f64(v[th * V + j]);
            double b = bf16_to_f64(beta[th]);
            if (sig) b = 1.0 / (1.0 + exp(-b));

            /* decay */
            if (kda) {
                for (int d = 0; d < K; ++d) {
                    double f = exp2((double)g[th * K + d]);
                    for (int j = 0; j < V; ++j) S[(size_t)d * V + j] *= f;
                }
            } else {
                double f = exp((double)g[th]);
                for (long i = 0; i < (long)K * V; ++i) S[i] *= f;
            }
            /* delta rule: S += b k (v - S^T k)^T */
            for (int j = 0; j < V; ++j) pred[j] = 0.0;
            for (int d = 0; d < K; ++d)
                for (int j = 0; j < V; ++j) pred[j] += S[(size_t)d * V + j] * kh[d];
            for (int d = 0; d < K; ++d) {
                double bk = b * kh[d];
                for (int j = 0; j < V; ++j) S[(size_t)d * V + j] += bk * (vt[j] - pred[j]);
            }
            /* output */
            double* orow = o + th * V;
            for (int j = 0; j < V; ++j) orow[j] = 0.0;
            for (int d = 0; d < K; ++d)
                for (int j = 0; j < V; ++j) orow[j] += S[(size_t)d * V + j] * qh[d];
            for (int j = 0; j < V; ++j) orow[j] *= scale;
        }
        if (final_state) {
            double* dst = final_state + ((size_t)n * H + h) * K * V;
            memcpy(dst, S, sizeof(double) * (size_t)K * V);
        }
        free(S); free(qh); free(kh); free(vt); free(pred);
    }
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
