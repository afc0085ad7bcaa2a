/*
 * fp64 CPU oracle for the Kimi Delta Attention (KDA) recurrence.
 * TEST INFRASTRUCTURE ONLY: nothing on the product path links or loads this file.
 *
 * It is the same plain token-by-token recurrence as kda_ref.py, written in C so the
 * full-size workloads (96 heads x 128 x 128 states, up to 65,536 tokens) finish in
 * seconds.  OpenMP runs independent (sequence, head) units in parallel; inside a unit
 * the tokens are taken strictly in order and each step is the definition, unfused:
 *
 *   (nnterp Kimi-Linear page, Notes on KDA's per-key-channel decay, and section 04)
 *   k <- k / sqrt(sum k^2 + eps);  q <- q / sqrt(sum q^2 + eps) / sqrt(dk)
 *   S[i][:] *= exp(g[i])                      decay each key channel first
 *   r[j]     = sum_i k[i] S[i][j]             k^T S
 *   S[i][j] += k[i] * beta * (v[j] - r[j])    delta-rule removal and write
 *   o[j]     = sum_i q[i] S[i][j]             read the updated state
 *
 * A zero in the padding mask skips the token (state unchanged, output zero);
 * cu_seqlens restarts the state per sequence from that sequence's initial state.
 * Inputs are read in their stored precision (fp32, or bf16 widened exactly); all
 * arithmetic is fp64.  Parity status: pinned against kda_ref.py and the closed forms
 * in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double load_in(const void *p, int bf16, size_t idx) {
    if (bf16) {
        uint32_t bits = ((uint32_t)((const uint16_t *)p)[idx]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float *)p)[idx];
}

/* Returns 0 on success, 1 on bad arguments, 2 on allocation failure. */
int kda_oracle_recurrence(int B, int T, int H, int dk, int dv, int in_bf16,
                          const void *q, const void *k, const void *v,
                          const float *g, const float *beta, const float *initial_state,
                          const int32_t *cu_seqlens, int num_seqs, const uint8_t *mask,
                          double scale, int use_qk_l2norm, double l2_eps,
                          const int32_t *heads, int n_heads,
                          double *o, double *final_state, int num_threads) {
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0 || n_heads <= 0) return 1;
    if (cu_seqlens && (B != 1 || mask)) return 1;
    const int N = cu_seqlens ? num_seqs : B;
    const long units = (long)N * n_heads;
    int bad = 0;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif
    /* Outputs of skipped (padding) tokens are zero. */
    memset(o, 0, sizeof(double) * (size_t)B * T * n_heads * dv);

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (long unit = 0; unit < units; ++unit) {
        const int n = (int)(unit / n_heads);
        const int hs = (int)(unit % n_heads);            /* index into the head subset */
        const int h = heads ? heads[hs] : hs;            /* head in the full tensors   */
        const int b = cu_seqlens ? 0 : n;
        const int t0 = cu_seqlens ? cu_seqlens[n] : 0;
        const int t1 = cu_seqlens ? cu_seqlens[n + 1] : T;
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *kk = (double *)malloc(sizeof(double) * (size_t)dk);
        double *qq = (double *)malloc(sizeof(double) * (size_t)dk);
        double *r = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !kk || !qq || !r) {
            bad |= 1;
        } else {
            if (initial_state) {
                const float *s0 = initial_state + ((size_t)n * H + h) * dk * dv;
                for (long e = 0; e < (long)dk * dv; ++e) S[e] = (double)s0[e];
            } else {
                memset(S, 0, sizeof(double) * (size_t)dk * dv);
            }
            for (int t = t0; t < t1; ++t) {
                if (mask && mask[(size_t)b * T + t] == 0) continue;
                const size_t tok = ((size_t)b * T + t) * H + h;
                double kn = 0.0, qn = 0.0;
                for (int i = 0; i < dk; ++i) {
                    kk[i] = load_in(k, in_bf16, tok * dk + i);
                    qq[i] = load_in(q, in_bf16, tok * dk + i);
                    kn += kk[i] * kk[i];
                    qn += qq[i] * qq[i];
                }
                const double kinv = use_qk_l2norm ? 1.0 / sqrt(kn + l2_eps) : 1.0;
                const double qinv = (use_qk_l2norm ? 1.0 / sqrt(qn + l2_eps) : 1.0) * scale;
                for (int i = 0; i < dk; ++i) {
                    kk[i] *= kinv;
                    qq[i] *= qinv;
                }
                /* decay */
                for (int i = 0; i < dk; ++i) {
                    const double a = exp((double)g[tok * dk + i]);
                    double *row = S + (size_t)i * dv;
                    for (int j = 0; j < dv; ++j) row[j] *= a;
                }
                /* r = k^T S */
                for (int j = 0; j < dv; ++j) r[j] = 0.0;
                for (int i = 0; i < dk; ++i) {
                    const double ki = kk[i];
                    const double *row = S + (size_t)i * dv;
                    for (int j = 0; j < dv; ++j) r[j] += ki * row[j];
                }
                /* u = beta (v - r), kept in r */
                const double bt = (double)beta[tok];
                for (int j = 0; j < dv; ++j) r[j] = bt * (load_in(v, in_bf16, tok * dv + j) - r[j]);
                /* S += k u^T */
                for (int i = 0; i < dk; ++i) {
                    const double ki = kk[i];
                    double *row = S + (size_t)i * dv;
                    for (int j = 0; j < dv; ++j) row[j] += ki * r[j];
                }
                /* o = S^T q */
                double *out = o + (((size_t)b * T + t) * n_heads + hs) * dv;
                for (int i = 0; i < dk; ++i) {
                    const double qi = qq[i];
                    const double *row = S + (size_t)i * dv;
                    for (int j = 0; j < dv; ++j) out[j] += qi * row[j];
                }
            }
            memcpy(final_state + ((size_t)n * n_heads + hs) * dk * dv, S,
                   sizeof(double) * (size_t)dk * dv);
        }
        free(S);
        free(kk);
        free(qq);
        free(r);
    }
    return bad ? 2 : 0;
}

int kda_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
