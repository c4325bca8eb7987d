/*
 * kda_oracle.c -- plain, slow, fp64 CPU oracle for the Kimi Delta Attention
 * (KDA) state recurrence.  TEST INFRASTRUCTURE ONLY: it exists so that the
 * GPU kernels can be checked against an obviously correct definition.  Only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it; the product library never calls it and shares no code with it.
 *
 * Everything here is written straight from the definitions on the pages:
 *
 *  - "Kimi K3: Bounded Decay and Delta Memory" (PaperLeet exercise),
 *    section "Formula and conventions": the bounded gate
 *        g = g_min * sigmoid(e^A * z),   alpha = e^g,
 *    and the per-token fade / correct / read recurrence
 *        Sbar_t = Diag(alpha_t) S_{t-1}
 *        S_t    = Sbar_t + beta_t k_t (v_t - k_t^T Sbar_t)^T
 *        o_t    = S_t^T q_t,
 *    plus its argument-contract table (shapes, empty sequence, initial
 *    state omitted means zeros, the scan itself applies no scale to q).
 *  - "KDARecurrent" page, section "The state recurrence in source order":
 *    the same loop order (decay rows indexed by key features, predict with
 *    the decayed state, rank-one correction scaled by beta, read after write)
 *    and "Decay and write strength" for the bias (dt_bias) that is added to
 *    the gate input before the per-head positive scale.
 *
 * The method is exact: a chunkwise evaluation reaches the same numbers up
 * to rounding order, so the oracle is the token-by-token definition, not a
 * chunked algorithm.  Arithmetic is IEEE double with libm exp; the only
 * parallelism is OpenMP over independent (sequence, head) pairs, which
 * does not change any result.
 *
 * Parity status: every function here is pinned by CPU tests (worked
 * example, closed forms, invariants, an independent matrix-form
 * recurrence); nothing is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Logistic sigmoid, evaluated in the branch that never overflows exp(). */
static double sigmoid(double x) {
    if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/*
 * Bounded per-channel decay (PaperLeet "Formula and conventions", the
 * bounded_decay operator; KDA cheat sheet, table "Lower-bounded decay -- the
 * g_min trick", column "Kimi K3").
 *   z        [rows, H, K]   decay logits (rows = B*T)
 *   log_scale[H]            per-head A (the scale applied is e^A)
 *   bias     [H*K] or NULL  featurewise offset added to z before scaling
 *   g_min    < 0            lower bound of the log-decay
 *   out_log  0: write alpha = e^g (retention), 1: write g = ln alpha
 */
void kda_oracle_bounded_decay(const double *z, const double *log_scale, const double *bias,
                              double g_min, int64_t rows, int64_t H, int64_t K, int out_log,
                              double *out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t h = 0; h < H; ++h) {
            double scale = exp(log_scale[h]);
            for (int64_t c = 0; c < K; ++c) {
                int64_t i = (r * H + h) * K + c;
                double x = z[i] + (bias ? bias[h * K + c] : 0.0);
                double g = g_min * sigmoid(scale * x);
                out[i] = out_log ? g : exp(g);
            }
        }
}

/*
 * One (sequence, head) pair of the recurrence, token by token.
 * Rows t0 .. t0+len-1 of the [*, T, H, *] token tensors are this sequence.
 * S is a K x V row-major scratch holding the state (key rows, value columns).
 */
static void scan_pair(const double *q, const double *k, const double *v, const double *alpha,
                      const double *beta, const double *s0, int64_t t0, int64_t len, int64_t h,
                      int64_t H, int64_t K, int64_t V, double scale, double *out, double *s_final,
                      double *S, double *pred) {
    if (s0)
        memcpy(S, s0, (size_t)(K * V) * sizeof(double));
    else
        memset(S, 0, (size_t)(K * V) * sizeof(double));

    for (int64_t t = t0; t < t0 + len; ++t) {
        const double *kt = k + (t * H + h) * K;
        const double *qt = q + (t * H + h) * K;
        const double *vt = v + (t * H + h) * V;
        const double *at = alpha + (t * H + h) * K;
        double bt = beta[t * H + h];

        /* fade: every key row c of the state is multiplied by alpha_t[c] */
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j) S[c * V + j] *= at[c];

        /* predict: what the faded memory returns for k_t, i.e. Sbar^T k_t */
        for (int64_t j = 0; j < V; ++j) pred[j] = 0.0;
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j) pred[j] += S[c * V + j] * kt[c];

        /* correct: S += beta_t * k_t (v_t - prediction)^T */
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j) S[c * V + j] += bt * kt[c] * (vt[j] - pred[j]);

        /* read after write: o_t = scale * S_t^T q_t */
        double *ot = out + (t * H + h) * V;
        for (int64_t j = 0; j < V; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < K; ++c) acc += S[c * V + j] * qt[c];
            ot[j] = scale * acc;
        }
    }
    if (s_final) memcpy(s_final, S, (size_t)(K * V) * sizeof(double));
}

/*
 * The full scan (PaperLeet recurrent_kda contract).
 *   q, k     [B, T, H, K];  v [B, T, H, V];  alpha [B, T, H, K];  beta [B, T, H]
 *   initial_state [N, H, K, V] or NULL (zeros);  final_state [N, H, K, V] or NULL
 *   cu_seqlens NULL: N = B independent batch rows of length T.
 *   cu_seqlens [num_seqs + 1] (B must be 1): sequence s is rows
 *              cu_seqlens[s] .. cu_seqlens[s+1]-1 of the single batch row, and
 *              its state restarts from initial_state[s] (or zeros).
 *   out [B, T, H, V]; scale multiplies the read (1.0 leaves q unscaled).
 * Returns 0, or -1 on an inconsistent argument (nothing is written then).
 */
int kda_oracle_scan(const double *q, const double *k, const double *v, const double *alpha,
                    const double *beta, const double *initial_state, const int64_t *cu_seqlens,
                    int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                    double scale, double *out, double *final_state, int nthreads) {
    if (B < 0 || T < 0 || H <= 0 || K <= 0 || V <= 0) return -1;
    int64_t N = cu_seqlens ? num_seqs : B;
    if (cu_seqlens) {
        if (B != 1 || num_seqs < 0 || cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != T) return -1;
        for (int64_t s = 0; s < num_seqs; ++s)
            if (cu_seqlens[s + 1] < cu_seqlens[s]) return -1;
    }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int64_t pairs = N * H;
#pragma omp parallel
    {
        double *S = (double *)malloc((size_t)(K * V) * sizeof(double));
        double *pred = (double *)malloc((size_t)V * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t p = 0; p < pairs; ++p) {
            int64_t s = p / H, h = p % H;
            int64_t t0, len;
            if (cu_seqlens) {
                t0 = cu_seqlens[s];
                len = cu_seqlens[s + 1] - cu_seqlens[s];
            } else {
                t0 = s * T; /* batch row s: rows s*T .. s*T+T-1 of the flattened [B*T] axis */
                len = T;
            }
            const double *s0 = initial_state ? initial_state + (s * H + h) * K * V : NULL;
            double *sf = final_state ? final_state + (s * H + h) * K * V : NULL;
            scan_pair(q, k, v, alpha, beta, s0, t0, len, h, H, K, V, scale, out, sf, S, pred);
        }
        free(S);
        free(pred);
    }
    return 0;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int kda_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
