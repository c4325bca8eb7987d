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
 * The gradients (kda_oracle_scan_bwd, kda_oracle_bounded_decay_bwd) are the
 * reverse-mode derivatives of the same token loop and gate, written out step by
 * step; PaperLeet's "Return requirements" ask for gradients into every input.
 *
 * Parity status: every function here is pinned by CPU tests (worked
 * example, closed forms, invariants, an independent matrix-form
 * recurrence; the gradients by element-wise central finite differences of
 * the forward functions and by closed forms); nothing is "parity unpinned".
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

/*
 * Gradients of the bounded decay (PaperLeet "Return requirements": bounded_decay keeps
 * gradients into logits and log_scale; the function is g = g_min sigmoid(x),
 * x = e^A (z + bias), alpha = e^g, differentiated by the chain rule):
 *   dg = grad (grad_is_log) or grad * alpha (grad is dL/dalpha)
 *   dx = dg * g_min * sigmoid(x) (1 - sigmoid(x)),  dz = dx * e^A
 *   dbias[h,c] = sum over rows of dz,  dlog_scale[h] = sum over rows and c of dx * x
 * dlog_scale and dbias may be NULL (not wanted); they are overwritten, not accumulated.
 */
void kda_oracle_bounded_decay_bwd(const double *z, const double *log_scale, const double *bias,
                                  double g_min, int64_t rows, int64_t H, int64_t K,
                                  const double *grad, int grad_is_log, double *dz,
                                  double *dlog_scale, double *dbias) {
    if (dlog_scale)
        for (int64_t h = 0; h < H; ++h) dlog_scale[h] = 0.0;
    if (dbias)
        for (int64_t i = 0; i < H * K; ++i) dbias[i] = 0.0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t h = 0; h < H; ++h) {
            double e = exp(log_scale[h]);
            for (int64_t c = 0; c < K; ++c) {
                int64_t i = (r * H + h) * K + c;
                double x = e * (z[i] + (bias ? bias[h * K + c] : 0.0));
                double s = sigmoid(x);
                double g = g_min * s;
                double dg = grad_is_log ? grad[i] : grad[i] * exp(g);
                double dx = dg * g_min * s * (1.0 - s);
                dz[i] = dx * e;
                if (dbias) dbias[h * K + c] += dx * e;
                if (dlog_scale) dlog_scale[h] += dx * x;
            }
        }
}

/*
 * The state update of one token (fade, predict, correct; no read), used by the
 * backward pass to rebuild the states it needs.
 */
static void advance(double *S, const double *kt, const double *vt, const double *at, double bt,
                    int64_t K, int64_t V, double *pred) {
    for (int64_t c = 0; c < K; ++c)
        for (int64_t j = 0; j < V; ++j) S[c * V + j] *= at[c];
    for (int64_t j = 0; j < V; ++j) pred[j] = 0.0;
    for (int64_t c = 0; c < K; ++c)
        for (int64_t j = 0; j < V; ++j) pred[j] += S[c * V + j] * kt[c];
    for (int64_t c = 0; c < K; ++c)
        for (int64_t j = 0; j < V; ++j) S[c * V + j] += bt * kt[c] * (vt[j] - pred[j]);
}

#define BWD_SEG 64 /* tokens between stored states in the backward pass */

/*
 * Reverse-mode derivative of one (sequence, head) pair (PaperLeet "Return requirements":
 * gradients reach q, k, v, alpha, beta and the initial state through every non-empty
 * scan).  The loss seen is L = <d_out, out> + <d_final, S_T>.  Walking the tokens
 * backwards with dS = dL/dS_t:
 *   read     o_t = scale S_t^T q_t:       dq_t = scale S_t do_t,  dS += scale q_t do_t^T
 *   correct  S_t = P + beta_t k_t delta^T, P = Diag(alpha_t) S_{t-1}, delta = v_t - P^T k_t:
 *            dbeta_t = k_t^T dS delta,  dk_t = beta_t dS delta,  ddelta = beta_t dS^T k_t,
 *            dv_t = ddelta,  dP = dS - k_t ddelta^T,  dk_t -= P ddelta
 *   fade     dalpha_t[c] = sum_j dP[c,j] S_{t-1}[c,j],  dS_{t-1} = Diag(alpha_t) dP.
 * The states S_{t-1}, S_t are rebuilt from copies stored every BWD_SEG tokens (a
 * replay of the same arithmetic, so they equal the forward's states exactly).
 * work: (nseg + BWD_SEG + 3) * K * V + 3 * V doubles, nseg = ceil(len / BWD_SEG).
 */
static void bwd_pair(const double *q, const double *k, const double *v, const double *alpha,
                     const double *beta, const double *s0, const double *dout, const double *dsT,
                     int64_t t0, int64_t len, int64_t h, int64_t H, int64_t K, int64_t V,
                     double scale, double *dq, double *dk, double *dv, double *dalpha,
                     double *dbeta, double *ds0, double *work) {
    const int64_t KV = K * V;
    int64_t nseg = (len + BWD_SEG - 1) / BWD_SEG;
    double *ckpt = work;                     /* nseg states: the state before each segment */
    double *st = ckpt + nseg * KV;           /* BWD_SEG + 1 states of the replayed segment */
    double *dS = st + (BWD_SEG + 1) * KV;
    double *dP = dS + KV;
    double *pred = dP + KV, *delta = pred + V, *dd = delta + V;

    double *S = st; /* forward pass: store the checkpoints */
    if (s0)
        memcpy(S, s0, (size_t)KV * sizeof(double));
    else
        memset(S, 0, (size_t)KV * sizeof(double));
    for (int64_t i = 0; i < nseg; ++i) {
        memcpy(ckpt + i * KV, S, (size_t)KV * sizeof(double));
        int64_t a = t0 + i * BWD_SEG, b = a + BWD_SEG < t0 + len ? a + BWD_SEG : t0 + len;
        for (int64_t t = a; t < b; ++t)
            advance(S, k + (t * H + h) * K, v + (t * H + h) * V, alpha + (t * H + h) * K, beta[t * H + h],
                    K, V, pred);
    }

    if (dsT)
        memcpy(dS, dsT, (size_t)KV * sizeof(double));
    else
        memset(dS, 0, (size_t)KV * sizeof(double));
    for (int64_t i = nseg - 1; i >= 0; --i) {
        int64_t a = t0 + i * BWD_SEG, b = a + BWD_SEG < t0 + len ? a + BWD_SEG : t0 + len;
        memcpy(st, ckpt + i * KV, (size_t)KV * sizeof(double));
        for (int64_t t = a; t < b; ++t) {
            double *nx = st + (t - a + 1) * KV;
            memcpy(nx, nx - KV, (size_t)KV * sizeof(double));
            advance(nx, k + (t * H + h) * K, v + (t * H + h) * V, alpha + (t * H + h) * K, beta[t * H + h],
                    K, V, pred);
        }
        for (int64_t t = b - 1; t >= a; --t) {
            const double *Sprev = st + (t - a) * KV, *Scur = Sprev + KV;
            const double *kt = k + (t * H + h) * K, *qt = q + (t * H + h) * K;
            const double *vt = v + (t * H + h) * V, *at = alpha + (t * H + h) * K;
            const double *dot = dout + (t * H + h) * V;
            double bt = beta[t * H + h];

            /* read */
            for (int64_t c = 0; c < K; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < V; ++j) acc += Scur[c * V + j] * dot[j];
                dq[(t * H + h) * K + c] = scale * acc;
            }
            for (int64_t c = 0; c < K; ++c)
                for (int64_t j = 0; j < V; ++j) dS[c * V + j] += scale * qt[c] * dot[j];

            /* correct: delta = v_t - P^T k_t with P = Diag(alpha_t) S_{t-1} */
            for (int64_t j = 0; j < V; ++j) {
                double acc = 0.0;
                for (int64_t c = 0; c < K; ++c) acc += at[c] * Sprev[c * V + j] * kt[c];
                delta[j] = vt[j] - acc;
            }
            double db = 0.0;
            for (int64_t c = 0; c < K; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < V; ++j) acc += dS[c * V + j] * delta[j];
                db += kt[c] * acc;
                dk[(t * H + h) * K + c] = bt * acc;
            }
            dbeta[t * H + h] = db;
            for (int64_t j = 0; j < V; ++j) {
                double acc = 0.0;
                for (int64_t c = 0; c < K; ++c) acc += dS[c * V + j] * kt[c];
                dd[j] = bt * acc;
                dv[(t * H + h) * V + j] = dd[j];
            }
            for (int64_t c = 0; c < K; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < V; ++j) {
                    dP[c * V + j] = dS[c * V + j] - kt[c] * dd[j];
                    acc += at[c] * Sprev[c * V + j] * dd[j];
                }
                dk[(t * H + h) * K + c] -= acc;
            }

            /* fade */
            for (int64_t c = 0; c < K; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < V; ++j) acc += dP[c * V + j] * Sprev[c * V + j];
                dalpha[(t * H + h) * K + c] = acc;
                for (int64_t j = 0; j < V; ++j) dS[c * V + j] = at[c] * dP[c * V + j];
            }
        }
    }
    if (ds0) memcpy(ds0, dS, (size_t)KV * sizeof(double));
}

/*
 * Gradients of kda_oracle_scan for L = <d_out, out> + <d_final_state, final_state>.
 * Arguments as kda_oracle_scan, plus d_out [B, T, H, V] and d_final_state [N, H, K, V]
 * (NULL = zeros); outputs dq, dk [B, T, H, K], dv [B, T, H, V], dalpha [B, T, H, K],
 * dbeta [B, T, H] and d_initial_state [N, H, K, V] (NULL = not wanted; for an
 * omitted initial state it is the gradient at the zero state).  An empty sequence
 * passes d_final_state through to d_initial_state.  Returns 0, or -1 as kda_oracle_scan.
 */
int kda_oracle_scan_bwd(const double *q, const double *k, const double *v, const double *alpha,
                        const double *beta, const double *initial_state, const int64_t *cu_seqlens,
                        int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                        double scale, const double *d_out, const double *d_final_state, double *dq,
                        double *dk, double *dv, double *dalpha, double *dbeta,
                        double *d_initial_state, int nthreads) {
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
    int64_t maxlen = cu_seqlens ? 0 : T;
    for (int64_t s = 0; cu_seqlens && s < num_seqs; ++s)
        if (cu_seqlens[s + 1] - cu_seqlens[s] > maxlen) maxlen = cu_seqlens[s + 1] - cu_seqlens[s];
    int64_t nseg = (maxlen + BWD_SEG - 1) / BWD_SEG;
    size_t wsize = (size_t)((nseg + BWD_SEG + 3) * K * V + 3 * V);
    int64_t pairs = N * H;
#pragma omp parallel
    {
        double *work = (double *)malloc(wsize * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t p = 0; p < pairs; ++p) {
            int64_t s = p / H, h = p % H;
            int64_t t0 = cu_seqlens ? cu_seqlens[s] : s * T;
            int64_t len = cu_seqlens ? cu_seqlens[s + 1] - cu_seqlens[s] : T;
            const double *s0 = initial_state ? initial_state + (s * H + h) * K * V : NULL;
            const double *dsT = d_final_state ? d_final_state + (s * H + h) * K * V : NULL;
            double *ds0 = d_initial_state ? d_initial_state + (s * H + h) * K * V : NULL;
            bwd_pair(q, k, v, alpha, beta, s0, d_out, dsT, t0, len, h, H, K, V, scale, dq, dk, dv,
                     dalpha, dbeta, ds0, work);
        }
        free(work);
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
