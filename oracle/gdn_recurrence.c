/*
 * ORACLE — test infrastructure only.
 *
 * Plain, slow, fp64 token-by-token Gated DeltaNet recurrence.  Only tests/,
 * the smoke check and the bench's CPU-baseline leg may load this library; the
 * product path never calls it.  It shares no code with the HIP library.
 *
 * What it computes (row-vector convention: q_t, k_t in R^{1 x d_k},
 * v_t in R^{1 x d_v}, S in R^{d_k x d_v}, stored d_v-contiguous), following
 * "实验三：GDN Prefill 前向优化", section "GLA, DeltaNet 与 Gated DeltaNet"
 * (the Gated DeltaNet update):
 *
 *     Sbar_t = alpha_t * S_{t-1}                    (gated forgetting)
 *     S_t    = Sbar_t + beta_t * k_t^T (v_t - k_t Sbar_t)   (delta rule)
 *     o_t    = scale * q_t S_t                      (read after the update)
 *
 * with alpha_t = exp(g_t) (the gate arrives in log space, same page, section
 * "输入输出定义", raw_g = log alpha), the value head h using query/key head
 * floor(h / G), G = H_v / H_q (same section, GVA paragraph), and scale the
 * 1/sqrt(d_k) factor the chunk output formula on that page carries
 * (section "计算过程描述").  Each sequence of a packed batch starts from its
 * own initial state (or zeros) and returns its own final state.
 *
 * The same per-token update, applied once to a batch of states, is the decode
 * step ("Qwen3.5-397B-A17B" trace page, Decode-GDN node 7,
 * gdn_packed_recurrent_qk_norm_gating_state_update: decay, predict, delta
 * write, read) without that node's gating / normalisation front end.
 *
 * Build: gcc -O3 -fopenmp -fPIC -shared (see oracle/build.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of the recurrence on one (sequence, value-head) state; q and k in fp64. */
static void gdn_token_update_d(double *S, const double *q, const double *k, const float *v, double g, double beta,
                               int64_t dk, int64_t dv, double scale, double *out /* may be NULL */, double *p,
                               double *delta) {
    const double alpha = exp(g);
    /* Sbar = alpha * S */
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= alpha;
    /* prediction p = k Sbar  (p_j = sum_i k_i Sbar_ij) */
    for (int64_t j = 0; j < dv; ++j) p[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i) {
        const double ki = k[i];
        for (int64_t j = 0; j < dv; ++j) p[j] += ki * S[i * dv + j];
    }
    /* delta = beta (v - p) */
    for (int64_t j = 0; j < dv; ++j) delta[j] = beta * ((double)v[j] - p[j]);
    /* S = Sbar + k^T delta */
    for (int64_t i = 0; i < dk; ++i) {
        const double ki = k[i];
        for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += ki * delta[j];
    }
    /* o = scale * q S */
    if (out) {
        for (int64_t j = 0; j < dv; ++j) p[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i) {
            const double qi = q[i];
            for (int64_t j = 0; j < dv; ++j) p[j] += qi * S[i * dv + j];
        }
        for (int64_t j = 0; j < dv; ++j) out[j] = scale * p[j];
    }
}

/* The same with the q, k values the device receives (upcast exactly). */
static void gdn_token_update(double *S, const float *q, const float *k, const float *v, double g, double beta,
                             int64_t dk, int64_t dv, double scale, double *out, double *p, double *delta) {
    double qd[1024], kd[1024];
    for (int64_t i = 0; i < dk; ++i) {
        qd[i] = (double)q[i];
        kd[i] = (double)k[i];
    }
    gdn_token_update_d(S, qd, kd, v, g, beta, dk, dv, scale, out, p, delta);
}

/*
 * Packed variable-length forward.
 *   q, k:  [T, H_q, d_k] float (exact values the device receives)
 *   v:     [T, H_v, d_v] float
 *   g:     [T, H_v] float, log decay per token (NOT cumulative)
 *   beta:  [T, H_v] float
 *   cu_seqlens: [num_seqs + 1] int64, 0 = cu[0] <= ... <= cu[N] = T
 *   initial_state: [N, H_v, d_k, d_v] double, or NULL for zeros
 *   out:   [T, H_v, d_v] double (rows of heads not selected are untouched)
 *   final_state: [N, H_v, d_k, d_v] double, or NULL
 *   heads: list of value heads to compute (n_heads entries), or NULL for all
 *   delta_out: optional [T, H_v, d_v] double receiving beta (v - k Sbar) per token
 * Returns 0, or -1 on bad arguments.
 */
int gdn_oracle_forward(const float *q, const float *k, const float *v, const float *g, const float *beta,
                       const int64_t *cu_seqlens, int64_t num_seqs, int64_t H_q, int64_t H_v, int64_t dk,
                       int64_t dv, double scale, const double *initial_state, double *out, double *final_state,
                       const int32_t *heads, int64_t n_heads, double *delta_out, int num_threads) {
    if (num_seqs < 0 || H_q <= 0 || H_v <= 0 || dk <= 0 || dv <= 0 || H_v % H_q != 0 || dk > 1024) return -1;
    if (!heads) n_heads = H_v;
    const int64_t G = H_v / H_q;
    const int64_t npairs = num_seqs * n_heads;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t pi = 0; pi < npairs; ++pi) {
        const int64_t n = pi / n_heads;
        const int64_t h = heads ? (int64_t)heads[pi % n_heads] : (pi % n_heads);
        if (h < 0 || h >= H_v) {
            bad |= 1;
            continue;
        }
        const int64_t hq = h / G;
        double *S = (double *)malloc(sizeof(double) * (size_t)(dk * dv));
        double *p = (double *)malloc(sizeof(double) * (size_t)dv);
        double *delta = (double *)malloc(sizeof(double) * (size_t)dv);
        if (initial_state)
            memcpy(S, initial_state + (n * H_v + h) * dk * dv, sizeof(double) * (size_t)(dk * dv));
        else
            memset(S, 0, sizeof(double) * (size_t)(dk * dv));
        for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
            gdn_token_update(S, q + (t * H_q + hq) * dk, k + (t * H_q + hq) * dk, v + (t * H_v + h) * dv,
                             (double)g[t * H_v + h], (double)beta[t * H_v + h], dk, dv, scale,
                             out ? out + (t * H_v + h) * dv : NULL, p, delta);
            if (delta_out) memcpy(delta_out + (t * H_v + h) * dv, delta, sizeof(double) * (size_t)dv);
        }
        if (final_state) memcpy(final_state + (n * H_v + h) * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
        free(S);
        free(p);
        free(delta);
    }
    return bad ? -1 : 0;
}

/*
 * One decode step for N independent sequences, state updated in place.
 *   q, k: [N, H_q, d_k]; v: [N, H_v, d_v]; g, beta: [N, H_v]
 *   state: [N, H_v, d_k, d_v] double, in/out; out: [N, H_v, d_v] double
 *   heads / n_heads: optional subset of value heads (NULL = all)
 */
int gdn_oracle_decode_step(const float *q, const float *k, const float *v, const float *g, const float *beta,
                           int64_t N, int64_t H_q, int64_t H_v, int64_t dk, int64_t dv, double scale,
                           double *state, double *out, const int32_t *heads, int64_t n_heads, int num_threads) {
    if (N < 0 || H_q <= 0 || H_v <= 0 || dk <= 0 || dv <= 0 || H_v % H_q != 0 || dk > 1024) return -1;
    if (!heads) n_heads = H_v;
    const int64_t G = H_v / H_q;
    const int64_t npairs = N * n_heads;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t pi = 0; pi < npairs; ++pi) {
        const int64_t n = pi / n_heads;
        const int64_t h = heads ? (int64_t)heads[pi % n_heads] : (pi % n_heads);
        if (h < 0 || h >= H_v) {
            bad |= 1;
            continue;
        }
        const int64_t hq = h / G;
        double p[1024], delta[1024];
        if (dv > 1024) {
            bad |= 1;
            continue;
        }
        gdn_token_update(state + (n * H_v + h) * dk * dv, q + (n * H_q + hq) * dk, k + (n * H_q + hq) * dk,
                         v + (n * H_v + h) * dv, (double)g[n * H_v + h], (double)beta[n * H_v + h], dk, dv, scale,
                         out + (n * H_v + h) * dv, p, delta);
    }
    return bad ? -1 : 0;
}

/*
 * Decode step with the front end of the same node (trace page, Decode-GDN
 * node 7, its first two steps), in fp64:
 *   k_bar = k / sqrt(sum_j k_j^2 + 1e-6),  q_bar = scale * q / sqrt(sum_j q_j^2 + 1e-6)
 *     (an L2 norm over the sum of squares, not an RMS norm; the query scale
 *     multiplies once, after the norm)
 *   g = -exp(A_log[h]) * softplus(a + dt_bias[h]),  alpha = exp(g),
 *     softplus(x) = ln(1 + e^x) (the gate of the trace page's node 7; the
 *     "Kestrel_VLLM - 24" page, section 三, guards its exponential against
 *     overflow with branches at +-20, which change the value by less than
 *     fp32 rounding; here the overflow-free form max(x, 0) + ln(1 + e^-|x|)
 *     gives the exact value)
 *   beta = sigmoid(b), rounded to bf16 and back when beta_round_bf16 (the
 *     trace page keeps that rounding when b is bf16); sigmoid is taken in fp64
 *     and rounded to fp32 first, the precision the pages' kernels work in
 * then the update of gdn_token_update with q_bar (scale already applied), k_bar.
 *   a, b: [N, H_v] (exact values the device receives); A_log, dt_bias: [H_v]
 *   g_out, beta_out: [N, H_v] double or NULL (the gate and beta used)
 */
static double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

/* fp32 -> bf16 (round to nearest even) -> fp32; inputs here are finite. */
static float round_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    u &= 0xFFFF0000u;
    memcpy(&x, &u, 4);
    return x;
}

int gdn_oracle_decode_step_fused(const float *q, const float *k, const float *v, const float *a, const float *b,
                                 const float *A_log, const float *dt_bias, int beta_round_bf16, int64_t N,
                                 int64_t H_q, int64_t H_v, int64_t dk, int64_t dv, double scale, double *state,
                                 double *out, double *g_out, double *beta_out, const int32_t *heads, int64_t n_heads,
                                 int num_threads) {
    if (N < 0 || H_q <= 0 || H_v <= 0 || dk <= 0 || dv <= 0 || H_v % H_q != 0 || dk > 1024 || dv > 1024) return -1;
    if (!heads) n_heads = H_v;
    const int64_t G = H_v / H_q;
    const int64_t npairs = N * n_heads;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t pi = 0; pi < npairs; ++pi) {
        const int64_t n = pi / n_heads;
        const int64_t h = heads ? (int64_t)heads[pi % n_heads] : (pi % n_heads);
        if (h < 0 || h >= H_v) {
            bad |= 1;
            continue;
        }
        const int64_t hq = h / G;
        const float *qr = q + (n * H_q + hq) * dk, *kr = k + (n * H_q + hq) * dk;
        double qn[1024], kn[1024], p[1024], delta[1024];
        double sq = 0.0, sk = 0.0;
        for (int64_t i = 0; i < dk; ++i) {
            sq += (double)qr[i] * (double)qr[i];
            sk += (double)kr[i] * (double)kr[i];
        }
        const double rq = scale / sqrt(sq + 1e-6), rk = 1.0 / sqrt(sk + 1e-6);
        for (int64_t i = 0; i < dk; ++i) {
            qn[i] = (double)qr[i] * rq;
            kn[i] = (double)kr[i] * rk;
        }
        const double g = -exp((double)A_log[h]) * softplus((double)a[n * H_v + h] + (double)dt_bias[h]);
        float sig = (float)(1.0 / (1.0 + exp(-(double)b[n * H_v + h])));
        if (beta_round_bf16) sig = round_bf16(sig);
        const double beta = (double)sig;
        if (g_out) g_out[n * H_v + h] = g;
        if (beta_out) beta_out[n * H_v + h] = beta;
        gdn_token_update_d(state + (n * H_v + h) * dk * dv, qn, kn, v + (n * H_v + h) * dv, g, beta, dk, dv, 1.0,
                           out + (n * H_v + h) * dv, p, delta);
    }
    return bad ? -1 : 0;
}

int gdn_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
