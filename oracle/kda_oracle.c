/*
 * KDA CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 implementation of what the Kimi Delta Attention (KDA)
 * forward pass computes, used to check the HIP library.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path never does.  It shares no code, header or constant with the
 * HIP library: it has its own header (kda_oracle.h) and is compiled by gcc.
 *
 * Every function restates the pages it follows; nothing here is blocked,
 * fused or reordered beyond what those pages state.
 *
 * Pages cited:
 *   [recurrent.py]  "K3/kda/ops/reference/recurrent.py", naive_kda_fwd
 *                   (GQA expansion, scale default, initial state, time loop).
 *   [sec-01.tex]    "K3/notes/sections/sec-01.tex", section "KDA 递归核心",
 *                   subsection "逐步公式": the four-step update.
 *   [kda.rs]        "metrale_model_weights/kimi_k3_host/kda.rs": conv_update,
 *                   softplus, bounded_gate, l2norm_rows, kda_recurrent_step,
 *                   kda_decode_token.
 */
#include "kda_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the OpenMP loops below run with (1 without OpenMP). */
int kda_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One token of the recurrence for one (batch, value-head) chain, in place on
 * S[K][V] (V contiguous).  [sec-01.tex] steps 1-4, identical to the body of the
 * time loop in [recurrent.py] naive_kda_fwd:
 *   1. S_dec = exp(g) (.) S          (decay broadcast over V, per K channel)
 *   2. p = k^T S_dec,  r = v - p     (read the old prediction, residual)
 *   3. S = S_dec + (beta k) (x) r    (rank-1 write)
 *   4. o = (scale q)^T S             (readout after the write)
 * q_scaled already carries the readout scale.  r is caller scratch of size V. */
static void token_step(double *S, const double *q_scaled, const double *k,
                       const double *v, const double *g, double beta,
                       double *o, double *r, long K, long V)
{
    long i, j;
    /* step 1: decay */
    for (i = 0; i < K; ++i) {
        double d = exp(g[i]);
        for (j = 0; j < V; ++j) S[i * V + j] *= d;
    }
    /* step 2: residual r = v - k^T S_dec */
    for (j = 0; j < V; ++j) r[j] = 0.0;
    for (i = 0; i < K; ++i)
        for (j = 0; j < V; ++j) r[j] += k[i] * S[i * V + j];
    for (j = 0; j < V; ++j) r[j] = v[j] - r[j];
    /* step 3: rank-1 write with a = beta k */
    for (i = 0; i < K; ++i) {
        double a = beta * k[i];
        for (j = 0; j < V; ++j) S[i * V + j] += a * r[j];
    }
    /* step 4: readout o = q_scaled^T S */
    for (j = 0; j < V; ++j) o[j] = 0.0;
    for (i = 0; i < K; ++i)
        for (j = 0; j < V; ++j) o[j] += q_scaled[i] * S[i * V + j];
}

int kda_oracle_fwd(const double *q, const double *k, const double *v,
                   const double *g, const double *beta, const double *S0,
                   double *o, double *S_out, long B, long T, long H, long HV,
                   long K, long V, double scale)
{
    return kda_oracle_fwd_snapshots(q, k, v, g, beta, S0, o, S_out, NULL, 0,
                                    B, T, H, HV, K, V, scale);
}

/* The time loop of [recurrent.py] naive_kda_fwd, which can also keep copies of
 * the state along the way: the prefix-cache test of [kda.rs]
 * (prefix_hit_wrong_slot_diverges) clones the whole state after each token and
 * resumes decoding from such a clone.  Here snapshot j, for j < T / every, is
 * the state after the first (j + 1) * every tokens, written to
 * snaps[b][j][hv] ([B, T / every, HV, K, V]).  snaps == NULL keeps none. */
int kda_oracle_fwd_snapshots(const double *q, const double *k, const double *v,
                             const double *g, const double *beta, const double *S0,
                             double *o, double *S_out, double *snaps, long every,
                             long B, long T, long H, long HV, long K, long V,
                             double scale)
{
    long bh;
    int status = 0;
    if (B < 0 || T < 0 || H <= 0 || HV <= 0 || K <= 0 || V <= 0) return 1;
    if (HV % H != 0) return 1;
    if (snaps && every <= 0) return 1;
    /* [recurrent.py]: scale=None means 1/sqrt(K). */
    if (!(scale > 0.0)) scale = 1.0 / sqrt((double)K);

#pragma omp parallel for schedule(dynamic, 1) reduction(| : status)
    for (bh = 0; bh < B * HV; ++bh) {
        const long b = bh / HV, hv = bh % HV;
        /* [recurrent.py] GQA: q/k are repeat_interleave'd from H to HV heads,
         * so value head hv reads q/k head hv / (HV/H). */
        const long h = hv / (HV / H);
        double *S = (double *)calloc((size_t)(K * V), sizeof(double));
        double *qs = (double *)malloc((size_t)K * sizeof(double));
        double *r = (double *)malloc((size_t)V * sizeof(double));
        long t, i;
        if (!S || !qs || !r) {
            status |= 2;
        } else {
            /* [recurrent.py]: S = zeros + initial_state. */
            if (S0) memcpy(S, S0 + bh * K * V, (size_t)(K * V) * sizeof(double));
            for (t = 0; t < T; ++t) {
                const long tok = b * T + t;
                const double *qt = q + (tok * H + h) * K;
                const double *kt = k + (tok * H + h) * K;
                const double *vt = v + (tok * HV + hv) * V;
                const double *gt = g + (tok * HV + hv) * K;
                const double bt = beta[tok * HV + hv];
                for (i = 0; i < K; ++i) qs[i] = scale * qt[i];
                token_step(S, qs, kt, vt, gt, bt, o + (tok * HV + hv) * V, r, K, V);
                if (snaps && (t + 1) % every == 0) {
                    const long j = (t + 1) / every - 1, ns = T / every;
                    memcpy(snaps + ((b * ns + j) * HV + hv) * K * V, S,
                           (size_t)(K * V) * sizeof(double));
                }
            }
            if (S_out) memcpy(S_out + bh * K * V, S, (size_t)(K * V) * sizeof(double));
        }
        free(S);
        free(qs);
        free(r);
    }
    return status;
}

/* Gradients of the forward pass: back-propagation through time over the time
 * loop of [recurrent.py], the backward its docstring derives (KDAFunction in
 * [recurrent.py]), with the gradient of the initial state kept (the page's
 * backward drops it).  For a loss L with dL/do = dout ([B,T,HV,V]) and
 * dL/dS_T = dS_T ([B,HV,K,V], NULL = 0):
 *   forward, per (b, hv) chain: S_dec_t = exp(g_t) (.) S_{t-1},
 *     r_t = v_t - k_t^T S_dec_t,  a_t = beta_t k_t,  S_t = S_dec_t + a_t (x) r_t,
 *     o_t = qs_t^T S_t with qs_t = scale q_t;
 *   backward, t = T-1 .. 0, with D (= dL/dS_t, starting at dS_T):
 *     D += qs_t (x) dout_t             (the readout)
 *     dqs_t = S_t dout_t               (dq_t = scale dqs_t)
 *     da_t = D r_t,  dr_t = a_t^T D    (the rank-1 write)
 *     dbeta_t = k_t . da_t,  dk_t = beta_t da_t - S_dec_t dr_t,  dv_t = dr_t
 *     D_dec = D - k_t (x) dr_t         (r_t = v_t - k_t^T S_dec_t)
 *     dg_t = sum over V of S_dec_t (.) D_dec
 *     D = exp(g_t) (.) D_dec           (the decay)
 *   dS0 = D after t = 0.
 * GQA: q/k head h serves value heads h*G .. h*G+G-1 (G = HV/H), so dq and dk
 * of head h sum over them (the repeat_interleave of [recurrent.py] reversed).
 * Every array is row-major as in kda_oracle_fwd; dS_out may be NULL.  The
 * forward states of a chain are kept (T*K*V doubles per chain at a time). */
int kda_oracle_bwd(const double *q, const double *k, const double *v,
                   const double *g, const double *beta, const double *S0,
                   const double *dout, const double *dST,
                   double *dq, double *dk, double *dv, double *dg, double *dbeta,
                   double *dS_out, long B, long T, long H, long HV, long K, long V,
                   double scale)
{
    long bh;
    int status = 0;
    const long G = (H > 0 && HV % H == 0) ? HV / H : 0;
    if (B < 0 || T < 0 || H <= 0 || HV <= 0 || K <= 0 || V <= 0 || G == 0) return 1;
    if (!(scale > 0.0)) scale = 1.0 / sqrt((double)K);
    memset(dq, 0, (size_t)(B * T * H * K) * sizeof(double));
    memset(dk, 0, (size_t)(B * T * H * K) * sizeof(double));

    /* one q/k head (and its G value heads, one after another) per iteration,
     * so that the GQA sums into dq and dk need no synchronisation */
#pragma omp parallel for schedule(dynamic, 1) reduction(| : status)
    for (bh = 0; bh < B * H; ++bh) {
        const long b = bh / H, h = bh % H;
        const long KV = K * V;
        double *Sdec = (double *)malloc((size_t)(T > 0 ? T : 1) * KV * sizeof(double));
        double *R = (double *)malloc((size_t)(T > 0 ? T : 1) * V * sizeof(double));
        double *S = (double *)malloc((size_t)KV * sizeof(double));
        double *D = (double *)malloc((size_t)KV * sizeof(double));
        double *da = (double *)malloc((size_t)K * sizeof(double));
        double *dr = (double *)malloc((size_t)V * sizeof(double));
        long j, t, i, c;
        if (!Sdec || !R || !S || !D || !da || !dr) {
            status |= 2;
        } else {
            for (j = 0; j < G; ++j) {
                const long hv = h * G + j, chain = b * HV + hv;
                /* forward, keeping S_dec_t and r_t */
                if (S0) memcpy(S, S0 + chain * KV, (size_t)KV * sizeof(double));
                else memset(S, 0, (size_t)KV * sizeof(double));
                for (t = 0; t < T; ++t) {
                    const long tok = b * T + t;
                    const double *kt = k + (tok * H + h) * K;
                    const double *vt = v + (tok * HV + hv) * V;
                    const double *gt = g + (tok * HV + hv) * K;
                    const double bt = beta[tok * HV + hv];
                    double *Sd = Sdec + t * KV, *rt = R + t * V;
                    for (i = 0; i < K; ++i) {
                        const double d = exp(gt[i]);
                        for (c = 0; c < V; ++c) Sd[i * V + c] = d * S[i * V + c];
                    }
                    for (c = 0; c < V; ++c) {
                        double p = 0.0;
                        for (i = 0; i < K; ++i) p += kt[i] * Sd[i * V + c];
                        rt[c] = vt[c] - p;
                    }
                    for (i = 0; i < K; ++i)
                        for (c = 0; c < V; ++c) S[i * V + c] = Sd[i * V + c] + bt * kt[i] * rt[c];
                }
                /* backward */
                if (dST) memcpy(D, dST + chain * KV, (size_t)KV * sizeof(double));
                else memset(D, 0, (size_t)KV * sizeof(double));
                for (t = T - 1; t >= 0; --t) {
                    const long tok = b * T + t;
                    const double *qt = q + (tok * H + h) * K;
                    const double *kt = k + (tok * H + h) * K;
                    const double *gt = g + (tok * HV + hv) * K;
                    const double *dot = dout + (tok * HV + hv) * V;
                    const double bt = beta[tok * HV + hv];
                    const double *Sd = Sdec + t * KV, *rt = R + t * V;
                    double *dqt = dq + (tok * H + h) * K, *dkt = dk + (tok * H + h) * K;
                    double db = 0.0;
                    /* the readout: D += qs (x) dout, dqs = S_t dout */
                    for (i = 0; i < K; ++i) {
                        const double qs = scale * qt[i];
                        double acc = 0.0;
                        for (c = 0; c < V; ++c) {
                            const double St = Sd[i * V + c] + bt * kt[i] * rt[c];
                            D[i * V + c] += qs * dot[c];
                            acc += St * dot[c];
                        }
                        dqt[i] += scale * acc;
                    }
                    /* the write S_t = S_dec + a (x) r: da = D r, dr = a^T D */
                    for (i = 0; i < K; ++i) {
                        double acc = 0.0;
                        for (c = 0; c < V; ++c) acc += D[i * V + c] * rt[c];
                        da[i] = acc;
                        db += kt[i] * acc;
                    }
                    for (c = 0; c < V; ++c) {
                        double acc = 0.0;
                        for (i = 0; i < K; ++i) acc += bt * kt[i] * D[i * V + c];
                        dr[c] = acc;
                        dv[(tok * HV + hv) * V + c] = acc;
                    }
                    dbeta[tok * HV + hv] = db;
                    /* the residual r = v - k^T S_dec, then the decay */
                    for (i = 0; i < K; ++i) {
                        const double e = exp(gt[i]);
                        double acc_k = 0.0, acc_g = 0.0;
                        for (c = 0; c < V; ++c) {
                            const double Dd = D[i * V + c] - kt[i] * dr[c];
                            acc_k += Sd[i * V + c] * dr[c];
                            acc_g += Sd[i * V + c] * Dd;
                            D[i * V + c] = e * Dd;
                        }
                        dkt[i] += bt * da[i] - acc_k;
                        dg[(tok * HV + hv) * K + i] = acc_g;
                    }
                }
                if (dS_out) memcpy(dS_out + chain * KV, D, (size_t)KV * sizeof(double));
            }
        }
        free(Sdec);
        free(R);
        free(S);
        free(D);
        free(da);
        free(dr);
    }
    return status;
}

/* [kda.rs] sigmoid and softplus (softplus written in its overflow-safe form
 * max(x,0) + log1p(exp(-|x|)), as on the page). */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }
static double softplus(double x) { return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))); }

double kda_oracle_sigmoid(double x) { return sigmoid(x); }
double kda_oracle_softplus(double x) { return softplus(x); }

/* [kda.rs] bounded_gate, for one channel: with d = exp(A_log[head]) and
 * x = z + dt_bias[channel], the gate is lb * sigmoid(d * x) when a lower bound
 * lb is given, and -d * softplus(x) when it is not.  The only statement of the
 * gate in this file: the gate entry point, the decode step and the prefill
 * prologue all call it. */
static double gate_value(double z, double dt_bias, double A_log_head, int bounded,
                         double lower_bound)
{
    const double d = exp(A_log_head);
    const double x = z + dt_bias;
    if (bounded) return lower_bound * sigmoid(d * x);
    return -(d * softplus(x));
}

/* [kda.rs] conv_update, for one row of channels, from its definition: channel
 * c keeps a register of its last KW inputs (oldest first).  The window of this
 * step is the register's newest KW - 1 values followed by the new input; the
 * output is the SiLU of the window's dot product with the channel's KW weights
 * (weight j on window position j), and the window becomes the register. */
static void conv_update(double *state, const double *x, const double *w,
                        double *y, long channels, long KW)
{
    double *win = (double *)malloc((size_t)KW * sizeof(double));
    long c, j;
    if (!win) abort();
    for (c = 0; c < channels; ++c) {
        double *reg = state + c * KW; /* KW slots; slot 0 is the oldest */
        double pre = 0.0;
        /* the window: the register's newest KW - 1 values, then x[c] */
        for (j = 0; j < KW - 1; ++j) win[j] = reg[j + 1];
        win[KW - 1] = x[c];
        for (j = 0; j < KW; ++j) pre += w[c * KW + j] * win[j];
        y[c] = pre / (1.0 + exp(-pre)); /* SiLU(pre) = pre * sigmoid(pre) */
        memcpy(reg, win, (size_t)KW * sizeof(double));
    }
    free(win);
}

/* [kda.rs] l2norm_rows: each row divided by its norm sqrt(sum x^2 + eps), the
 * eps inside the root. */
static void l2norm_row(double *x, long d, double eps)
{
    long i;
    double ss = 0.0, norm;
    for (i = 0; i < d; ++i) ss += x[i] * x[i];
    norm = sqrt(ss + eps);
    for (i = 0; i < d; ++i) x[i] = x[i] / norm;
}

int kda_oracle_decode_step(const double *x, const double *conv_w, double *conv_state,
                           long KW, int l2norm_qk, double eps,
                           const double *gate_in, const double *A_log,
                           const double *dt_bias, int gate_bounded, double lower_bound,
                           const double *beta_in, int beta_is_logit, double *state,
                           double *out, long B, long H, long HV, long K, long V,
                           double scale)
{
    const long Cch = 2 * H * K + HV * V; /* channels: q (H*K) | k (H*K) | v (HV*V) */
    long b;
    int status = 0;
    if (B < 0 || H <= 0 || HV <= 0 || K <= 0 || V <= 0 || HV % H != 0) return 1;
    if (conv_w && (KW < 1 || !conv_state)) return 1;
    if (A_log && !dt_bias) return 1;
    if (!(scale > 0.0)) scale = 1.0 / sqrt((double)K);

#pragma omp parallel for schedule(dynamic, 1) reduction(| : status)
    for (b = 0; b < B; ++b) {
        double *y = (double *)malloc((size_t)Cch * sizeof(double));
        double *qs = (double *)malloc((size_t)K * sizeof(double));
        double *g = (double *)malloc((size_t)K * sizeof(double));
        double *r = (double *)malloc((size_t)V * sizeof(double));
        long hv, i;
        if (!y || !qs || !g || !r) {
            status |= 2;
            goto done;
        }
        /* [kda.rs] kda_decode_token: the short conv runs first on all channels. */
        if (conv_w)
            conv_update(conv_state + b * Cch * KW, x + b * Cch, conv_w, y, Cch, KW);
        else
            memcpy(y, x + b * Cch, (size_t)Cch * sizeof(double));
        /* [kda.rs] kda_recurrent_step: q and k rows are L2-normalised per head. */
        if (l2norm_qk)
            for (i = 0; i < 2 * H; ++i) l2norm_row(y + i * K, K, eps);
        for (hv = 0; hv < HV; ++hv) {
            const long h = hv / (HV / H);
            const double *qh = y + h * K;
            const double *kh = y + H * K + h * K;
            const double *vh = y + 2 * H * K + hv * V;
            double bt = beta_in[b * HV + hv];
            /* [kda.rs] kda_recurrent_step: beta arrives as a logit -> sigmoid. */
            if (beta_is_logit) bt = sigmoid(bt);
            for (i = 0; i < K; ++i) {
                const double gi = gate_in[(b * HV + hv) * K + i];
                if (A_log) {
                    g[i] = gate_value(gi, dt_bias[hv * K + i], A_log[hv], gate_bounded,
                                      lower_bound);
                } else {
                    g[i] = gi;
                }
                qs[i] = scale * qh[i];
            }
            token_step(state + (b * HV + hv) * K * V, qs, kh, vh, g, bt,
                       out + (b * HV + hv) * V, r, K, V);
        }
    done:
        free(y);
        free(qs);
        free(g);
        free(r);
    }
    return status;
}

int kda_oracle_gate(const double *z, const double *A_log, const double *dt_bias,
                    int gate_bounded, double lower_bound, double *g, long rows,
                    long HV, long K)
{
    long r, hv, i;
    for (r = 0; r < rows; ++r)
        for (hv = 0; hv < HV; ++hv)
            for (i = 0; i < K; ++i) {
                const long idx = (r * HV + hv) * K + i;
                g[idx] = gate_value(z[idx], dt_bias[hv * K + i], A_log[hv], gate_bounded,
                                    lower_bound);
            }
    return 0;
}

int kda_oracle_conv_update(double *state, const double *x, const double *w, double *y,
                           long rows, long channels, long KW)
{
    long r;
    if (KW < 1) return 1;
    for (r = 0; r < rows; ++r)
        conv_update(state + r * channels * KW, x + r * channels, w, y + r * channels,
                    channels, KW);
    return 0;
}

int kda_oracle_l2norm_rows(double *x, long rows, long d, double eps)
{
    long r;
    for (r = 0; r < rows; ++r) l2norm_row(x + r * d, d, eps);
    return 0;
}

/* The stages [kda.rs] kda_decode_token runs in front of the recurrence
 * (conv_update on the packed q | k | v channels, then in kda_recurrent_step
 * l2norm_rows on q and k, the gate from bounded_gate, a sigmoid on beta),
 * applied to the T tokens of each sequence in order: the per-token inputs of a
 * whole prefill.  The conv register of each channel is carried from token to
 * token and left in conv_state, as T decode steps would leave it.
 *   x [B,T,C] (C = 2HK + HV V), conv_state [B,C,KW] (in/out; unused without
 *   conv_w), gate_in [B,T,HV,K] (g itself when A_log == NULL, else z),
 *   beta_in [B,T,HV];  outputs q, k [B,T,H,K], v [B,T,HV,V], g [B,T,HV,K],
 *   beta_out [B,T,HV]. */
int kda_oracle_prefill_prologue(const double *x, const double *conv_w, double *conv_state,
                                long KW, int l2norm_qk, double eps,
                                const double *gate_in, const double *A_log,
                                const double *dt_bias, int gate_bounded, double lower_bound,
                                const double *beta_in, int beta_is_logit,
                                double *q, double *k, double *v, double *g, double *beta_out,
                                long B, long T, long H, long HV, long K, long V)
{
    const long Cch = 2 * H * K + HV * V;
    long b;
    int status = 0;
    if (B < 0 || T < 0 || H <= 0 || HV <= 0 || K <= 0 || V <= 0 || HV % H != 0) return 1;
    if (conv_w && (KW < 1 || !conv_state)) return 1;
    if (A_log && !dt_bias) return 1;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : status)
    for (b = 0; b < B; ++b) {
        double *y = (double *)malloc((size_t)Cch * sizeof(double));
        long t, i, hv;
        if (!y) {
            status |= 2;
            continue;
        }
        for (t = 0; t < T; ++t) {
            const long bt = b * T + t;
            if (conv_w)
                conv_update(conv_state + b * Cch * KW, x + bt * Cch, conv_w, y, Cch, KW);
            else
                memcpy(y, x + bt * Cch, (size_t)Cch * sizeof(double));
            if (l2norm_qk)
                for (i = 0; i < 2 * H; ++i) l2norm_row(y + i * K, K, eps);
            memcpy(q + bt * H * K, y, (size_t)(H * K) * sizeof(double));
            memcpy(k + bt * H * K, y + H * K, (size_t)(H * K) * sizeof(double));
            memcpy(v + bt * HV * V, y + 2 * H * K, (size_t)(HV * V) * sizeof(double));
            for (hv = 0; hv < HV; ++hv) {
                const double bl = beta_in[bt * HV + hv];
                beta_out[bt * HV + hv] = beta_is_logit ? sigmoid(bl) : bl;
                for (i = 0; i < K; ++i) {
                    const long idx = (bt * HV + hv) * K + i;
                    if (A_log) {
                        g[idx] = gate_value(gate_in[idx], dt_bias[hv * K + i], A_log[hv],
                                            gate_bounded, lower_bound);
                    } else {
                        g[idx] = gate_in[idx];
                    }
                }
            }
        }
        free(y);
    }
    return status;
}

/* [kda.rs] full_rank_output_gate: for each row of d values,
 * y = sigmoid(gate) * o / sqrt(mean(o^2) + eps)  (an RMS norm of o without a
 * learned scale, gated elementwise). */
int kda_oracle_output_gate(const double *o, const double *gate, double *y, long rows,
                           long d, double eps)
{
    long r, i;
    if (rows < 0 || d <= 0) return 1;
    for (r = 0; r < rows; ++r) {
        const double *orow = o + r * d, *grow = gate + r * d;
        double ms = 0.0, inv;
        for (i = 0; i < d; ++i) ms += orow[i] * orow[i];
        ms /= (double)d;
        inv = 1.0 / sqrt(ms + eps);
        for (i = 0; i < d; ++i) y[r * d + i] = sigmoid(grow[i]) * orow[i] * inv;
    }
    return 0;
}
