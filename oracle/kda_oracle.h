/*
 * KDA CPU oracle (fp64) -- TEST INFRASTRUCTURE ONLY; see kda_oracle.c.
 *
 * Layouts are row-major and contiguous, as in the time loop of
 * "K3/kda/ops/reference/recurrent.py" (naive_kda_fwd):
 *   q, k  [B, T, H, K]     v [B, T, HV, V]     g [B, T, HV, K]   beta [B, T, HV]
 *   S0, S_out [B, HV, K, V]                    o [B, T, HV, V]
 * HV must be a multiple of H; value head hv reads q/k head hv / (HV / H).
 * scale <= 0 selects 1/sqrt(K).  S0 == NULL means a zero initial state;
 * S_out == NULL skips writing the final state.
 * Return: 0 on success, 1 on bad sizes, 2 on host allocation failure.
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Threads the oracle's OpenMP loops use. */
int kda_oracle_threads(void);

int kda_oracle_fwd(const double *q, const double *k, const double *v,
                   const double *g, const double *beta, const double *S0,
                   double *o, double *S_out, long B, long T, long H, long HV,
                   long K, long V, double scale);

/* kda_oracle_fwd that also keeps snapshots of the state: snapshot j
 * (j < T / every) is the state after the first (j + 1) * every tokens, stored
 * at snaps[b][j][hv] ([B, T / every, HV, K, V]).  snaps == NULL keeps none;
 * otherwise every must be >= 1. */
int kda_oracle_fwd_snapshots(const double *q, const double *k, const double *v,
                             const double *g, const double *beta, const double *S0,
                             double *o, double *S_out, double *snaps, long every,
                             long B, long T, long H, long HV, long K, long V,
                             double scale);

/* Gradients of kda_oracle_fwd by back-propagation through time: from dL/do
 * (dout [B,T,HV,V]) and dL/dS_T (dST [B,HV,K,V], NULL = 0) to dq, dk
 * [B,T,H,K], dv [B,T,HV,V], dg [B,T,HV,K], dbeta [B,T,HV] and dS_out
 * [B,HV,K,V] (NULL = not written).  Keeps the T forward states of one chain
 * at a time. */
int kda_oracle_bwd(const double *q, const double *k, const double *v,
                   const double *g, const double *beta, const double *S0,
                   const double *dout, const double *dST,
                   double *dq, double *dk, double *dv, double *dg, double *dbeta,
                   double *dS_out, long B, long T, long H, long HV, long K, long V,
                   double scale);

/* One decode token for B sequences ("metrale_model_weights/kimi_k3_host/kda.rs",
 * kda_decode_token / kda_recurrent_step), with every prologue stage optional:
 *   x          [B, 2*H*K + HV*V]  packed q | k | v channels (before the conv)
 *   conv_w     [2*H*K + HV*V, KW] or NULL (no short conv: channels used as is)
 *   conv_state [B, 2*H*K + HV*V, KW], updated in place (ignored without conv_w)
 *   l2norm_qk  nonzero: q and k rows divided by sqrt(sum x^2 + eps)
 *   gate_in    [B, HV, K]: the log-decay g itself when A_log == NULL, else z
 *   A_log [HV], dt_bias [HV*K]: gate = lower_bound*sigmoid(exp(A_log)*(z+dt_bias))
 *              when gate_bounded, else -exp(A_log)*softplus(z+dt_bias)
 *   beta_in    [B, HV], a logit when beta_is_logit (beta = sigmoid(beta_in))
 *   state      [B, HV, K, V] updated in place;  out [B, HV, V]. */
int kda_oracle_decode_step(const double *x, const double *conv_w, double *conv_state,
                           long KW, int l2norm_qk, double eps,
                           const double *gate_in, const double *A_log,
                           const double *dt_bias, int gate_bounded, double lower_bound,
                           const double *beta_in, int beta_is_logit, double *state,
                           double *out, long B, long H, long HV, long K, long V,
                           double scale);

/* The decode prologue's stages applied to T tokens of each sequence in order
 * (a prefill's per-token inputs from the raw projections):
 *   x [B,T,2HK+HV*V]; conv_state [B,2HK+HV*V,KW] in/out; gate_in [B,T,HV,K];
 *   beta_in [B,T,HV];  q, k [B,T,H,K], v [B,T,HV,V], g [B,T,HV,K], beta_out [B,T,HV]
 * with the options of kda_oracle_decode_step. */
int kda_oracle_prefill_prologue(const double *x, const double *conv_w, double *conv_state,
                                long KW, int l2norm_qk, double eps,
                                const double *gate_in, const double *A_log,
                                const double *dt_bias, int gate_bounded, double lower_bound,
                                const double *beta_in, int beta_is_logit,
                                double *q, double *k, double *v, double *g, double *beta_out,
                                long B, long T, long H, long HV, long K, long V);

/* full_rank_output_gate ("metrale_model_weights/kimi_k3_host/kda.rs"):
 * y = sigmoid(gate) * o / sqrt(mean(o^2) + eps) per row of d values. */
int kda_oracle_output_gate(const double *o, const double *gate, double *y, long rows,
                           long d, double eps);

/* The decode prologue stages on their own, for pinning them separately. */
int kda_oracle_gate(const double *z, const double *A_log, const double *dt_bias,
                    int gate_bounded, double lower_bound, double *g, long rows,
                    long HV, long K);
int kda_oracle_conv_update(double *state, const double *x, const double *w, double *y,
                           long rows, long channels, long KW);
int kda_oracle_l2norm_rows(double *x, long rows, long d, double eps);
double kda_oracle_sigmoid(double x);
double kda_oracle_softplus(double x);

#ifdef __cplusplus
}
#endif

#endif
