/*
 * libkda -- Kimi Delta Attention (KDA) forward and backward on AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (page "K3/notes/sections/sec-01.tex", section "KDA 递归核心",
 * subsection "逐步公式"; the same loop is naive_kda_fwd on the page
 * "K3/kda/ops/reference/recurrent.py"), per batch b, value head hv and token t,
 * with S the [K x V] state of (b, hv) and h = hv / (HV / H) the q/k head that
 * hv reads (GQA repeat-interleave):
 *
 *     S_dec = exp(g_t) (.) S_{t-1}              decay, one factor per K row
 *     r_t   = v_t - k_t^T S_dec                 delta-rule residual
 *     S_t   = S_dec + (beta_t k_t) (x) r_t      rank-1 write
 *     o_t   = (scale q_t)^T S_t                 readout after the write
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees, or keeps them; the one entry point that needs
 *    scratch memory (kda_recurrent_bwd) takes it as a workspace argument.  Tensors are dense row-major with
 *    the last dimension contiguous, and every base address must be 16-byte
 *    aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *    work; they never synchronise.  Results are deterministic: the same inputs
 *    give bit-identical outputs on every run (no floating-point atomics).
 *  - Every argument is validated on the host before anything is enqueued; a
 *    rejected call has no side effects.  The library never aborts or throws.
 *  - Return codes: KDA_OK, KDA_EINVAL (bad pointer, size, alignment or
 *    aliasing), KDA_EUNSUPPORTED (valid but not built: head dim, chunk size,
 *    dtype, conv width), KDA_EHIP (the HIP runtime reported an error at
 *    launch).  kda_last_error() returns a message for the calling thread's most
 *    recent non-zero code.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

enum kda_status { KDA_OK = 0, KDA_EINVAL = 1, KDA_EUNSUPPORTED = 2, KDA_EHIP = 3 };

/* Element type of q, k, v (and qkv) and of the output o.  g, beta and the
 * recurrent state are always fp32. */
enum kda_dtype { KDA_DTYPE_F32 = 0, KDA_DTYPE_BF16 = 1 };

/* Gate modes of the decode prologue ("metrale_model_weights/kimi_k3_host/kda.rs",
 * bounded_gate).  DIRECT: the gate argument is g itself. */
enum kda_gate_mode { KDA_GATE_DIRECT = 0, KDA_GATE_BOUNDED = 1, KDA_GATE_SOFTPLUS = 2 };

int kda_abi_version(void);

/* Message for the calling thread's last non-zero status ("" if none). */
const char *kda_last_error(void);

/*
 * kda_chunk_fwd -- chunk-parallel prefill over T tokens.
 *
 * Computes o and the final state of the recurrence above for all b, t, hv,
 * starting from initial_state (zeros when NULL); the same interface as
 * naive_kda_fwd(q, k, v, g, beta, scale, initial_state, output_final_state) on
 * the "K3/kda/ops/reference/recurrent.py" page.  Internally it uses the chunk
 * form of the page "src/tinycenn_lm/research_layers.py" (delta_recurrence:
 * chunk-local cumulative decay, a unit-lower-triangular solve inside each
 * chunk, the state carried from chunk to chunk).
 *
 *   q, k          [B, T, H, K]   dtype
 *   v             [B, T, HV, V]  dtype
 *   g             [B, T, HV, K]  fp32, log-space decay; PRECONDITION -5 <= g <= 0
 *                                (the lower bound of the bounded gate).  Values
 *                                below -5 are not detected and can overflow the
 *                                in-chunk exponent factorisation; gates without
 *                                that bound go to kda_recurrent_fwd.
 *   beta          [B, T, HV]     fp32, write strength used as given
 *   initial_state [B, HV, K, V]  fp32 or NULL (zeros)
 *   out           [B, T, HV, V]  dtype; must not overlap any input
 *   final_state   [B, HV, K, V]  fp32 or NULL (not written); may be the same
 *                                pointer as initial_state (in-place resume), may
 *                                not otherwise overlap an input or out
 *   B, T >= 0 (either 0: nothing but the final state, which then equals the
 *   initial state, is written); H, HV >= 1 with HV % H == 0;
 *   K, V in {32, 64, 128};  scale <= 0 (or NaN) selects 1/sqrt(K);
 *   chunk 0 selects the default, 32 (the only size built);
 *   dtype KDA_DTYPE_F32 or KDA_DTYPE_BF16.
 */
int kda_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                  const float *beta, const float *initial_state, void *out,
                  float *final_state, int B, int T, int H, int HV, int K, int V,
                  float scale, int chunk, int dtype, void *stream);

/*
 * kda_recurrent_fwd -- the same computation and interface as kda_chunk_fwd
 * (without the chunk size), for gates with no lower bound.
 *
 * It runs the recurrence of the page "K3/notes/sections/sec-01.tex" (section
 * "KDA 递归核心") one token at a time with the state kept on chip, so it takes
 * exp(g) of single tokens only and is exact for any finite g -- for instance
 * the unbounded gate -exp(A_log) * softplus(z + dt_bias) of bounded_gate on
 * the page "metrale_model_weights/kimi_k3_host/kda.rs" (no lower bound),
 * which kda_chunk_fwd's -5 <= g <= 0 precondition excludes.  Slower than
 * kda_chunk_fwd where both apply.  Arguments, layouts, aliasing rules and
 * return codes are those of kda_chunk_fwd.
 */
int kda_recurrent_fwd(const void *q, const void *k, const void *v, const float *g,
                      const float *beta, const float *initial_state, void *out,
                      float *final_state, int B, int T, int H, int HV, int K, int V,
                      float scale, int dtype, void *stream);

/*
 * kda_recurrent_bwd -- gradients of the forward pass (kda_recurrent_fwd, or
 * kda_chunk_fwd where it applies: both compute the same function).
 *
 * Back-propagation through time over the recurrence, as the backward of
 * KDAFunction on the page "K3/kda/ops/reference/recurrent.py" derives it (the
 * derivation in its module docstring), with the gradient of the initial state
 * returned as well.  Given dL/do and dL/dS_T it returns
 * dL/dq, dL/dk, dL/dv, dL/dg, dL/dbeta and dL/dS0 for the same inputs and
 * scale as the forward call.  Exact for any finite g (no lower bound).
 *
 *   q, k, v, g, beta, initial_state, B, T, H, HV, K, V, scale, dtype
 *                   as for kda_recurrent_fwd (the forward inputs)
 *   dout          [B, T, HV, V]  dtype, dL/do
 *   dfinal_state  [B, HV, K, V]  fp32 or NULL (0): dL/dS_T
 *   dq, dk        [B, T, H, K]   dtype outputs (GQA: summed over the value
 *                                heads of each q/k head)
 *   dv            [B, T, HV, V]  dtype output
 *   dg            [B, T, HV, K]  fp32 output
 *   dbeta         [B, T, HV]     fp32 output
 *   dinitial_state [B, HV, K, V] fp32 output, or NULL (not written)
 *   workspace     device memory of at least
 *                 kda_recurrent_bwd_workspace_size(B, T, H, HV, K, V) bytes,
 *                 16-byte aligned, owned by the caller; its contents are
 *                 scratch (nothing carries over between calls).  May be NULL
 *                 when B * T == 0.
 * Outputs and the workspace may not overlap each other or any input.  With
 * T = 0 only dinitial_state is written (= dfinal_state, or zeros).
 * kda_recurrent_bwd_workspace_size returns the workspace size in bytes, or -1
 * (message in kda_last_error) for sizes kda_recurrent_bwd rejects.
 * Runs the forward recurrence once more (keeping its residuals and final
 * state in the workspace), then a reverse pass for the state gradient and a
 * forward pass for the gradients that need the state; all asynchronous on
 * `stream`.
 */
long long kda_recurrent_bwd_workspace_size(int B, int T, int H, int HV, int K, int V);
int kda_recurrent_bwd(const void *q, const void *k, const void *v, const float *g,
                      const float *beta, const float *initial_state, const void *dout,
                      const float *dfinal_state, void *dq, void *dk, void *dv, float *dg,
                      float *dbeta, float *dinitial_state, int B, int T, int H, int HV, int K,
                      int V, float scale, int dtype, void *workspace, long long workspace_bytes,
                      void *stream);

/*
 * kda_chunk_fwd_snapshots -- kda_chunk_fwd that also writes prefix snapshots
 * of the state, so that decoding can later resume from any whole multiple of
 * snapshot_every tokens (the prefix cache of the page
 * "metrale_model_weights/kimi_k3_host/kda.rs": its test
 * prefix_hit_wrong_slot_diverges keeps a clone of the state after each token
 * and resumes decoding from one; a resumed decode must equal the sequential
 * one).
 *
 *   snapshots       [B, NS, HV, K, V] fp32 with NS = T / snapshot_every
 *                   (rounded down); snapshot j of sequence b holds, for each
 *                   value head, the state after the first
 *                   (j + 1) * snapshot_every tokens, i.e. exactly what
 *                   final_state would hold for a call on that prefix.  So
 *                   snapshots[b][j] is laid out as the initial_state of one
 *                   sequence.  NULL: none are written (the call is then
 *                   kda_chunk_fwd).  Must not overlap any other argument.
 *   snapshot_every  tokens between snapshots; when snapshots is not NULL it
 *                   must be a positive multiple of the chunk size (32), else
 *                   KDA_EINVAL.
 * All other arguments, their layouts and the error behaviour are those of
 * kda_chunk_fwd.  When T is a multiple of snapshot_every the last snapshot
 * equals the final state.  Writing snapshots adds B*NS*HV*K*V*4 bytes of
 * stores to the call.
 */
int kda_chunk_fwd_snapshots(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *initial_state, void *out,
                            float *final_state, float *snapshots, int snapshot_every,
                            int B, int T, int H, int HV, int K, int V, float scale,
                            int chunk, int dtype, void *stream);

/*
 * Optional stages fused in front of the decode step, as the host decode on the
 * page "metrale_model_weights/kimi_k3_host/kda.rs" runs them (kda_decode_token:
 * conv_update, then kda_recurrent_step with l2norm_rows and a sigmoid on beta;
 * the gate from bounded_gate).  Zero-initialise and set what is wanted.
 */
typedef struct kda_decode_prologue {
    const float *conv_weight; /* [C, conv_kernel], C = 2*H*K + HV*V; NULL: no conv */
    float *conv_state;        /* [B, C, conv_kernel], oldest value first; updated in place */
    int conv_kernel;          /* 1..8 when conv_weight != NULL */
    int l2norm_qk;            /* nonzero: q, k rows become x / sqrt(sum x^2 + l2_eps) */
    float l2_eps;             /* e.g. 1e-6 */
    int gate_mode;            /* enum kda_gate_mode */
    const float *A_log;       /* [HV]      (BOUNDED, SOFTPLUS) */
    const float *dt_bias;     /* [HV * K]  (BOUNDED, SOFTPLUS) */
    float gate_lower_bound;   /* BOUNDED: g = lb * sigmoid(exp(A_log) * (z + dt_bias)) */
    int beta_is_logit;        /* nonzero: beta = sigmoid(beta argument) */
} kda_decode_prologue;

/*
 * kda_prefill_prologue -- the stages of the decode prologue applied to all T
 * tokens of a prefill at once, producing the inputs of kda_chunk_fwd from the
 * raw projections.  Per token, in the order of kda_decode_token on the page
 * "metrale_model_weights/kimi_k3_host/kda.rs": conv_update (causal depthwise
 * short conv over the packed q | k | v channels, then SiLU), l2norm_rows on
 * the q and k head rows, the gate of bounded_gate, a sigmoid on beta -- each
 * stage as selected in `pro` (NULL: none; q, k, v are then the channels of x
 * and g, beta pass through).
 *
 *   x        [B, T, 2*H*K + HV*V] dtype: q | k | v channels of every token
 *   gate     [B, T, HV, K] fp32: g (GATE_DIRECT) or the pre-activation z
 *   beta     [B, T, HV] fp32: beta, or its logit when pro->beta_is_logit
 *   pro->conv_state  [B, 2*H*K + HV*V, conv_kernel] fp32 or NULL: the conv
 *            registers before token 0 (oldest first), overwritten with those
 *            after token T-1, so that kda_decode_step continues the sequence;
 *            NULL means zero registers and none written
 *   q, k     [B, T, H, K] dtype;  v [B, T, HV, V] dtype
 *   g        [B, T, HV, K] fp32;  beta_out [B, T, HV] fp32
 *   B, T >= 0 (either 0: no-op); H, HV >= 1, HV % H == 0; K, V in {32, 64, 128};
 *   conv_kernel 1..8; dtype as above.
 * Outputs may not overlap each other or any input.  The SOFTPLUS gate mode can
 * produce g < -5, which kda_chunk_fwd does not accept (see its precondition).
 */
int kda_prefill_prologue(const void *x, const float *gate, const float *beta,
                         const kda_decode_prologue *pro, void *q, void *k, void *v,
                         float *g, float *beta_out, int B, int T, int H, int HV, int K,
                         int V, int dtype, void *stream);

/*
 * kda_output_gate -- full_rank_output_gate of the page
 * "metrale_model_weights/kimi_k3_host/kda.rs": for each row of head_dim values,
 *     y = sigmoid(gate) * o / sqrt(mean(o^2) + eps)
 * (an RMS norm of the attention output without a learned scale, gated
 * elementwise).
 *
 *   o, gate, y  [rows, head_dim] dtype; y may be o itself (in place) but may
 *               not otherwise overlap o or gate
 *   rows >= 0 (0: no-op); head_dim in {32, 64, 128}; eps >= 0 and finite
 *   (with eps = 0 an all-zero row gives NaN).
 */
int kda_output_gate(const void *o, const void *gate, void *y, long long rows, int head_dim,
                    float eps, int dtype, void *stream);

/*
 * kda_decode_step -- one token of the recurrence for B sequences, state
 * updated in place.
 *
 *   qkv    [B, 2*H*K + HV*V] dtype: q (H*K) | k (H*K) | v (HV*V) channels of one
 *          token, before the short conv when the prologue has one
 *   gate   [B, HV, K] fp32: g (GATE_DIRECT) or the pre-activation z
 *   beta   [B, HV] fp32: beta, or its logit when pro->beta_is_logit
 *   state  [B, HV, K, V] fp32, read and written in place
 *   out    [B, HV, V] dtype; must not overlap any other argument
 *   pro    NULL for the plain step (g and beta as given, no conv, no L2 norm)
 *   B >= 0 (0: no-op); H, HV >= 1, HV % H == 0; K, V in {32, 64, 128};
 *   scale <= 0 (or NaN) selects 1/sqrt(K); dtype as above.
 * With GATE_DIRECT the caller owns the range of g; the other modes produce
 * g <= 0.  Calls that share a state or conv_state buffer must be ordered by
 * the caller (same stream or events).
 */
int kda_decode_step(const void *qkv, const float *gate, const float *beta, float *state,
                    void *out, const kda_decode_prologue *pro, int B, int H, int HV,
                    int K, int V, float scale, int dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
