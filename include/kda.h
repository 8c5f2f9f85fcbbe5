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
 *    never allocates, frees, or keeps them; entry points that may need
 *    scratch memory take it as a workspace argument whose size a
 *    *_workspace_size query returns.  Tensors are dense row-major with the
 *    last dimension contiguous, and every base address must be 16-byte
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

#define KDA_ABI_VERSION 6

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
 *   chunk 0 selects the default, 32 (the only size built; the chunk bounds
 *   of delta_recurrence on "src/tinycenn_lm/research_layers.py" are checked
 *   the same way: other sizes return KDA_EUNSUPPORTED);
 *   dtype KDA_DTYPE_F32 or KDA_DTYPE_BF16;
 *   workspace     device scratch of workspace_bytes bytes, owned by the
 *                 caller, 16-byte aligned, disjoint from every other
 *                 argument; its contents carry nothing between calls.  It
 *                 must hold at least kda_chunk_fwd_workspace_size(...) bytes
 *                 for the same sizes (else KDA_EINVAL); when that is 0 it may
 *                 be NULL and is not touched.  workspace_bytes < 0: KDA_EINVAL.
 *
 * kda_chunk_fwd_workspace_size returns the workspace bytes kda_chunk_fwd (and
 * kda_chunk_fwd_snapshots) needs for these sizes, chunk and dtype, or -1 with
 * a message in kda_last_error for arguments those calls reject.  The fused
 * kernels built here keep every intermediate on chip, so it is 0 for all of
 * them; callers that query it stay correct for builds that need scratch.
 */
long long kda_chunk_fwd_workspace_size(int B, int T, int H, int HV, int K, int V, int chunk,
                                       int dtype);
int kda_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                  const float *beta, const float *initial_state, void *out,
                  float *final_state, int B, int T, int H, int HV, int K, int V,
                  float scale, int chunk, int dtype, void *workspace,
                  long long workspace_bytes, void *stream);

/*
 * kda_chunk_fwd_gated -- kda_chunk_fwd with the layer stages on either side
 * fused in: the gate and beta are formed inside the chunk kernel from their
 * pre-activations, and the output gate is applied to o, as the host layer on
 * the page "metrale_model_weights/kimi_k3_host/kda.rs" computes them
 * (bounded_gate with a lower bound, a sigmoid on the beta logit,
 * full_rank_output_gate).  Per token, value head hv and key channel f:
 *     g    = gate_lower_bound * sigmoid(exp(A_log[hv]) * (z + dt_bias[hv*K + f]))
 *     beta = sigmoid(beta_logit)
 * then o as kda_chunk_fwd computes it from q, k, v, g, beta, and, when
 * out_gate is given, per row of V values (o rounded to dtype first)
 *     y = sigmoid(out_gate) * o / sqrt(mean(o^2) + out_gate_eps).
 * g never goes to memory.  The output gate runs in the chunk kernel's o
 * stores when one workgroup holds whole rows of V (the launch splits V over
 * workgroups only when B * HV < 160), else as a pass over out after it.
 *
 *   z             [B, T, HV, K]  fp32 gate pre-activation (read where g would be)
 *   beta_logit    [B, T, HV]     fp32
 *   A_log         [HV] fp32;  dt_bias [HV * K] fp32
 *   gate_lower_bound  in [-5, 0] (so -5 <= g <= 0, kda_chunk_fwd's precondition)
 *   out_gate      [B, T, HV, V]  dtype, or NULL: out holds o itself
 *   out_gate_eps  finite, >= 0 (used when out_gate is given)
 *   out           [B, T, HV, V]  dtype: y (or o); may not overlap any input
 * q, k, v, initial_state, final_state, sizes, scale, chunk, the workspace
 * (kda_chunk_fwd_workspace_size gives its size here too) and the errors are
 * those of kda_chunk_fwd.  Built for KDA_DTYPE_BF16 only (KDA_EUNSUPPORTED
 * for KDA_DTYPE_F32).  kda_prefill_prologue with g and beta_out NULL gives
 * its q, k, v inputs without writing g.
 */
int kda_chunk_fwd_gated(const void *q, const void *k, const void *v, const float *z,
                        const float *beta_logit, const float *A_log, const float *dt_bias,
                        float gate_lower_bound, const float *initial_state, const void *out_gate,
                        float out_gate_eps, void *out, float *final_state, int B, int T, int H,
                        int HV, int K, int V, float scale, int chunk, int dtype, void *workspace,
                        long long workspace_bytes, void *stream);

/*
 * kda_recurrent_fwd -- the same computation and interface as kda_chunk_fwd
 * (without the chunk size and the workspace), for gates with no lower bound.
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
 * kda_chunk_fwd_unbounded -- kda_chunk_fwd for gates with no lower bound, on
 * the matrix cores: the chunk form of kda_chunk_fwd with the in-chunk decay
 * factors split around several reference rows (none more than 4 tokens from
 * the rows it serves) instead of one, so that no factor leaves fp32 however
 * strongly a token decays -- for instance under the unbounded gate
 * -exp(A_log) * softplus(z + dt_bias) of bounded_gate on the page
 * "metrale_model_weights/kimi_k3_host/kda.rs" (no lower bound).  The in-chunk
 * matrices of every chunk are formed first by a chunk-parallel pass into the
 * workspace, then the chunk kernel carries the state.
 *
 *   g  [B, T, HV, K]  fp32, log-space decay; PRECONDITION g <= 0 (finite or
 *      -inf).  Each token's g is floored at -17 first: a token that would keep
 *      less than e^-17 (about 4e-8) of the state keeps exactly that much,
 *      a change of at most 4e-8 of the state's magnitude per such token.
 *   workspace  device scratch of workspace_bytes bytes owned by the caller,
 *      16-byte aligned, disjoint from every other argument, at least
 *      kda_chunk_fwd_unbounded_workspace_size(...) bytes (B * HV * ceil(T/32)
 *      * 7168: bf16 in-chunk matrices of every chunk); its contents carry
 *      nothing between calls (else KDA_EINVAL).
 * q, k, v, beta, initial_state, out, final_state, sizes, scale and the
 * errors are those of kda_chunk_fwd (chunk 32).  Built for KDA_DTYPE_BF16
 * only: KDA_EUNSUPPORTED for KDA_DTYPE_F32, whose unbounded gates go to
 * kda_recurrent_fwd.
 *
 * kda_chunk_fwd_unbounded_workspace_size returns those bytes for these sizes,
 * or -1 with a message in kda_last_error for arguments the call rejects.
 */
long long kda_chunk_fwd_unbounded_workspace_size(int B, int T, int H, int HV, int K, int V, int dtype);
int kda_chunk_fwd_unbounded(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *initial_state, void *out,
                            float *final_state, int B, int T, int H, int HV, int K, int V,
                            float scale, int dtype, void *workspace, long long workspace_bytes,
                            void *stream);

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
 * Runs the forward recurrence once more (keeping its residuals, its final
 * state and the state every 1024 tokens in the workspace), then, one slab of
 * 1024 tokens at a time from the last, a reverse pass for the state gradient,
 * a forward pass for the gradients that need the state and the sums that
 * finish them; all asynchronous on `stream`.  The workspace therefore grows
 * with T only by the residuals (4 V bytes per token and value head): 1.16 GB
 * at B = 1, T = 8192, HV = 96, K = V = 128.
 */
long long kda_recurrent_bwd_workspace_size(int B, int T, int H, int HV, int K, int V);
int kda_recurrent_bwd(const void *q, const void *k, const void *v, const float *g,
                      const float *beta, const float *initial_state, const void *dout,
                      const float *dfinal_state, void *dq, void *dk, void *dv, float *dg,
                      float *dbeta, float *dinitial_state, int B, int T, int H, int HV, int K,
                      int V, float scale, int dtype, void *workspace, long long workspace_bytes,
                      void *stream);

/*
 * kda_chunk_bwd -- the same gradients as kda_recurrent_bwd for bf16 inputs in
 * the bounded-gate range of kda_chunk_fwd (-5 <= g <= 0), computed in the
 * chunk form on the matrix cores.
 *
 * The chunk form of delta_recurrence on the page
 * "src/tinycenn_lm/research_layers.py" (as kda_chunk_fwd evaluates it),
 * differentiated chunk by chunk in reverse: the backward of KDAFunction on
 * the page "K3/kda/ops/reference/recurrent.py" restated for chunks of 32
 * tokens.  Arguments, layouts, outputs and return codes as kda_recurrent_bwd,
 * with dtype KDA_DTYPE_BF16 only (others: KDA_EUNSUPPORTED) and
 *   workspace     device memory of at least
 *                 kda_chunk_bwd_workspace_size(B, T, H, HV, K, V, dtype)
 *                 bytes, 16-byte aligned, owned by the caller, scratch
 *                 between calls; may be NULL when B * T == 0.
 * With g outside [-5, 0] the result is not defined (use kda_recurrent_bwd).
 * Runs the chunked forward once over the sequence (keeping the final state
 * and the state every 1024 tokens), then, one slab of 1024 tokens at a time
 * from the last: the forward over the slab again (the state at every chunk
 * start and the in-chunk solve's input and result), a chunk-parallel pass
 * forming the reverse chain's operands, the reverse chain of state gradients
 * (one workgroup per value head), a chunk-parallel pass for dq, dk, dv, dbeta
 * and the dg terms, and the reverse sum that forms dg.  The chain runs on
 * `stream`; the forward passes, the operand pass, and the gradient pass
 * with the dg sum run on three further streams of the library's (one set per
 * device, default priority, created on the first call), ordered against
 * `stream` by events; the call returns when all is enqueued, and work
 * enqueued on `stream` afterwards runs after all of it.  Calls from several
 * host threads on one device are serialized while they enqueue.  While
 * `stream` is being captured into a HIP graph, every pass is enqueued in the
 * same order on `stream` alone (no further streams or events: same results,
 * no overlap between the passes).  Workspace
 * about 1.5 GB at B = 1, T = 8192, HV = 96, K = V = 128.
 * kda_chunk_bwd_workspace_size returns the workspace size in bytes, or -1
 * (message in kda_last_error) for sizes or a dtype kda_chunk_bwd rejects.
 */
long long kda_chunk_bwd_workspace_size(int B, int T, int H, int HV, int K, int V, int dtype);
int kda_chunk_bwd(const void *q, const void *k, const void *v, const float *g, const float *beta,
                  const float *initial_state, const void *dout, const float *dfinal_state, void *dq,
                  void *dk, void *dv, float *dg, float *dbeta, float *dinitial_state, int B, int T,
                  int H, int HV, int K, int V, float scale, int dtype, void *workspace,
                  long long workspace_bytes, void *stream);

/*
 * kda_chunk_bwd_saved -- kda_chunk_bwd given the forward pass's own states,
 * so that it does not run the forward over the whole sequence again (its
 * first step).  For training, where the forward has just run: the forward of
 * the same inputs by kda_chunk_fwd_snapshots with snapshot_every = 1024
 * provides both.
 *   saved_states  [B, T / 1024, HV, K, V] fp32: the state after the first
 *                 1024, 2048, ... tokens of each sequence (the snapshots of
 *                 kda_chunk_fwd_snapshots at snapshot_every = 1024); may be
 *                 NULL when T <= 1024 (else KDA_EINVAL)
 *   final_state   [B, HV, K, V] fp32: the forward's final state; needed when
 *                 dfinal_state is given (for dg's final-state term; else
 *                 KDA_EINVAL), otherwise not read
 * Both are inputs (not written; neither may overlap an output or the
 * workspace).  Everything else -- arguments, layouts, the workspace and its
 * size, the streams, return codes -- as kda_chunk_bwd.  The gradients
 * are those of the forward that produced the states: with states from
 * different inputs they are not defined.
 */
int kda_chunk_bwd_saved(const void *q, const void *k, const void *v, const float *g, const float *beta,
                        const float *initial_state, const float *saved_states, const float *final_state,
                        const void *dout, const float *dfinal_state, void *dq, void *dk, void *dv, float *dg,
                        float *dbeta, float *dinitial_state, int B, int T, int H, int HV, int K, int V,
                        float scale, int dtype, void *workspace, long long workspace_bytes, void *stream);

/*
 * kda_recurrent_bwd_noalloc -- kda_recurrent_bwd for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The same arguments, results, validation
 * and return codes as kda_recurrent_bwd, without the workspace: a scratch
 * array of KDA_NOALLOC_SCRATCH_BYTES (128 MiB) in the library's own device
 * memory takes its place, one per GPU, held from the first call on that GPU
 * until the process ends.  Nothing is allocated or freed by the call.
 *  - Sizes whose kda_recurrent_bwd_workspace_size exceeds the array return
 *    KDA_EUNSUPPORTED, with no side effects (at K = V = 128, B = 1, T = 1024,
 *    HV = 16 fits; the HV96 shape at T = 8192 needs 1.16 GB and does not).
 *  - The array serves the GPU `stream` runs on (the current device for the
 *    NULL stream).  Every call on that GPU shares it and leaves its last
 *    contents there; nothing in it needs clearing, since each call writes
 *    every scratch value before reading it.  Calls that overlap in time on
 *    one GPU (on different streams, or from several host threads without
 *    ordering) RACE on the array and give wrong gradients: order them on one
 *    stream or with events.
 *  - The first call on a GPU looks up the array's device address
 *    (hipGetSymbolAddress); a failure there returns KDA_EHIP.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (128ull << 20)
int kda_recurrent_bwd_noalloc(const void *q, const void *k, const void *v, const float *g,
                              const float *beta, const float *initial_state, const void *dout,
                              const float *dfinal_state, void *dq, void *dk, void *dv, float *dg,
                              float *dbeta, float *dinitial_state, int B, int T, int H, int HV,
                              int K, int V, float scale, int dtype, void *stream);

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
 * All other arguments (the workspace included: its size is
 * kda_chunk_fwd_workspace_size), their layouts and the error behaviour are
 * those of kda_chunk_fwd.  When T is a multiple of snapshot_every the last snapshot
 * equals the final state.  Writing snapshots adds B*NS*HV*K*V*4 bytes of
 * stores to the call.
 */
int kda_chunk_fwd_snapshots(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *initial_state, void *out,
                            float *final_state, float *snapshots, int snapshot_every,
                            int B, int T, int H, int HV, int K, int V, float scale,
                            int chunk, int dtype, void *workspace, long long workspace_bytes,
                            void *stream);

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
    int conv_ring;            /* nonzero: conv_state is a ring of slot arrays (below) */
    int conv_pos;             /* ring: the slot of the oldest register, 0..conv_kernel-1 */
} kda_decode_prologue;

/*
 * Two layouts of the conv registers, the last conv_kernel (W) inputs of each
 * channel (the window of conv_update on the page
 * "metrale_model_weights/kimi_k3_host/kda.rs"):
 *   conv_ring == 0: [B, C, W], oldest first.  A decode step shifts each row
 *     and appends the token, so it reads and rewrites all W values.
 *   conv_ring != 0: [W, B, C], W slot arrays used as a ring.  Register j
 *     (0 = oldest) of channel c of sequence b sits in slot (conv_pos + j) % W,
 *     at conv_state[((conv_pos + j) % W) * B * C + b * C + c].  A decode step
 *     reads the W - 1 newest registers and writes the token into slot
 *     conv_pos alone (the oldest, which its window no longer uses); a
 *     prefill of T tokens writes its last min(T, W) inputs into slots
 *     (conv_pos + t) % W.  The library never changes conv_pos: after a call
 *     the caller advances it, by 1 for a decode step and by T for a prefill
 *     (mod W).  Both layouts give identical results; the ring moves W - 1
 *     reads and one write per channel and token instead of W of each.
 *     conv_pos is an argument of the call, so a decode loop under HIP graph
 *     capture captures one graph per slot and replays them in turn.
 */

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
 * g and beta_out may both be NULL: the gate and beta stages are then skipped
 * and gate and beta are not read (kda_chunk_fwd_gated forms them itself).
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
 * updated in place: the host decode of the page
 * "metrale_model_weights/kimi_k3_host/kda.rs" (kda_decode_token: conv_update
 * on the packed channels, then kda_recurrent_step: l2norm_rows on q and k, a
 * sigmoid on the beta logit, the gate from bounded_gate, and the step of the
 * recurrence above on the in-place recurrent state, readout after the write
 * with scale 1/sqrt(K)), the stages selected by `pro`.  The step itself is
 * the four-step update of "K3/notes/sections/sec-01.tex" (section "KDA 递归核心")
 * for T = 1.
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
