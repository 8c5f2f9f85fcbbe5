// Internal interface between the C-ABI layer (kda_api.hip) and the kernels.
// Sizes reaching these launchers have already been validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Arguments of one prefill call; pointers are device pointers.
struct PrefillArgs {
    const void *q, *k, *v;      // [B,T,H,K], [B,T,H,K], [B,T,HV,V] (dtype)
    const float *g, *beta;      // [B,T,HV,K], [B,T,HV]
    const float *S0;            // [B,HV,K,V] or nullptr
    void *out;                  // [B,T,HV,V] (dtype)
    float *ST;                  // [B,HV,K,V] or nullptr
    float *snap;                // [B,NS,HV,K,V] prefix snapshots or nullptr (also
                                // the residual variant of the token-recurrent
                                // kernel: the states at the backward's slab starts)
    int snap_chunks;            // chunks of 32 tokens between snapshots (>= 1 when snap is set)
    int NS;                     // snapshots per sequence, T / (32 * snap_chunks)
    float *aux;                 // token-recurrent kernel only: when set, the
                                // residuals r_t = v_t - k_t^T S_dec ([B,T,HV,V]
                                // fp32) are written here instead of out
    int B, T, H, HV, K, V;
    float scale;
    bool bf16;
    // Fused layer stages (kda_chunk_fwd_gated; bf16 chunk kernel only).
    // A_log set: g holds the pre-activation z and beta the logits, and the
    // kernel forms g = lower_bound * sigmoid(exp(A_log[hv]) (z + dt_bias[hv K + f]))
    // and beta = sigmoid(logit) itself.
    const float *A_log, *dt_bias;   // [HV], [HV*K] or nullptr
    float lower_bound;
    // ogate set: out receives y = sigmoid(ogate) * o / sqrt(mean(o^2) + og_eps)
    // per row of V values, o rounded to the output dtype first.
    const void *ogate;              // [B,T,HV,V] (dtype) or nullptr
    float og_eps;
    // Sub-range of the sequences (bf16 chunk kernel): the call processes
    // tokens [t_off, t_off + T) of sequences Tseq tokens long in memory
    // (Tseq = 0 means T, t_off = 0: the whole sequence).
    int t_off, Tseq;
    // Chunked backward's forward pass (bf16 chunk kernel, with snap): when
    // u_out is set, U = (I + A_kk)^-1 diag(beta) (v - (k Gamma) M) of every
    // chunk goes to u_out ([B, Lw, HV, V] fp32, token index relative to
    // t_off) and no o is written.
    float *u_out;
    int Lw;
    bool bwd;                   // the backward's forward pass: no o; U where set
    long long s0_bstride;       // elements between the sequences of S0 (0: HV K V)
    // Gates without a lower bound (bf16 chunk kernel): the in-chunk matrices
    // come from img ([B,HV,NC,kUnbImgElems] bf16, written by the pass of
    // kda_unb_prep.hip) and the state products use forward-only decay factors.
    const uint16_t *img;
    bool unb;
};

// Floor of each token's log-decay on the unbounded chunked path (natural log):
// e^-17 ~ 4e-8 of the state is the least a token keeps there.  With it, the
// in-chunk factors around a reference row at most 4 tokens away stay within
// [2^-98, 2^98].
constexpr float kUnbFloor = -17.0f;
// bf16 elements of one chunk's in-chunk matrices on that path (A_qk, -A21,
// T11, T22, each as hi/lo pairs)
constexpr int kUnbImgElems = 3584;

// Arguments of one decode step.
struct DecodeArgs {
    const void *qkv;            // [B, 2HK + HV V] (dtype)
    const float *gate;          // [B,HV,K]
    const float *beta;          // [B,HV]
    float *state;               // [B,HV,K,V]
    void *out;                  // [B,HV,V] (dtype)
    const float *conv_w;        // [C,KW] or nullptr
    float *conv_state;          // [B,C,KW]; ring: [KW,B,C], oldest register in slot conv_pos
    int conv_kernel;
    int conv_ring, conv_pos;
    int l2norm;
    float l2_eps;
    int gate_mode;
    const float *A_log, *dt_bias;
    float lower_bound;
    int beta_is_logit;
    int B, H, HV, K, V;
    float scale;
    bool bf16;
};

// Arguments of the prefill prologue (the decode prologue's stages over T tokens).
struct PrologueArgs {
    const void *x;              // [B,T,C] (dtype), C = 2HK + HV V
    const float *conv_w;        // [C,KW] or nullptr (no conv)
    const float *conv_state;    // [B,C,KW] registers before token 0, or nullptr (zeros)
    float *conv_state_out;      // [B,C,KW] registers after token T-1, or nullptr
    int KW;
    int conv_ring, conv_pos;    // ring: both [KW,B,C], oldest register in slot conv_pos
    int l2norm;
    float l2_eps;
    const float *gate;          // [B,T,HV,K]: g, or z for the gate modes
    int gate_mode;              // 0 direct, 1 bounded, 2 softplus
    const float *A_log, *dt_bias;
    float lower_bound;
    const float *beta_in;       // [B,T,HV]
    int beta_is_logit;
    void *q, *k, *v;            // [B,T,H,K], [B,T,H,K], [B,T,HV,V] (dtype)
    float *g, *beta_out;        // [B,T,HV,K], [B,T,HV]
    int B, T, H, HV, K, V;
    bool bf16;
};

// Arguments of the output gate: rows of D values.
struct OutputGateArgs {
    const void *o, *gate;       // [rows, D] (dtype)
    void *y;                    // [rows, D] (dtype), may be o
    long rows;
    int D;
    float eps;
    bool bf16;
};

// Arguments of the backward of the token recurrence (kda_recurrent_bwd).
struct BwdArgs {
    const void *q, *k, *v;      // [B,T,H,K], [B,T,H,K], [B,T,HV,V] (dtype)
    const float *g, *beta;      // [B,T,HV,K], [B,T,HV]
    const float *S0;            // [B,HV,K,V] or nullptr
    const void *dout;           // [B,T,HV,V] (dtype): dL/do
    const float *dST;           // [B,HV,K,V] or nullptr: dL/dS_T
    void *dq, *dk, *dv;         // [B,T,H,K], [B,T,H,K], [B,T,HV,V] (dtype)
    float *dg, *dbeta;          // [B,T,HV,K], [B,T,HV]
    float *dS0;                 // [B,HV,K,V] or nullptr
    // workspace, fp32
    float *r, *dr;              // [B,T,HV,V]: forward residuals, their gradients
    float *ST;                  // [B,HV,K,V]: forward final state
    float *daP, *dqP, *dkrP;    // [NCB,B,T,HV,K]: per column-block partial sums
    float *e;                   // [B,Ls,HV,K]: per-token terms of dg
    float *bs;                  // [B,HV,NB,K]: sums of e over blocks of kDgBlock tokens
    int NCB, NB;                // column blocks; dg blocks per slab (Ls / kDgBlock)
    // The passes after the forward one run slab by slab, the last slab first:
    // tokens [t_begin, t_end) of every sequence per launch.  dr, the partial
    // sums and e hold one slab (slab-local token index, Ls tokens per
    // sequence); the state gradient D and the dg carry go from slab to slab.
    int t_begin, t_end, Ls;
    float *Dc;                  // [B,HV,K,V]: D at the start of the slab just done
    const float *snap;          // [B,NS,HV,K,V]: forward state after (j+1) Ls tokens
    int NS;
    const float *gc_in;         // [B,HV,K]: dg carried in (later tokens, the final-state term)
    float *gc_out;              // [B,HV,K]: dg carried to the slab before
    int B, T, H, HV, K, V;
    float scale;
    bool bf16;
};
// Arguments of the chunked backward (kda_chunk_bwd, bf16 inputs, bounded gate).
struct ChunkBwdArgs {
    const void *q, *k, *v;      // [B,T,H,K], [B,T,H,K], [B,T,HV,V] bf16
    const float *g, *beta;      // [B,T,HV,K], [B,T,HV]
    const float *S0;            // [B,HV,K,V] or nullptr
    const void *dout;           // [B,T,HV,V] bf16
    const float *dST;           // [B,HV,K,V] or nullptr
    void *dq, *dk, *dv;         // [B,T,H,K], [B,T,H,K], [B,T,HV,V] bf16
    float *dg, *dbeta;          // [B,T,HV,K], [B,T,HV]
    float *dS0;                 // [B,HV,K,V] or nullptr
    // workspace (fp32): see chunk_bwd_layout in kda_api.hip
    float *ST, *snap1, *Dc, *snapc, *U, *img, *dR, *dMs, *e, *cs, *gc;
    float *snapc2, *U2, *img2;   // second copies for the slabs of odd index
    float *dR2, *dMs2;
    int Ls;                     // tokens per slab (a multiple of 32)
    int NS1;                    // slab starts kept by the first forward pass (slabs - 1)
    // The forward's own states instead of the first forward pass: ST (S_T)
    // and snap1 ([B, NSsaved, HV, K, V], the state after every Ls tokens)
    // come from the caller and nothing recomputes them.
    bool saved;
    int NSsaved;
    int B, T, H, HV, K, V;
    float scale;
};
hipError_t launch_chunk_backward(const ChunkBwdArgs &a, hipStream_t stream);
// floats of one chunk's operand image (the chunked backward's pre-pass output)
int chunk_bwd_image_floats(int K);

constexpr int kBwdCols = 32;    // state columns per workgroup of the backward passes
constexpr int kDgBlock = 64;    // tokens per block of the reverse sum that forms dg
constexpr int kBwdSlab = 1024;  // tokens per slab of the backward passes (a multiple of kDgBlock)
constexpr int kMaxConvKernel = 8;

// Launch on `stream`; return the hipError_t of the launch.
hipError_t launch_prologue(const PrologueArgs &a, hipStream_t stream);
hipError_t launch_recurrent(const PrefillArgs &a, hipStream_t stream);
// the backward after the forward residuals and final state are in the
// workspace: the reverse state-gradient pass, the forward gradient pass and
// the reductions
hipError_t launch_backward(const BwdArgs &a, hipStream_t stream);
hipError_t launch_output_gate(const OutputGateArgs &a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillArgs &a, hipStream_t stream);
// kda_chunk_fwd_unbounded: the in-chunk matrix pass into img, then the bf16
// chunk kernel's unbounded instantiation
hipError_t launch_unbounded_prefill(const PrefillArgs &a, uint16_t *img, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

// ---------------------------------------------------------------- device helpers

__device__ __forceinline__ float bf16_bits_to_float(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16 with round-to-nearest-even (NaN stays NaN).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float sigmoidf_dev(float x) { return 1.0f / (1.0f + __expf(-x)); }

}  // namespace kda
