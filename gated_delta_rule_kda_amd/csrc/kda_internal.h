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
    float *snap;                // [B,NS,HV,K,V] prefix snapshots or nullptr
    int snap_chunks;            // chunks between snapshots (>= 1 when snap is set)
    int NS;                     // snapshots per sequence, T / (32 * snap_chunks)
    float *aux;                 // token-recurrent kernel only: when set, the
                                // residuals r_t = v_t - k_t^T S_dec ([B,T,HV,V]
                                // fp32) are written here instead of out
    int B, T, H, HV, K, V;
    float scale;
    bool bf16;
};

// Arguments of one decode step.
struct DecodeArgs {
    const void *qkv;            // [B, 2HK + HV V] (dtype)
    const float *gate;          // [B,HV,K]
    const float *beta;          // [B,HV]
    float *state;               // [B,HV,K,V]
    void *out;                  // [B,HV,V] (dtype)
    const float *conv_w;        // [C,KW] or nullptr
    float *conv_state;          // [B,C,KW]
    int conv_kernel;
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
    float *e;                   // [B,T,HV,K]: per-token terms of dg
    float *bs;                  // [B,HV,NB+1,K]: sums of e over blocks of kDgBlock
                                // tokens, then the final-state term of dg
    int NCB, NB;
    int B, T, H, HV, K, V;
    float scale;
    bool bf16;
};
constexpr int kBwdCols = 32;    // state columns per workgroup of the backward passes
constexpr int kDgBlock = 64;    // tokens per block of the reverse sum that forms dg
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
