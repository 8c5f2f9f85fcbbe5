// KDA single-token decode step for gfx950.
//
// One workgroup per (sequence b, q/k head h).  It runs the optional prologue
// of the host decode on the page "metrale_model_weights/kimi_k3_host/kda.rs"
// (conv_update with SiLU on the q|k|v channels, l2norm_rows on q and k, the
// gate of bounded_gate, a sigmoid on beta as in kda_recurrent_step), then, for
// each of the G = HV/H value heads that read head h, one step of the
// recurrence of the page "K3/notes/sections/sec-01.tex" (section "KDA 递归核心",
// four-step update):
//     S_dec = exp(g) (.) S,  r = v - k^T S_dec,  S = S_dec + (beta k) (x) r,
//     o = scale q^T S.
// The step is a pure HBM stream over the fp32 [K x V] state.  It is read once
// and written once: the readout uses q^T S = q^T S_dec + (q.k) beta r, so both
// column reductions (k^T S_dec and q^T S_dec) come from the same registers and
// the new state is written straight from them.
//
// Layout: each thread owns one float4 column group (4 consecutive V columns)
// of K / RPP state rows, so a wave's loads and stores cover whole 16-byte
// segments of consecutive rows.  At K = V = 128 a workgroup has 512 threads
// holding 8 float4 each: smaller per-thread footprints keep more workgroups
// resident, which streams the read-modify-write of the state faster than
// fewer, fatter threads.  Handling all G value heads of a q/k head in one
// workgroup means the q/k conv channels are shifted exactly once.

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kMaxThreads = 512;   // threads per workgroup for the largest state tiles
constexpr int kMaxConv = 8;

typedef float f32x4 __attribute__((ext_vector_type(4)));
// The state is streamed: each 16-byte segment is read once and written once
// per step, so both go through the non-temporal path and do not displace
// reusable lines (conv weights, dt_bias) from the caches.
__device__ __forceinline__ float4 ld_stream(const float4 *p) {
    return __builtin_bit_cast(float4, __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p)));
}
__device__ __forceinline__ void st_stream(float4 *p, const float4 &x) {
    __builtin_nontemporal_store(__builtin_bit_cast(f32x4, x), reinterpret_cast<f32x4 *>(p));
}

__device__ __forceinline__ float load_io(const void *p, size_t i, bool bf16) {
    return bf16 ? bf16_bits_to_float(static_cast<const uint16_t *>(p)[i])
                : static_cast<const float *>(p)[i];
}

__device__ __forceinline__ void store_io(void *p, size_t i, float x, bool bf16) {
    if (bf16)
        static_cast<uint16_t *>(p)[i] = float_to_bf16_bits(x);
    else
        static_cast<float *>(p)[i] = x;
}

__device__ __forceinline__ float sigmoid_acc(float x) { return 1.0f / (1.0f + expf(-x)); }

// One input channel of the token: the raw value, or conv_update + SiLU.
__device__ __forceinline__ float channel_value(const DecodeArgs &a, int b, int c, int C) {
    const float x = load_io(a.qkv, static_cast<size_t>(b) * C + c, a.bf16);
    if (a.conv_w == nullptr) return x;
    const int KW = a.conv_kernel;
    const float *w = a.conv_w + static_cast<size_t>(c) * KW;
    if (a.conv_ring) {
        // slot arrays [KW][B][C]: register j (0 = oldest) in slot (conv_pos + j) % KW.
        // The window is registers 1..KW-1 and the token; the token goes into
        // the oldest register's slot, the only store.
        const size_t slot = static_cast<size_t>(a.B) * C;
        float *col = a.conv_state + static_cast<size_t>(b) * C + c;
        if (KW == 4) {
            // the common width: the weights in one 16-byte load, the slots of
            // registers 1..3 by a mask
            const float4 wv = *reinterpret_cast<const float4 *>(w);
            const float r1 = col[((a.conv_pos + 1) & 3) * slot];
            const float r2 = col[((a.conv_pos + 2) & 3) * slot];
            const float r3 = col[((a.conv_pos + 3) & 3) * slot];
            col[a.conv_pos * slot] = x;
            const float acc = fmaf(wv.w, x, fmaf(wv.z, r3, fmaf(wv.y, r2, wv.x * r1)));
            return acc * sigmoid_acc(acc);
        }
        float acc = 0.f;
#pragma unroll
        for (int j = 1; j < kMaxConv; ++j)
            if (j < KW) {
                const int p = a.conv_pos + j < KW ? a.conv_pos + j : a.conv_pos + j - KW;
                acc = fmaf(w[j - 1], col[p * slot], acc);
            }
        acc = fmaf(w[KW - 1], x, acc);
        col[a.conv_pos * slot] = x;
        return acc * sigmoid_acc(acc);
    }
    float *st = a.conv_state + (static_cast<size_t>(b) * C + c) * KW;
    if (KW == 4) {
        // the common width: one 16-byte load and store of the channel's register
        const float4 o = *reinterpret_cast<const float4 *>(st);
        const float4 wv = *reinterpret_cast<const float4 *>(w);
        const float4 n = make_float4(o.y, o.z, o.w, x);
        *reinterpret_cast<float4 *>(st) = n;
        const float acc = fmaf(wv.w, n.w, fmaf(wv.z, n.z, fmaf(wv.y, n.y, wv.x * n.x)));
        return acc * sigmoid_acc(acc);
    }
    float reg[kMaxConv];
#pragma unroll
    for (int j = 0; j < kMaxConv; ++j)
        if (j + 1 < KW) reg[j] = st[j + 1];
    reg[KW - 1] = x;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxConv; ++j)
        if (j < KW) {
            acc = fmaf(w[j], reg[j], acc);
            st[j] = reg[j];
        }
    return acc * sigmoid_acc(acc);
}

// Sum over the workgroup of NW waves; every thread gets the result (fixed
// order, so the result is reproducible).  `red` holds NW floats.
template <int NW>
__device__ __forceinline__ float block_sum(float x, float *red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wave] = x;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += red[w];
    return t;
}

// Threads of a workgroup: one float4 column group of at least 4 state rows each,
// capped at kMaxThreads.
template <int K, int V>
constexpr int decode_threads() { return K * V / 16 < kMaxThreads ? K * V / 16 : kMaxThreads; }

// At most 80 VGPRs (6 waves per SIMD): three 512-thread workgroups per CU
// instead of two, so one workgroup's prologue and reductions overlap the
// others' state streams (3 % faster at B256 HV96 K = V = 128 than the 93 the
// compiler picks unbounded; a 64-VGPR budget spills).
template <int K, int V>
__global__ __launch_bounds__((decode_threads<K, V>()), 6) void decode_kernel(DecodeArgs a) {
    constexpr int kThreads = decode_threads<K, V>();
    constexpr int kWaves = kThreads / 64;
    constexpr int TPR = V / 4;          // threads per state row (one float4 each)
    constexpr int RPP = kThreads / TPR; // state rows per pass of the workgroup
    constexpr int NP = K / RPP;         // passes; each thread holds NP float4
    static_assert(K % RPP == 0, "state rows must tile the workgroup");

    __shared__ float s_q[K], s_k[K], s_v[V], s_eg[K], s_u[V];
    __shared__ float s_red[kWaves][2][V];
    __shared__ float s_tmp[kWaves];

    const int tid = threadIdx.x;
    const int b = blockIdx.x / a.H;
    const int h = blockIdx.x % a.H;
    const int G = a.HV / a.H;
    const int C = 2 * a.H * K + a.HV * V;
    const int c4 = tid % TPR;
    const int r0 = tid / TPR;

    // The state of the first value head streams in while the prologue runs.
    float4 st[NP];
    {
        const float4 *S0 = reinterpret_cast<const float4 *>(
            a.state + (static_cast<size_t>(b) * a.HV + h * G) * K * V);
#pragma unroll
        for (int p = 0; p < NP; ++p) st[p] = ld_stream(&S0[(p * RPP + r0) * TPR + c4]);
    }

    // ---- q/k channels of head h (conv + SiLU when enabled)
    for (int i = tid; i < 2 * K; i += kThreads) {
        const int c = (i < K) ? h * K + i : a.H * K + h * K + (i - K);
        const float y = channel_value(a, b, c, C);
        if (i < K) s_q[i] = y; else s_k[i - K] = y;
    }
    __syncthreads();
    float qk;
    {
        // L2 norm of the q and k rows (eps inside the root), then q.k.
        float sq = 0.f, sk = 0.f;
        for (int f = tid; f < K; f += kThreads) {
            sq += s_q[f] * s_q[f];
            sk += s_k[f] * s_k[f];
        }
        float inv_q = 1.f, inv_k = 1.f;
        if (a.l2norm) {
            sq = block_sum<kWaves>(sq, s_tmp);
            sk = block_sum<kWaves>(sk, s_tmp);
            inv_q = 1.0f / sqrtf(sq + a.l2_eps);
            inv_k = 1.0f / sqrtf(sk + a.l2_eps);
        }
        float d = 0.f;
        for (int f = tid; f < K; f += kThreads) {
            const float qn = s_q[f] * inv_q * a.scale;  // readout scale folded into q
            const float kn = s_k[f] * inv_k;
            s_q[f] = qn;
            s_k[f] = kn;
            d += qn * kn;
        }
        qk = block_sum<kWaves>(d, s_tmp);
    }

    for (int gi = 0; gi < G; ++gi) {
        const int hv = h * G + gi;
        const size_t bhv = static_cast<size_t>(b) * a.HV + hv;
        float4 *S = reinterpret_cast<float4 *>(a.state + bhv * K * V);

        // Later value heads issue their state loads first; the value channels
        // and the gate below hide part of the latency.
        if (gi > 0)
#pragma unroll
            for (int p = 0; p < NP; ++p) st[p] = ld_stream(&S[(p * RPP + r0) * TPR + c4]);

        for (int j = tid; j < V; j += kThreads)
            s_v[j] = channel_value(a, b, 2 * a.H * K + hv * V + j, C);
        for (int f = tid; f < K; f += kThreads) {
            const float z = a.gate[bhv * K + f];
            float g = z;
            if (a.gate_mode != 0) {
                const float x = z + a.dt_bias[hv * K + f];
                const float decay = expf(a.A_log[hv]);
                if (a.gate_mode == 1) {
                    g = a.lower_bound * sigmoid_acc(decay * x);
                } else {
                    // softplus in its overflow-safe form max(x,0) + log1p(exp(-|x|))
                    g = -decay * (fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))));
                }
            }
            s_eg[f] = expf(g);
        }
        float beta = a.beta[bhv];
        if (a.beta_is_logit) beta = sigmoid_acc(beta);
        __syncthreads();

        // Column partial sums of k^T S_dec and q^T S_dec over this thread's rows.
        float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int row = p * RPP + r0;
            const float e = s_eg[row];
            const float ke = s_k[row] * e, qe = s_q[row] * e;
            const float s4[4] = {st[p].x, st[p].y, st[p].z, st[p].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pk[j] = fmaf(ke, s4[j], pk[j]);
                pq[j] = fmaf(qe, s4[j], pq[j]);
            }
        }
#pragma unroll
        for (int off = TPR; off < 64; off <<= 1)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pk[j] += __shfl_xor(pk[j], off);
                pq[j] += __shfl_xor(pq[j], off);
            }
        const int wave = tid >> 6, lane = tid & 63;
        if (lane < TPR)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s_red[wave][0][c4 * 4 + j] = pk[j];
                s_red[wave][1][c4 * 4 + j] = pq[j];
            }
        __syncthreads();
        for (int j = tid; j < V; j += kThreads) {
            float pkv = 0.f, pqv = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                pkv += s_red[w][0][j];
                pqv += s_red[w][1][j];
            }
            const float u = beta * (s_v[j] - pkv);
            s_u[j] = u;
            store_io(a.out, bhv * V + j, fmaf(qk, u, pqv), a.bf16);
        }
        __syncthreads();

        // S_new = exp(g) S + k u^T, written from the registers that were read.
        const float u4[4] = {s_u[c4 * 4], s_u[c4 * 4 + 1], s_u[c4 * 4 + 2], s_u[c4 * 4 + 3]};
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int row = p * RPP + r0;
            const float e = s_eg[row], kr = s_k[row];
            float4 n;
            n.x = fmaf(kr, u4[0], e * st[p].x);
            n.y = fmaf(kr, u4[1], e * st[p].y);
            n.z = fmaf(kr, u4[2], e * st[p].z);
            n.w = fmaf(kr, u4[3], e * st[p].w);
            st_stream(&S[(p * RPP + r0) * TPR + c4], n);
        }
        __syncthreads();  // s_v / s_eg / s_u are reused by the next value head
    }
}

template <int K, int V>
hipError_t launch_kv(const DecodeArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((decode_kernel<K, V>), dim3(a.B * a.H), dim3(decode_threads<K, V>()), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
#define KDA_DEC_CASE(KK, VV) \
    if (a.K == KK && a.V == VV) return launch_kv<KK, VV>(a, stream);
    KDA_DEC_CASE(32, 32) KDA_DEC_CASE(32, 64) KDA_DEC_CASE(32, 128)
    KDA_DEC_CASE(64, 32) KDA_DEC_CASE(64, 64) KDA_DEC_CASE(64, 128)
    KDA_DEC_CASE(128, 32) KDA_DEC_CASE(128, 64) KDA_DEC_CASE(128, 128)
#undef KDA_DEC_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
