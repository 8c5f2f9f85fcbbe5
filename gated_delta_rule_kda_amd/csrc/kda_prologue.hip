// The per-token stages on either side of the chunked prefill, for gfx950:
//
//  * the prologue: the stages the host decode on the page
//    "metrale_model_weights/kimi_k3_host/kda.rs" runs in front of each
//    recurrence step (conv_update: a causal depthwise short conv over the
//    packed q | k | v channels followed by SiLU; l2norm_rows on the q and k
//    head rows; the gate of bounded_gate; a sigmoid on beta), applied to all T
//    tokens of a prefill at once;
//  * the output gate of the same page (full_rank_output_gate): an RMS norm of
//    each head row of o, gated elementwise by sigmoid(gate).
//
// Both are HBM streams.  Layout of the row kernels: a lane owns 8 consecutive
// channels of a head row (16 bytes of bf16), D/8 lanes cover a row, so a wave
// reads and writes whole rows; the L2 / RMS sums reduce over those lanes with
// cross-lane shuffles.  In the conv kernel each group of D/8 lanes walks a run
// of consecutive tokens, keeping the conv window in registers, so x is read
// once (plus KW-1 rows of history per run).

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kRowThreads = 256;
constexpr int kTile = 256;   // tokens per workgroup of the conv kernel

typedef float f32x4 __attribute__((ext_vector_type(4)));

// 8 consecutive elements of a bf16 or fp32 row.
template <bool BF16>
__device__ __forceinline__ void load8(const void *base, size_t i, float (&x)[8]) {
    if constexpr (BF16) {
        const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + i);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(w[e] << 16);
            x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    } else {
        const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + i);
        const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + i + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// (a, b) -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

template <bool BF16>
__device__ __forceinline__ void store8(void *base, size_t i, const float (&y)[8]) {
    if constexpr (BF16) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16(y[2 * e], y[2 * e + 1]);
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(base) + i) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(base) + i) = make_float4(y[0], y[1], y[2], y[3]);
        *reinterpret_cast<float4 *>(static_cast<float *>(base) + i + 4) = make_float4(y[4], y[5], y[6], y[7]);
    }
}

__device__ __forceinline__ float sigmoid_acc(float x) { return 1.0f / (1.0f + expf(-x)); }
// x * sigmoid(x) from the hardware exponential and reciprocal (a few ulp;
// 0 for x -> -inf, x for x -> +inf)
__device__ __forceinline__ float silu_fast(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// x of another lane (DPP); the 0 that stands for lanes without a source lets
// the compiler fold the move into the add that consumes it
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Sum over the LPR consecutive lanes that hold one row (LPR 4, 8 or 16; the
// groups are aligned within the 16-lane DPP rows): xor 1 and xor 2 inside
// each quad, then the mirrored quad of the half row, then the mirrored half.
template <int LPR>
__device__ __forceinline__ float row_sum(float s) {
    static_assert(LPR == 4 || LPR == 8 || LPR == 16, "row of 4, 8 or 16 lanes");
    s += dpp<0xb1>(s);                        // quad_perm [1,0,3,2]
    s += dpp<0x4e>(s);                        // quad_perm [2,3,0,1]
    if constexpr (LPR >= 8) s += dpp<0x141>(s);   // row_half_mirror
    if constexpr (LPR >= 16) s += dpp<0x140>(s);  // row_mirror
    return s;
}

// One launch covers `nseg` head rows of D channels each, starting at channel
// c_base of x: rows s < split go to out0 (head s of `heads0`), the others to
// out1 (head s - split).  Grid: (nseg, token tiles, B): workgroups that run
// together cover neighbouring head rows of the same tokens, so their 256-byte
// row pieces fill whole DRAM pages.
struct RowLaunch {
    int c_base, nseg, split, heads0, heads1;
    void *out0, *out1;
    int l2;
};

template <int D, int KW, bool BF16>
__global__ __launch_bounds__(kRowThreads) void prologue_rows_kernel(PrologueArgs a, RowLaunch L) {
    constexpr int LPR = D / 8;                       // lanes per row
    constexpr int RUNS = kRowThreads / LPR;          // token runs per workgroup
    constexpr int R = kTile / RUNS;                  // tokens per run
    static_assert(R >= 1 && kTile % RUNS == 0, "tile must split into runs");
    const int C = 2 * a.H * a.K + a.HV * a.V;
    const int lr = threadIdx.x % LPR, run = threadIdx.x / LPR;
    const int s = blockIdx.x, b = blockIdx.z;
    const int t0 = blockIdx.y * kTile + run * R;
    if (t0 >= a.T) return;
    const int c = L.c_base + s * D + lr * 8;         // first of this lane's 8 channels
    void *out = s < L.split ? L.out0 : L.out1;
    const int head = s < L.split ? s : s - L.split;
    const int heads = s < L.split ? L.heads0 : L.heads1;
    const bool conv = a.conv_w != nullptr;

    // h[i] holds token t0 - (KW - 1) + i: KW - 1 rows of history, then the R
    // rows of the run, all loaded up front (rows past the end re-read the last
    // row and are not stored), so every load of the run is in flight at once
    // and the conv reads fixed registers (no window shifts)
    constexpr int NH = KW - 1;
    float h[NH + R][8];
    float w[8][KW];
    if (conv) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int j = 0; j < KW; ++j) w[e][j] = a.conv_w[static_cast<size_t>(c + e) * KW + j];
        // tokens before 0 come from the conv registers: register KW + t holds
        // x_t for t = -1 .. -(KW - 1); in the ring layout ([KW][B][C], register
        // j in slot (conv_pos + j) % KW) that is slot (conv_pos + KW + t) % KW
#pragma unroll
        for (int i = 0; i < NH; ++i) {
            const int t = t0 - NH + i;
            if (t >= 0) {
                load8<BF16>(a.x, (static_cast<size_t>(b) * a.T + t) * C + c, h[i]);
            } else if (a.conv_ring && a.conv_state) {
                const int p = (a.conv_pos + KW + t) % KW;
                const float *col = a.conv_state + (static_cast<size_t>(p) * a.B + b) * C + c;
#pragma unroll
                for (int e = 0; e < 8; ++e) h[i][e] = col[e];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    h[i][e] = a.conv_state ? a.conv_state[(static_cast<size_t>(b) * C + c + e) * KW + KW + t] : 0.f;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
        load8<BF16>(a.x, (static_cast<size_t>(b) * a.T + min(t0 + r, a.T - 1)) * C + c, h[NH + r]);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int t = t0 + r;
        float y[8];
        if (conv) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < KW; ++j) acc = fmaf(w[e][j], h[r + j][e], acc);
                y[e] = silu_fast(acc);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = h[NH + r][e];
        }
        if (L.l2) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(y[e], y[e], ss);
            ss = row_sum<LPR>(ss);
            const float inv = __frsqrt_rn(ss + a.l2_eps);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] *= inv;
        }
        if (t < a.T) store8<BF16>(out, ((static_cast<size_t>(b) * a.T + t) * heads + head) * D + lr * 8, y);
    }
}

// g and beta, elementwise: 4 gate values per thread, then one beta per thread.
__global__ __launch_bounds__(kRowThreads) void prologue_gate_kernel(PrologueArgs a) {
    const size_t i = static_cast<size_t>(blockIdx.x) * kRowThreads + threadIdx.x;
    const size_t ng4 = static_cast<size_t>(a.B) * a.T * a.HV * a.K / 4;
    const size_t nb = static_cast<size_t>(a.B) * a.T * a.HV;
    if (i < ng4) {
        const float4 z = reinterpret_cast<const float4 *>(a.gate)[i];
        float zz[4] = {z.x, z.y, z.z, z.w}, g[4];
        const size_t e0 = i * 4;
        const int hv = static_cast<int>((e0 / a.K) % a.HV), f0 = static_cast<int>(e0 % a.K);
        if (a.gate_mode == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) g[e] = zz[e];
        } else {
            const float decay = expf(a.A_log[hv]);
            const float4 db = *reinterpret_cast<const float4 *>(a.dt_bias + hv * a.K + f0);
            const float dd[4] = {db.x, db.y, db.z, db.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float xz = zz[e] + dd[e];
                if (a.gate_mode == 1)
                    g[e] = a.lower_bound * sigmoid_acc(decay * xz);
                else   // -decay * softplus(xz), softplus in its overflow-safe form
                    g[e] = -decay * (fmaxf(xz, 0.f) + log1pf(expf(-fabsf(xz))));
            }
        }
        reinterpret_cast<float4 *>(a.g)[i] = make_float4(g[0], g[1], g[2], g[3]);
    } else if (i - ng4 < nb) {
        const size_t j = i - ng4;
        const float bl = a.beta_in[j];
        a.beta_out[j] = a.beta_is_logit ? sigmoid_acc(bl) : bl;
    }
}

// Conv registers after the last token: register j holds input T - KW + j,
// which for T < KW reaches back into the registers the call started from.
// Runs after the row kernels, which read the old registers.
__global__ __launch_bounds__(kRowThreads) void prologue_conv_state_kernel(PrologueArgs a) {
    const int C = 2 * a.H * a.K + a.HV * a.V;
    const size_t i = static_cast<size_t>(blockIdx.x) * kRowThreads + threadIdx.x;
    if (i >= static_cast<size_t>(a.B) * C) return;
    const int b = static_cast<int>(i / C), c = static_cast<int>(i % C);
    if (a.conv_ring) {
        // [KW][B][C] ring: input t goes into slot (conv_pos + t) % KW, the slot
        // of the register it replaces; only the last min(T, KW) inputs are
        // stored, and the slots of older registers that stay are not touched
        const size_t slot = static_cast<size_t>(a.B) * C;
        for (int t = a.T > a.KW ? a.T - a.KW : 0; t < a.T; ++t) {
            const float x = a.bf16 ? bf16_bits_to_float(static_cast<const uint16_t *>(a.x)[(static_cast<size_t>(b) * a.T + t) * C + c])
                                   : static_cast<const float *>(a.x)[(static_cast<size_t>(b) * a.T + t) * C + c];
            a.conv_state_out[static_cast<size_t>((a.conv_pos + t) % a.KW) * slot + i] = x;
        }
        return;
    }
    float *st = a.conv_state_out + i * a.KW;
    float nw[kMaxConvKernel];
#pragma unroll
    for (int j = 0; j < kMaxConvKernel; ++j) {
        if (j >= a.KW) break;
        const int t = a.T - a.KW + j;
        if (t >= 0)
            nw[j] = a.bf16 ? bf16_bits_to_float(static_cast<const uint16_t *>(a.x)[(static_cast<size_t>(b) * a.T + t) * C + c])
                           : static_cast<const float *>(a.x)[(static_cast<size_t>(b) * a.T + t) * C + c];
        else
            nw[j] = a.conv_state ? a.conv_state[i * a.KW + a.KW + t] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kMaxConvKernel; ++j)
        if (j < a.KW) st[j] = nw[j];
}

template <int D, bool BF16>
__global__ __launch_bounds__(kRowThreads) void output_gate_kernel(OutputGateArgs a) {
    constexpr int LPR = D / 8;
    constexpr int RPB = kRowThreads / LPR;
    const size_t row = static_cast<size_t>(blockIdx.x) * RPB + threadIdx.x / LPR;
    const int lr = threadIdx.x % LPR;
    // rows are whole per LPR-lane group, so a group is all in or all out
    if (row >= static_cast<size_t>(a.rows)) return;
    const size_t i = row * D + lr * 8;
    float o[8], gt[8];
    load8<BF16>(a.o, i, o);
    load8<BF16>(a.gate, i, gt);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(o[e], o[e], ss);
    ss = row_sum<LPR>(ss);
    const float inv = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = sigmoid_acc(gt[e]) * o[e] * inv;
    store8<BF16>(a.y, i, y);
}

template <int D, bool BF16>
hipError_t launch_rows_d(const PrologueArgs &a, const RowLaunch &L, hipStream_t stream) {
    const dim3 grid(L.nseg, (a.T + kTile - 1) / kTile, a.B);
    switch (a.conv_w ? a.KW : 1) {
#define KDA_KW(n) case n: hipLaunchKernelGGL((prologue_rows_kernel<D, n, BF16>), grid, dim3(kRowThreads), 0, stream, a, L); break;
        KDA_KW(1) KDA_KW(2) KDA_KW(3) KDA_KW(4) KDA_KW(5) KDA_KW(6) KDA_KW(7) KDA_KW(8)
#undef KDA_KW
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_rows(const PrologueArgs &a, int D, const RowLaunch &L, hipStream_t stream) {
    if (D == 32) return launch_rows_d<32, BF16>(a, L, stream);
    if (D == 64) return launch_rows_d<64, BF16>(a, L, stream);
    if (D == 128) return launch_rows_d<128, BF16>(a, L, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs &a, hipStream_t stream) {
    if (a.B == 0 || a.T == 0) return hipSuccess;
    // q and k heads (L2 norm when asked), then the v heads
    const RowLaunch qk{0, 2 * a.H, a.H, a.H, a.H, a.q, a.k, a.l2norm};
    const RowLaunch vv{2 * a.H * a.K, a.HV, a.HV, a.HV, a.HV, a.v, a.v, 0};
    hipError_t e = a.bf16 ? launch_rows<true>(a, a.K, qk, stream) : launch_rows<false>(a, a.K, qk, stream);
    if (e != hipSuccess) return e;
    e = a.bf16 ? launch_rows<true>(a, a.V, vv, stream) : launch_rows<false>(a, a.V, vv, stream);
    if (e != hipSuccess) return e;
    if (a.g) {   // the gate and beta stage (skipped when the chunk kernel forms them)
        const size_t n = static_cast<size_t>(a.B) * a.T * a.HV * (a.K / 4 + 1);
        hipLaunchKernelGGL(prologue_gate_kernel, dim3(static_cast<unsigned>((n + kRowThreads - 1) / kRowThreads)),
                           dim3(kRowThreads), 0, stream, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.conv_w && a.conv_state_out) {
        const size_t nc = static_cast<size_t>(a.B) * (2 * a.H * a.K + a.HV * a.V);
        hipLaunchKernelGGL(prologue_conv_state_kernel, dim3(static_cast<unsigned>((nc + kRowThreads - 1) / kRowThreads)),
                           dim3(kRowThreads), 0, stream, a);
        e = hipGetLastError();
    }
    return e;
}

hipError_t launch_output_gate(const OutputGateArgs &a, hipStream_t stream) {
    if (a.rows == 0) return hipSuccess;
    const int rpb = kRowThreads / (a.D / 8);
    const dim3 grid(static_cast<unsigned>((a.rows + rpb - 1) / rpb));
#define KDA_OG(d, bf)                                                                         \
    if (a.D == d && a.bf16 == bf) {                                                           \
        hipLaunchKernelGGL((output_gate_kernel<d, bf>), grid, dim3(kRowThreads), 0, stream, a); \
        return hipGetLastError();                                                             \
    }
    KDA_OG(32, true) KDA_OG(64, true) KDA_OG(128, true)
    KDA_OG(32, false) KDA_OG(64, false) KDA_OG(128, false)
#undef KDA_OG
    return hipErrorInvalidValue;
}

}  // namespace kda
