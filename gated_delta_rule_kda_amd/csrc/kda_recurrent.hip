// KDA forward as the token recurrence itself, for gfx950: the prefill path for
// gates without a lower bound.
//
// The chunked kernels factor every within-chunk decay product around a
// reference row, which needs g >= -5 (the bounded gate) to stay inside fp32.
// A gate such as -exp(A_log) * softplus(z + dt_bias) (the page
// "metrale_model_weights/kimi_k3_host/kda.rs", bounded_gate without a lower
// bound) has no such bound.  This kernel runs the four-step update of the page
// "K3/notes/sections/sec-01.tex" (section "KDA 递归核心") token by token --
//     S_dec = exp(g) (.) S,  r = v - k^T S_dec,  S = S_dec + (beta k) (x) r,
//     o = scale q^T S
// -- with the state on chip for the whole sequence, so only exp(g) of single
// tokens is ever formed and any finite g is exact.  The readout uses
// q^T S = q^T S_dec + (q.k) beta r, so q^T S_dec and k^T S_dec come from the
// same decayed state.
//
// Work decomposition: one workgroup of 4 waves per (b, hv, 16 state columns);
// lane = (column, row group), 16 row groups of K/16 rows each (runs of four
// rows spread so that a column's float4 operand reads hit every LDS bank once).
// The 16 lanes of a column are one DPP row: k^T S_dec, needed at once for the
// write, is summed by four DPP steps; the lanes' parts of q^T S are left in
// LDS and summed once per round, a whole row at a time.  Tokens are staged 16
// at a time in LDS (k, scale q, exp(g) as fp32 rows, v of the workgroup's
// columns, beta, q.k), shared by the 4 waves, and the next round's inputs are
// loaded into registers while the current round runs.  96 value heads of
// K = V = 128 give 768 workgroups, 3072 waves: three per SIMD.

#include "kda_lanes.h"

namespace kda {
namespace {

constexpr int kTC = 16;        // tokens staged per round (even)
constexpr int kRG = 16;        // lanes (row groups) per state column: 8 or 16
static_assert(kRG == 8 || kRG == 16, "a column's lanes are a half or a whole DPP row");
constexpr int kThreads = 256;  // 4 waves
constexpr int kWGCols = kThreads / kRG;   // state columns per workgroup
using namespace lanes;

// sum over the kRG lanes of one state column (a half or a whole DPP row)
__device__ __forceinline__ float col_sum(float s) { return group_sum<kRG>(s); }

// RES: the variant that writes the residuals r_t (a.aux) in place of the
// outputs, the forward half of the backward pass
template <int K, bool BF16, bool RES>
__global__ __launch_bounds__(kThreads) void recurrent_kernel(PrefillArgs a) {
    constexpr int RPL = K / kRG;                // state rows per lane
    constexpr int NP = kTC * K / 4;             // 4-element pieces of one staged [kTC][K] array
    static_assert(NP % kThreads == 0 || NP < kThreads, "pieces split over the threads");
    constexpr int NPT = NP < kThreads ? 1 : NP / kThreads;     // pieces per thread
    constexpr int NVT = kTC * kWGCols / kThreads;               // v values per thread
    static_assert(NVT * kThreads == kTC * kWGCols, "v values split over the threads");
    // q.k of a staged token: the lanes that hold its K / 4 pieces reduce by DPP
    // in groups of QKR (within one DPP row) and leave QKN partial sums
    constexpr int QKR = K / 4 < 16 ? K / 4 : 16;
    constexpr int QKN = K / 4 / QKR;
    static_assert(QKR == 8 || QKR == 16, "a token's pieces fill half or whole DPP rows");
    static_assert(QKN <= kRG, "one q.k partial per row group at most");
    __shared__ __attribute__((aligned(16))) float sK[kTC][K];
    __shared__ __attribute__((aligned(16))) float sQ[kTC][K];
    __shared__ __attribute__((aligned(16))) float sD[kTC][K];
    // Each lane's part of q^T S for every token of the round: the sum over a
    // column's kRG lanes is taken once per round, by whole rows, instead of a
    // DPP reduction per token.
    // (rows padded by 4: the per-round sums read them 16 bytes at a time
    // without bank conflicts, and the per-token writes stay conflict-free)
    __shared__ __attribute__((aligned(16))) float sW[kTC][kWGCols][kRG + 4];
    // q.k partial sums of a token at [t][0 .. QKN - 1], zeros after them: row
    // group j reads entry j, so the (q.k) beta r term of the readout lands in
    // the first QKN row groups' parts and nowhere else
    __shared__ float sQKz[kTC][kRG];
    __shared__ float sV[kTC][kWGCols], sB[kTC], sRes[RES ? kTC : 1][kWGCols];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = wave * (64 / kRG) + lane / kRG;     // this lane's column within the workgroup
    const int rg = lane % kRG;
    const int ncb = a.V / kWGCols;
    const int cb = blockIdx.x % ncb, bhv = blockIdx.x / ncb;
    const int b = bhv / a.HV, hv = bhv % a.HV;
    const int h = hv / (a.HV / a.H);
    const int c0 = cb * kWGCols;
    // The lane's state rows: runs of four, run j at row 4 kRG j + 4 rg (or
    // pairs at 2 rg when K / kRG = 2).  A float4 read of one run by the kRG
    // lanes of a column then covers 16 kRG consecutive bytes: all LDS banks
    // once, with no conflicts.
    constexpr int RUN = RPL < 4 ? RPL : 4;
    auto row_of = [&](int r) { return (r / RUN) * (RUN * kRG) + rg * RUN + r % RUN; };
    const size_t tok_b = static_cast<size_t>(b) * a.T;

    for (int i = tid; i < kTC * kRG; i += kThreads) sQKz[i / kRG][i % kRG] = 0.f;
    __syncthreads();   // before store_round puts the partial sums in

    float S[RPL];
    const size_t st_off = (static_cast<size_t>(b) * a.HV + hv) * K * a.V;
#pragma unroll
    for (int r = 0; r < RPL; ++r) S[r] = a.S0 ? a.S0[st_off + static_cast<size_t>(row_of(r)) * a.V + c0 + c] : 0.f;

    // ---- the next round's inputs (4-element pieces of q, k and g, v values
    // and one beta per thread), prefetched into registers while the current
    // round runs
    Raw4<BF16> pk[NPT], pq[NPT];
    float4 pg[NPT];
    uint32_t pv[NVT];
    float pb = 0.f;
    constexpr int ESZ = BF16 ? 2 : 4;
    // Loads go through buffer resources that cover exactly the round's valid
    // tokens: tokens past the end read 0 (k = q = 0, g = 0 so exp(g) = 1,
    // v = beta = 0: a no-op step) with no branches around the loads, so no
    // register copy has to wait for them.
    auto load_round = [&](int t0) {
        const int nv = min(kTC, a.T - t0);
        const size_t tb = tok_b + t0;
        auto span = [&](int stride, int rowlen, int esz) -> uint32_t {
            return nv > 0 ? static_cast<uint32_t>(((nv - 1) * stride + rowlen) * esz) : 0u;
        };
        const auto rk = make_rsrc(static_cast<const char *>(a.k) + ((tb * a.H + h) * K) * ESZ, span(a.H * K, K, ESZ));
        const auto rq = make_rsrc(static_cast<const char *>(a.q) + ((tb * a.H + h) * K) * ESZ, span(a.H * K, K, ESZ));
        const auto rgr = make_rsrc(a.g + (tb * a.HV + hv) * K, span(a.HV * K, K, 4));
        const auto rv = make_rsrc(static_cast<const char *>(a.v) + ((tb * a.HV + hv) * a.V + c0) * ESZ,
                                  span(a.HV * a.V, kWGCols, ESZ));
        const auto rb = make_rsrc(a.beta + tb * a.HV + hv, span(a.HV, 1, 4));
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int e = min(tid + i * kThreads, NP - 1);
            const int t = e / (K / 4), f = (e % (K / 4)) * 4;
            pk[i] = load_raw4<BF16>(rk, (t * a.H * K + f) * ESZ);
            if constexpr (!RES) pq[i] = load_raw4<BF16>(rq, (t * a.H * K + f) * ESZ);   // no readout in RES
            const auto gg = __builtin_amdgcn_raw_buffer_load_b128(rgr, (t * a.HV * K + f) * 4, 0, 0);
            pg[i] = make_float4(__uint_as_float(gg[0]), __uint_as_float(gg[1]), __uint_as_float(gg[2]),
                                __uint_as_float(gg[3]));
        }
#pragma unroll
        for (int i = 0; i < NVT; ++i) {
            const int e = tid + i * kThreads, t = e / kWGCols, cc = e % kWGCols;
            if constexpr (BF16)
                pv[i] = __builtin_amdgcn_raw_buffer_load_b16(rv, (t * a.HV * a.V + cc) * 2, 0, 0);
            else
                pv[i] = __builtin_amdgcn_raw_buffer_load_b32(rv, (t * a.HV * a.V + cc) * 4, 0, 0);
        }
        pb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, (tid & (kTC - 1)) * a.HV * 4, 0, 0));
    };
    // registers -> LDS: k, scale q, exp(g), v, beta,
    // and the partial sums of (scale q).k
    auto store_round = [&]() {
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int e = tid + i * kThreads;
            // whole groups of QKR lanes are in or out, so the DPP sum below
            // reads only lanes that took part
            if (e < NP) {
                const int t = e / (K / 4), f = (e % (K / 4)) * 4;
                const float4 k = widen<BF16>(pk[i]), g = pg[i];
                *reinterpret_cast<float4 *>(&sK[t][f]) = k;
                *reinterpret_cast<float4 *>(&sD[t][f]) = make_float4(ex2(g.x * kLog2e), ex2(g.y * kLog2e),
                                                                    ex2(g.z * kLog2e), ex2(g.w * kLog2e));
                if constexpr (!RES) {
                    const float4 q = widen<BF16>(pq[i]);
                    const float4 qs = make_float4(a.scale * q.x, a.scale * q.y, a.scale * q.z, a.scale * q.w);
                    *reinterpret_cast<float4 *>(&sQ[t][f]) = qs;
                    float s = fmaf(qs.x, k.x, fmaf(qs.y, k.y, fmaf(qs.z, k.z, qs.w * k.w)));
                    s += dpp<0xb1>(s);    // quad_perm [1,0,3,2]
                    s += dpp<0x4e>(s);    // quad_perm [2,3,0,1]
                    s += dpp<0x141>(s);   // row_half_mirror
                    if constexpr (QKR == 16) s += dpp<0x140>(s);   // row_mirror
                    if (e % QKR == 0) sQKz[t][(e % (K / 4)) / QKR] = s;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NVT; ++i) {
            const int e = tid + i * kThreads;
            sV[e / kWGCols][e % kWGCols] = BF16 ? __uint_as_float(pv[i] << 16) : __uint_as_float(pv[i]);
        }
        if (tid < kTC) sB[tid] = pb;
        // every prefetched register has now been consumed (beta only by the
        // first kTC threads): wait for all of them here, so that the
        // compiler's own bookkeeping sees no load pending into the token loop
        // (where it would otherwise wait for the round's output stores)
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    };
    // one token's operands, read from LDS a token ahead of their use so that
    // the LDS latency is off the token-to-token dependency chain
    struct Tok {
        float d[RPL], k[RPL], q[RPL];
        float v, b, qk;
    };
    auto read_tok = [&](int t, Tok &x) {
        if constexpr (RPL >= 4) {
#pragma unroll
            for (int r = 0; r < RPL; r += 4) {
                const float4 d4 = *reinterpret_cast<const float4 *>(&sD[t][row_of(r)]);
                const float4 k4 = *reinterpret_cast<const float4 *>(&sK[t][row_of(r)]);
                const float4 q4 = *reinterpret_cast<const float4 *>(&sQ[t][row_of(r)]);
                x.d[r] = d4.x; x.d[r + 1] = d4.y; x.d[r + 2] = d4.z; x.d[r + 3] = d4.w;
                x.k[r] = k4.x; x.k[r + 1] = k4.y; x.k[r + 2] = k4.z; x.k[r + 3] = k4.w;
                x.q[r] = q4.x; x.q[r + 1] = q4.y; x.q[r + 2] = q4.z; x.q[r + 3] = q4.w;
            }
        } else {
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                x.d[r] = sD[t][row_of(r)];
                x.k[r] = sK[t][row_of(r)];
                x.q[r] = sQ[t][row_of(r)];
            }
        }
        x.v = sV[t][c];
        x.b = sB[t];
        x.qk = sQKz[t][rg];
    };
    // one token: decay, k^T S_dec (summed over the column's lanes) and this
    // lane's part of q^T S_dec, the rank-1 write, and the lane's part of the
    // readout
    auto step = [&](int t, const Tok &x) {
        float p0 = 0.f, p1 = 0.f, w0 = 0.f, w1 = 0.f;
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            S[r] *= x.d[r];                                          // decay
            if (r & 1) { p1 = fmaf(x.k[r], S[r], p1); w1 = fmaf(x.q[r], S[r], w1); }
            else       { p0 = fmaf(x.k[r], S[r], p0); w0 = fmaf(x.q[r], S[r], w0); }
        }
        const float p = col_sum(p0 + p1);
        const float u = x.b * (x.v - p);                             // beta r
#pragma unroll
        for (int r = 0; r < RPL; ++r) S[r] = fmaf(x.k[r], u, S[r]);  // rank-1 write
        if constexpr (RES) {
            if (rg == 0) sRes[t][c] = x.v - p;
        } else {
            sW[t][c][rg] = fmaf(x.qk, u, w0 + w1);                   // q^T S = q^T S_dec + (q.k) beta r
        }
    };

    load_round(0);
    store_round();
    __syncthreads();
    for (int t0 = 0; t0 < a.T; t0 += kTC) {
        load_round(t0 + kTC);                              // in flight during this round
        const int nt = min(kTC, a.T - t0);
        // All kTC tokens are stepped: those past the end of the sequence were
        // staged as k = q = 0, exp(g) = 1, v = beta = 0, an exact no-op.  With
        // a fixed count the loop unrolls and the compiler can wait for each
        // token's LDS reads alone, not for the next token's as well.  Two
        // operand sets alternate (even and odd tokens), so no copies.
        Tok x0, x1;
        read_tok(0, x0);
#pragma unroll
        for (int t = 0; t < kTC; t += 2) {
            read_tok(t + 1, x1);
            step(t, x0);
            if (t + 2 < kTC) read_tok(t + 2, x0);
            step(t + 1, x1);
        }
        __syncthreads();
        // the round's outputs: each the sum of its column's kRG parts
#pragma unroll
        for (int i = 0; i < NVT; ++i) {
            const int e = tid + i * kThreads, t = e / kWGCols, cc = e % kWGCols;
            if (RES && t < nt) {
                a.aux[((tok_b + t0 + t) * a.HV + hv) * a.V + c0 + cc] = sRes[t][cc];
            } else if (t < nt) {
                float o = 0.f;
#pragma unroll
                for (int j = 0; j < kRG; j += 4) {
                    const float4 w4 = *reinterpret_cast<const float4 *>(&sW[t][cc][j]);
                    o += (w4.x + w4.y) + (w4.z + w4.w);
                }
                const size_t oi = ((tok_b + t0 + t) * a.HV + hv) * a.V + c0 + cc;
                if (BF16)
                    static_cast<uint16_t *>(a.out)[oi] = float_to_bf16_bits(o);
                else
                    static_cast<float *>(a.out)[oi] = o;
            }
        }
        // RES: the state at the start of each later slab of the backward
        // (after every snap_chunks * 32 tokens, strictly inside the sequence)
        if constexpr (RES) {
            const int te = t0 + kTC;
            if (a.snap && te < a.T && te % (a.snap_chunks * 32) == 0) {
                const int j = te / (a.snap_chunks * 32) - 1;
                float *sn = a.snap + ((static_cast<size_t>(b) * a.NS + j) * a.HV + hv) * K * a.V;
#pragma unroll
                for (int r = 0; r < RPL; ++r) sn[static_cast<size_t>(row_of(r)) * a.V + c0 + c] = S[r];
            }
        }
        if (t0 + kTC < a.T) {
            store_round();                                 // the prefetched round to LDS
            __syncthreads();
        }
    }
    if (a.ST) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) a.ST[st_off + static_cast<size_t>(row_of(r)) * a.V + c0 + c] = S[r];
    }
}

template <int K>
hipError_t launch_k(const PrefillArgs &a, hipStream_t stream) {
    const unsigned grid = static_cast<unsigned>(a.B) * a.HV * (a.V / kWGCols);
    if (a.aux) {
        if (a.bf16)
            hipLaunchKernelGGL((recurrent_kernel<K, true, true>), dim3(grid), dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((recurrent_kernel<K, false, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    } else {
        if (a.bf16)
            hipLaunchKernelGGL((recurrent_kernel<K, true, false>), dim3(grid), dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((recurrent_kernel<K, false, false>), dim3(grid), dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_recurrent(const PrefillArgs &a, hipStream_t stream) {
    if (a.B == 0 || a.T == 0) return hipSuccess;
    if (a.K == 32) return launch_k<32>(a, stream);
    if (a.K == 64) return launch_k<64>(a, stream);
    if (a.K == 128) return launch_k<128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
