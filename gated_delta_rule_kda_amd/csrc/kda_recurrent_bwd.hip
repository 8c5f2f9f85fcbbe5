// Backward of the KDA forward, for gfx950: back-propagation through time over
// the token recurrence.
//
// The backward that the page "K3/kda/ops/reference/recurrent.py" derives in
// its module docstring (KDAFunction.backward: BPTT from t = T-1 to 0), with
// the gradient of the initial state kept.  With D = dL/dS_t carried backwards
// (D_T = dL/dS_T), per token and value head:
//     D~ = D + qs (x) dout               (qs = scale q: the readout)
//     dr = (beta k)^T D~,  dv = dr,  da = D~ r      (the rank-1 write, r its residual)
//     D  = exp(g) (.) (D~ - k (x) dr)    (the residual's read and the decay)
//     dq = scale S_t dout,  dk = beta da - S_dec dr,  dbeta = k . da
// and dS0 = D after token 0.  The per-token dg = sum over V of S_dec (.) D_dec
// needs both states at the same token; it is taken instead from the identity
//     dg_u = sum over t >= u of (qs_t (.) dqs_t - k_t (.) (S_dec,t dr_t)
//                                - k_t (.) beta_t da_t)  +  sum over V of S_T (.) dL/dS_T,
// which holds because adding eps to g_u[f] multiplies, in channel f, every
// product of a read (q_t, or k_t where it reads S_dec,t) at t >= u with a write
// (k_s as written, or S0) at s < u by e^eps, as scaling all reads at t >= u by
// e^eps and all writes at s >= u by e^-eps does; the tests compare the result
// with the oracle's direct sum (itself checked against finite differences).
//
// So the state gradient D never meets the forward state S: three passes over
// the sequence, each holding one K x 32 slice of one of them in registers --
//   1. forward (kda_recurrent.hip, residual variant): r_t and S_T;
//   2. reverse, this file: D, giving dv, dr, the partial sums of da, and dS0;
//   3. forward, this file: S again, giving the partial sums of S_t dout and
//      S_dec dr;
// then the partial sums are added (one per 32 state columns), dq and dk summed
// over the value heads of a q/k head (GQA), and dg formed by a blocked reverse
// sum over the tokens.
//
// Lanes as in the forward kernel: lane = (state column, row group), 16 row
// groups of K/16 rows (runs of four at stride 64), a column's 16 lanes one DPP
// row, so sums over K are four DPP steps.  Sums over V (da, S_t dout,
// S_dec dr: one K-vector per token) go over the four columns of a wave by the
// gfx950 lane swaps, then over the waves of the workgroup through LDS, once
// per round of staged tokens.

#include "kda_lanes.h"

namespace kda {
namespace {

using namespace lanes;

constexpr int kTA = 8;                          // tokens staged per round: reverse pass
constexpr int kTG = 8;                          // tokens staged per round: forward gradient pass
constexpr int kRG = 16;                         // lanes per state column
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kCols = kWaves * (64 / kRG);      // state columns per workgroup
static_assert(kCols == kBwdCols, "column blocks as the workspace is laid out");

// row of the lane's r-th state row (runs of four, or fewer for small K)
template <int K>
__device__ __forceinline__ int row_of(int r, int rg) {
    constexpr int RPL = K / kRG, RUN = RPL < 4 ? RPL : 4;
    return (r / RUN) * (RUN * kRG) + rg * RUN + r % RUN;
}
// RPL consecutive-in-runs values of one [K] row of LDS into registers
template <int K>
__device__ __forceinline__ void read_rows(const float *row, int rg, float (&x)[K / kRG]) {
    constexpr int RPL = K / kRG;
    if constexpr (RPL >= 4) {
#pragma unroll
        for (int r = 0; r < RPL; r += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(row + row_of<K>(r, rg));
            x[r] = v.x; x[r + 1] = v.y; x[r + 2] = v.z; x[r + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int r = 0; r < RPL; ++r) x[r] = row[row_of<K>(r, rg)];
    }
}
// The lane's RPL per-row values summed over the wave's four columns, into
// one [K] row of LDS: after across_rows_sums every lane holds some of the
// sums (RPL / 4 of them; with RPL = 2 the rows of the wave's halves hold the
// same ones, and one half writes).
template <int K>
__device__ __forceinline__ void put_column_sums(float *row, int lane, const float (&x)[K / kRG]) {
    constexpr int RPL = K / kRG;
    float sums[RPL < 4 ? 1 : RPL / 4];
    across_rows_sums<RPL>(x, sums);
    const int j = lane / kRG, rg = lane % kRG;
    if (RPL > 2 || (j & 1) == 0) {
#pragma unroll
        for (int i = 0; i < (RPL < 4 ? 1 : RPL / 4); ++i) row[row_of<K>(across_index<RPL>(i, j), rg)] = sums[i];
    }
}

// Bytes of TB tokens' rows from token t0 on, for a buffer resource: rows past
// the end of the sequence are not covered and read as 0.
template <int TB>
__device__ __forceinline__ uint32_t span_bytes(int T, int t0, int stride, int rowlen, int esz) {
    const int nv = min(TB, T - t0);
    return nv > 0 ? static_cast<uint32_t>(((nv - 1) * stride + rowlen) * esz) : 0u;
}

// ----------------------------------------------------------------------------
// Pass 2: the state gradient D, tokens in reverse.  Tokens past the end of the
// sequence (only in the first round processed) stage as q = k = 0, exp(g) = 1,
// beta = dout = r = 0: D passes through unchanged.
// (at most 128 VGPRs, so that two workgroups share a CU: 4 waves per SIMD)
template <int K, bool BF16>
__global__ __launch_bounds__(kThreads, 4) void bwd_state_kernel(BwdArgs a) {
    constexpr int RPL = K / kRG;
    constexpr int TB = kTA;
    static_assert(TB % 2 == 0, "tokens go in pairs");
    constexpr int NP = TB * K / 4;              // 4-element pieces of a [TB][K] array
    static_assert(NP <= kThreads, "one piece per thread at most");
    constexpr int NCV = TB * kCols;             // column values per round
    static_assert(NCV <= kThreads, "one column value per thread at most");
    constexpr int ESZ = BF16 ? 2 : 4;
    __shared__ __attribute__((aligned(16))) float sQ[TB][K], sK[TB][K], sA[TB][K], sD[TB][K];
    __shared__ float sDo[TB][kCols], sR[TB][kCols], sDr[TB][kCols];
    __shared__ __attribute__((aligned(16))) float sDa[TB][kWaves][K];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = wave * (64 / kRG) + lane / kRG, rg = lane % kRG;
    const int ncb = a.V / kCols;
    const int cb = blockIdx.x % ncb, bhv = blockIdx.x / ncb;
    const int b = bhv / a.HV, hv = bhv % a.HV, h = hv / (a.HV / a.H);
    const int c0 = cb * kCols;
    const size_t tok_b = static_cast<size_t>(b) * a.T;
    const size_t st_off = (static_cast<size_t>(b) * a.HV + hv) * K * a.V;
    // slab-local rows of dr and the partial sums: (b, t - t_begin, hv)
    const size_t loc_b = static_cast<size_t>(b) * a.Ls - a.t_begin;

    // D at the end of the slab: dL/dS_T for the last slab, else what the
    // slab after this one left in Dc
    const bool last_slab = a.t_end == a.T;
    const float *D_in = last_slab ? a.dST : a.Dc;
    float D[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r)
        D[r] = D_in ? D_in[st_off + static_cast<size_t>(row_of<K>(r, rg)) * a.V + c0 + c] : 0.f;

    // ---- a round's inputs, prefetched into registers
    Raw4<BF16> pq, pk;
    float4 pg;
    float pb = 0.f, pdo = 0.f, pr = 0.f;
    auto load_round = [&](int t0) {
        const size_t tb = tok_b + t0;
        const int e = min(tid, NP - 1);
        const int t = e / (K / 4), f = (e % (K / 4)) * 4;
        const auto rq = make_rsrc(static_cast<const char *>(a.q) + (tb * a.H + h) * K * ESZ,
                                  span_bytes<TB>(a.T, t0, a.H * K, K, ESZ));
        const auto rk = make_rsrc(static_cast<const char *>(a.k) + (tb * a.H + h) * K * ESZ,
                                  span_bytes<TB>(a.T, t0, a.H * K, K, ESZ));
        const auto rgr = make_rsrc(a.g + (tb * a.HV + hv) * K, span_bytes<TB>(a.T, t0, a.HV * K, K, 4));
        const auto rb = make_rsrc(a.beta + tb * a.HV + hv, span_bytes<TB>(a.T, t0, a.HV, 1, 4));
        pq = load_raw4<BF16>(rq, (t * a.H * K + f) * ESZ);
        pk = load_raw4<BF16>(rk, (t * a.H * K + f) * ESZ);
        pg = load_f4(rgr, (t * a.HV * K + f) * 4);
        pb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, t * a.HV * 4, 0, 0));
        const int ec = min(tid, NCV - 1), tc = ec / kCols, cc = ec % kCols;
        const auto rdo = make_rsrc(static_cast<const char *>(a.dout) + ((tb * a.HV + hv) * a.V + c0) * ESZ,
                                   span_bytes<TB>(a.T, t0, a.HV * a.V, kCols, ESZ));
        const auto rr = make_rsrc(a.r + (tb * a.HV + hv) * a.V + c0, span_bytes<TB>(a.T, t0, a.HV * a.V, kCols, 4));
        pdo = load1<BF16>(rdo, tc * a.HV * a.V + cc);
        pr = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rr, (tc * a.HV * a.V + cc) * 4, 0, 0));
    };
    auto store_round = [&]() {
        if (tid < NP) {
            const int t = tid / (K / 4), f = (tid % (K / 4)) * 4;
            const float4 q = widen<BF16>(pq), k = widen<BF16>(pk), g = pg;
            *reinterpret_cast<float4 *>(&sQ[t][f]) = make_float4(a.scale * q.x, a.scale * q.y, a.scale * q.z, a.scale * q.w);
            *reinterpret_cast<float4 *>(&sK[t][f]) = k;
            *reinterpret_cast<float4 *>(&sA[t][f]) = make_float4(pb * k.x, pb * k.y, pb * k.z, pb * k.w);
            *reinterpret_cast<float4 *>(&sD[t][f]) = make_float4(ex2(g.x * kLog2e), ex2(g.y * kLog2e),
                                                                 ex2(g.z * kLog2e), ex2(g.w * kLog2e));
        }
        if (tid < NCV) {
            sDo[tid / kCols][tid % kCols] = pdo;
            sR[tid / kCols][tid % kCols] = pr;
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): every prefetched register consumed
    };

    // rounds of TB tokens from the slab start (slabs start at multiples of TB)
    const int last0 = a.t_end > a.t_begin ? a.t_begin + ((a.t_end - 1 - a.t_begin) / TB) * TB : a.t_begin - TB;
    if (last0 >= a.t_begin) {
        load_round(last0);
        store_round();
    }
    __syncthreads();
    for (int t0 = last0; t0 >= a.t_begin; t0 -= TB) {
        if (t0 >= a.t_begin + TB) load_round(t0 - TB);   // in flight during this round
        // a token's operands are read a token ahead of their use (two
        // alternating register sets), off the token-to-token chain
        struct Tok {
            float q[RPL], k[RPL], a[RPL], d[RPL];
            float dout, r;
        };
        auto read_tok = [&](int t, Tok &x) {
            read_rows<K>(sQ[t], rg, x.q);
            read_rows<K>(sK[t], rg, x.k);
            read_rows<K>(sA[t], rg, x.a);
            read_rows<K>(sD[t], rg, x.d);
            x.dout = sDo[t][c];
            x.r = sR[t][c];
        };
        auto step = [&](int t, const Tok &x) {
            float Dt[RPL], s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                Dt[r] = fmaf(x.q[r], x.dout, D[r]);                  // D~ = D + qs (x) dout
                if (r & 1) s1 = fmaf(x.a[r], Dt[r], s1); else s0 = fmaf(x.a[r], Dt[r], s0);
            }
            const float dr = group_sum<kRG>(s0 + s1);               // (beta k)^T D~
            if (rg == 0) sDr[t][c] = dr;
            float pa[RPL];
#pragma unroll
            for (int r = 0; r < RPL; ++r) pa[r] = Dt[r] * x.r;
            put_column_sums<K>(sDa[t][wave], lane, pa);          // da over the wave's columns
#pragma unroll
            for (int r = 0; r < RPL; ++r) D[r] = x.d[r] * fmaf(-x.k[r], dr, Dt[r]);
        };
        Tok x0, x1;
        read_tok(TB - 1, x0);
#pragma unroll
        for (int t = TB - 1; t > 0; t -= 2) {
            read_tok(t - 1, x1);
            step(t, x0);
            if (t >= 2) read_tok(t - 2, x0);
            step(t - 1, x1);
        }
        __syncthreads();
        // the next round to LDS (its loads are waited for here, before this
        // round's stores are issued), then the round's dv, dr and da partial sums
        if (t0 >= a.t_begin + TB) store_round();
        if (tid < NCV) {
            const int t = tid / kCols, cc = tid % kCols;
            if (t0 + t < a.T) {
                store1<BF16>(a.dv, ((tok_b + t0 + t) * a.HV + hv) * a.V + c0 + cc, sDr[t][cc]);
                a.dr[((loc_b + t0 + t) * a.HV + hv) * a.V + c0 + cc] = sDr[t][cc];
            }
        }
        for (int i = tid; i < TB * K; i += kThreads) {
            const int t = i / K, kk = i % K;
            if (t0 + t < a.T) {
                float s = 0.f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) s += sDa[t][w][kk];
                a.daP[((static_cast<size_t>(cb) * a.B * a.Ls + loc_b + t0 + t) * a.HV + hv) * K + kk] = s;
            }
        }
        __syncthreads();
    }
    // D at the slab start: dS0 after the first slab, else for the slab before
    float *D_out = a.t_begin == 0 ? a.dS0 : a.Dc;
    if (D_out) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) D_out[st_off + static_cast<size_t>(row_of<K>(r, rg)) * a.V + c0 + c] = D[r];
    }
}

// ----------------------------------------------------------------------------
// Pass 3: the forward state again, tokens in order, with the partial sums of
// S_t dout (for dq) and S_dec dr (for dk).  Tokens past the end stage as
// k = 0, exp(g) = 1, v = beta = dout = dr = 0: no-ops.
template <int K, bool BF16>
__global__ __launch_bounds__(kThreads) void bwd_grad_kernel(BwdArgs a) {
    constexpr int RPL = K / kRG;
    constexpr int TB = kTG;
    static_assert(TB % 2 == 0, "tokens go in pairs");
    constexpr int NP = TB * K / 4;
    static_assert(NP <= kThreads, "one piece per thread at most");
    constexpr int NCV = TB * kCols;
    static_assert(NCV <= kThreads, "one column value per thread at most");
    constexpr int ESZ = BF16 ? 2 : 4;
    // LDS (dynamic: more than the 64 KB of static shared memory), carved as
    // sK, sD [TB][K]; sDq, sDk [TB][kWaves][K]; sV, sDo, sDr [TB][kCols]; sB [TB]
    extern __shared__ __attribute__((aligned(16))) float grad_lds[];
    float (*sK)[K] = reinterpret_cast<float (*)[K]>(grad_lds);
    float (*sD)[K] = reinterpret_cast<float (*)[K]>(grad_lds + TB * K);
    float (*sDq)[kWaves][K] = reinterpret_cast<float (*)[kWaves][K]>(grad_lds + 2 * TB * K);
    float (*sDk)[kWaves][K] = reinterpret_cast<float (*)[kWaves][K]>(grad_lds + 2 * TB * K + TB * kWaves * K);
    float *cols = grad_lds + 2 * TB * K + 2 * TB * kWaves * K;
    float (*sV)[kCols] = reinterpret_cast<float (*)[kCols]>(cols);
    float (*sDo)[kCols] = reinterpret_cast<float (*)[kCols]>(cols + TB * kCols);
    float (*sDr)[kCols] = reinterpret_cast<float (*)[kCols]>(cols + 2 * TB * kCols);
    float *sB = cols + 3 * TB * kCols;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = wave * (64 / kRG) + lane / kRG, rg = lane % kRG;
    const int ncb = a.V / kCols;
    const int cb = blockIdx.x % ncb, bhv = blockIdx.x / ncb;
    const int b = bhv / a.HV, hv = bhv % a.HV, h = hv / (a.HV / a.H);
    const int c0 = cb * kCols;
    const size_t tok_b = static_cast<size_t>(b) * a.T;
    const size_t st_off = (static_cast<size_t>(b) * a.HV + hv) * K * a.V;
    const size_t loc_b = static_cast<size_t>(b) * a.Ls - a.t_begin;

    // S at the slab start: S0 for the first slab, else the forward pass's
    // snapshot after t_begin tokens
    const float *S_in = a.t_begin == 0
                            ? (a.S0 ? a.S0 + st_off : nullptr)
                            : a.snap + ((static_cast<size_t>(b) * a.NS + a.t_begin / a.Ls - 1) * a.HV + hv) * K * a.V;
    float S[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r)
        S[r] = S_in ? S_in[static_cast<size_t>(row_of<K>(r, rg)) * a.V + c0 + c] : 0.f;

    Raw4<BF16> pk;
    float4 pg;
    float pb = 0.f, pv = 0.f, pdo = 0.f, pdr = 0.f;
    auto load_round = [&](int t0) {
        const size_t tb = tok_b + t0;
        const int e = min(tid, NP - 1);
        const int t = e / (K / 4), f = (e % (K / 4)) * 4;
        const auto rk = make_rsrc(static_cast<const char *>(a.k) + (tb * a.H + h) * K * ESZ,
                                  span_bytes<TB>(a.T, t0, a.H * K, K, ESZ));
        const auto rgr = make_rsrc(a.g + (tb * a.HV + hv) * K, span_bytes<TB>(a.T, t0, a.HV * K, K, 4));
        const auto rb = make_rsrc(a.beta + tb * a.HV + hv, span_bytes<TB>(a.T, t0, a.HV, 1, 4));
        pk = load_raw4<BF16>(rk, (t * a.H * K + f) * ESZ);
        pg = load_f4(rgr, (t * a.HV * K + f) * 4);
        pb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, (tid & (TB - 1)) * a.HV * 4, 0, 0));
        const int ec = min(tid, NCV - 1), tc = ec / kCols, cc = ec % kCols;
        const size_t cbase = (tb * a.HV + hv) * a.V + c0;
        const uint32_t cspan_d = span_bytes<TB>(a.T, t0, a.HV * a.V, kCols, ESZ);
        const uint32_t cspan_f = span_bytes<TB>(a.T, t0, a.HV * a.V, kCols, 4);
        const auto rv = make_rsrc(static_cast<const char *>(a.v) + cbase * ESZ, cspan_d);
        const auto rdo = make_rsrc(static_cast<const char *>(a.dout) + cbase * ESZ, cspan_d);
        const auto rdr = make_rsrc(a.dr + (((loc_b + t0) * a.HV + hv) * a.V + c0), cspan_f);
        pv = load1<BF16>(rv, tc * a.HV * a.V + cc);
        pdo = load1<BF16>(rdo, tc * a.HV * a.V + cc);
        pdr = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdr, (tc * a.HV * a.V + cc) * 4, 0, 0));
    };
    auto store_round = [&]() {
        if (tid < NP) {
            const int t = tid / (K / 4), f = (tid % (K / 4)) * 4;
            const float4 g = pg;
            *reinterpret_cast<float4 *>(&sK[t][f]) = widen<BF16>(pk);
            *reinterpret_cast<float4 *>(&sD[t][f]) = make_float4(ex2(g.x * kLog2e), ex2(g.y * kLog2e),
                                                                 ex2(g.z * kLog2e), ex2(g.w * kLog2e));
        }
        if (tid < NCV) {
            sV[tid / kCols][tid % kCols] = pv;
            sDo[tid / kCols][tid % kCols] = pdo;
            sDr[tid / kCols][tid % kCols] = pdr;
        }
        if (tid < TB) sB[tid] = pb;
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): every prefetched register consumed
    };

    if (a.t_end > a.t_begin) {
        load_round(a.t_begin);
        store_round();
    }
    __syncthreads();
    for (int t0 = a.t_begin; t0 < a.t_end; t0 += TB) {
        if (t0 + TB < a.t_end) load_round(t0 + TB);
        struct Tok {
            float k[RPL], d[RPL];
            float v, dout, dr, beta;
        };
        auto read_tok = [&](int t, Tok &x) {
            read_rows<K>(sK[t], rg, x.k);
            read_rows<K>(sD[t], rg, x.d);
            x.v = sV[t][c];
            x.dout = sDo[t][c];
            x.dr = sDr[t][c];
            x.beta = sB[t];
        };
        auto step = [&](int t, const Tok &x) {
            float pk_[RPL], s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                S[r] *= x.d[r];                                      // S_dec
                if (r & 1) s1 = fmaf(x.k[r], S[r], s1); else s0 = fmaf(x.k[r], S[r], s0);
            }
#pragma unroll
            for (int r = 0; r < RPL; ++r) pk_[r] = S[r] * x.dr;
            put_column_sums<K>(sDk[t][wave], lane, pk_);         // S_dec dr over the wave's columns
            const float u = x.beta * (x.v - group_sum<kRG>(s0 + s1));
            float pq_[RPL];
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                S[r] = fmaf(x.k[r], u, S[r]);                        // S_t
                pq_[r] = S[r] * x.dout;
            }
            put_column_sums<K>(sDq[t][wave], lane, pq_);         // S_t dout over the wave's columns
        };
        Tok x0, x1;
        read_tok(0, x0);
#pragma unroll
        for (int t = 0; t < TB; t += 2) {
            read_tok(t + 1, x1);
            step(t, x0);
            if (t + 2 < TB) read_tok(t + 2, x0);
            step(t + 1, x1);
        }
        __syncthreads();
        if (t0 + TB < a.t_end) store_round();             // the next round (see the reverse pass)
        for (int i = tid; i < TB * K; i += kThreads) {
            const int t = i / K, kk = i % K;
            if (t0 + t < a.T) {
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    sq += sDq[t][w][kk];
                    sk += sDk[t][w][kk];
                }
                const size_t o = ((static_cast<size_t>(cb) * a.B * a.Ls + loc_b + t0 + t) * a.HV + hv) * K + kk;
                a.dqP[o] = sq;
                a.dkrP[o] = sk;
            }
        }
        __syncthreads();
    }
}

// ----------------------------------------------------------------------------
// Partial sums over the column blocks, the per-token dg terms and dbeta, for
// the tokens of one slab.  One row (b, t, hv) of K values per K threads; the
// partial sums and e are indexed by the slab-local token, the inputs and
// outputs by the token itself.
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_sum_kernel(BwdArgs a) {
    __shared__ float sRed[256];
    const int K = a.K, rows_per_block = 256 / K;
    const int tid = threadIdx.x, rl = tid / K, kk = tid % K;
    const int len = a.t_end - a.t_begin;
    const long nrows = static_cast<long>(a.B) * len * a.HV;
    const long row = static_cast<long>(blockIdx.x) * rows_per_block + rl;
    const bool live = rl < rows_per_block && row < nrows;
    float prod = 0.f;
    long grow = 0;
    if (live) {
        const int hv = static_cast<int>(row % a.HV), h = hv / (a.HV / a.H);
        const long bt = row / a.HV;
        const int b = static_cast<int>(bt / len), lt = static_cast<int>(bt % len);
        const long tok = static_cast<long>(b) * a.T + a.t_begin + lt;     // b T + t
        grow = tok * a.HV + hv;
        const size_t plane = static_cast<size_t>(a.B) * a.Ls * a.HV * K;
        const size_t i = ((static_cast<size_t>(b) * a.Ls + lt) * a.HV + hv) * K + kk;
        float da = 0.f, dkr = 0.f, dqs = 0.f;
        for (int cb = 0; cb < a.NCB; ++cb) {
            da += a.daP[cb * plane + i];
            dkr += a.dkrP[cb * plane + i];
            dqs += a.dqP[cb * plane + i];
        }
        const size_t qi = (static_cast<size_t>(tok) * a.H + h) * K + kk;
        const float q = BF16 ? bf16_bits_to_float(static_cast<const uint16_t *>(a.q)[qi]) : static_cast<const float *>(a.q)[qi];
        const float k = BF16 ? bf16_bits_to_float(static_cast<const uint16_t *>(a.k)[qi]) : static_cast<const float *>(a.k)[qi];
        const float beta = a.beta[grow];
        a.e[i] = a.scale * q * dqs - k * (dkr + beta * da);
        prod = k * da;
        if (a.H == a.HV) {
            // one value head per q/k head: dq and dk are this row's own
            store1<BF16>(a.dq, qi, a.scale * dqs);
            store1<BF16>(a.dk, qi, beta * da - dkr);
        } else {
            // kept for the sums over the value heads of a q/k head
            a.daP[i] = da;
            a.dkrP[i] = dkr;
            a.dqP[i] = dqs;
        }
    }
    sRed[tid] = prod;
    __syncthreads();
    if (live && kk == 0) {
        float s = 0.f;
        for (int j = 0; j < K; ++j) s += sRed[rl * K + j];
        a.dbeta[grow] = s;                                         // k . da
    }
}

// With GQA (HV > H): dq = scale * sum over the q/k head's value heads of
// S_t dout; dk = sum of beta da - S_dec dr.  One element of [B,T,H,K] of the
// slab per thread.
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_qk_kernel(BwdArgs a) {
    const int len = a.t_end - a.t_begin;
    const long n = static_cast<long>(a.B) * len * a.H * a.K;
    const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    const int kk = static_cast<int>(i % a.K);
    const long th = i / a.K, bt = th / a.H;
    const int h = static_cast<int>(th % a.H), G = a.HV / a.H;
    const int b = static_cast<int>(bt / len), lt = static_cast<int>(bt % len);
    const long tok = static_cast<long>(b) * a.T + a.t_begin + lt;
    float dq = 0.f, dk = 0.f;
    for (int j = 0; j < G; ++j) {
        const int hv = h * G + j;
        const size_t ri = ((static_cast<size_t>(b) * a.Ls + lt) * a.HV + hv) * a.K + kk;
        dq += a.dqP[ri];
        dk += a.beta[tok * a.HV + hv] * a.daP[ri] - a.dkrP[ri];
    }
    const size_t o = (static_cast<size_t>(tok) * a.H + h) * a.K + kk;
    store1<BF16>(a.dq, o, a.scale * dq);
    store1<BF16>(a.dk, o, dk);
}

// Sums of e over the slab's blocks of kDgBlock tokens: bs[b, hv, block, k].
// In the last slab the same threads also start the dg carry with the
// final-state term sum over V of S_T (.) dL/dS_T (0 without dL/dS_T).
__global__ __launch_bounds__(256) void bwd_dg_blocks_kernel(BwdArgs a) {
    const int len = a.t_end - a.t_begin;
    const int nbs = (len + kDgBlock - 1) / kDgBlock;
    const long n = static_cast<long>(a.B) * a.HV * nbs * a.K;
    const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    const int kk = static_cast<int>(i % a.K);
    const long r = i / a.K;
    const int jb = static_cast<int>(r % nbs);
    const long bhv = r / nbs;
    const int b = static_cast<int>(bhv / a.HV), hv = static_cast<int>(bhv % a.HV);
    const int tb = jb * kDgBlock;
    const size_t step = static_cast<size_t>(a.HV) * a.K;
    const float *e = a.e + ((static_cast<size_t>(b) * a.Ls + tb) * a.HV + hv) * a.K + kk;
    float s = 0.f;
#pragma unroll 16
    for (int t = 0; t < kDgBlock; ++t)
        if (tb + t < len) s += e[t * step];
    // bs[b, hv, block, k]: the threads of one block read it k-contiguous
    a.bs[(bhv * a.NB + jb) * a.K + kk] = s;
    if (jb == nbs - 1 && a.t_end == a.T) {
        float c = 0.f;
        if (a.dST) {
            const float4 *st = reinterpret_cast<const float4 *>(a.ST + (static_cast<size_t>(bhv) * a.K + kk) * a.V);
            const float4 *ds = reinterpret_cast<const float4 *>(a.dST + (static_cast<size_t>(bhv) * a.K + kk) * a.V);
#pragma unroll 8
            for (int v = 0; v < a.V / 4; ++v) {
                const float4 x = st[v], y = ds[v];
                c += (x.x * y.x + x.y * y.y) + (x.z * y.z + x.w * y.w);
            }
        }
        const_cast<float *>(a.gc_in)[bhv * a.K + kk] = c;
    }
}

// dg_u = sum over V of S_T (.) dL/dS_T + sum over t >= u of e_t: each thread
// one block of tokens of one (b, hv, k) in the slab, starting from the carry
// (the final-state term and every later slab's e) and the slab's later
// blocks; the thread of the slab's first block leaves the carry for the slab
// before.
__global__ __launch_bounds__(256) void bwd_dg_kernel(BwdArgs a) {
    const int len = a.t_end - a.t_begin;
    const int nbs = (len + kDgBlock - 1) / kDgBlock;
    const long n = static_cast<long>(a.B) * a.HV * nbs * a.K;
    const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    const int kk = static_cast<int>(i % a.K);
    const long r = i / a.K;
    const int jb = static_cast<int>(r % nbs);
    const long bhv = r / nbs;
    const int b = static_cast<int>(bhv / a.HV), hv = static_cast<int>(bhv % a.HV);
    float acc = a.gc_in[bhv * a.K + kk];
    for (int j = nbs - 1; j > jb; --j) acc += a.bs[(bhv * a.NB + j) * a.K + kk];
    const int tb = jb * kDgBlock;
    const size_t step = static_cast<size_t>(a.HV) * a.K;
    const size_t lbase = ((static_cast<size_t>(b) * a.Ls + tb) * a.HV + hv) * a.K + kk;
    const size_t gbase = ((static_cast<size_t>(b) * a.T + a.t_begin + tb) * a.HV + hv) * a.K + kk;
#pragma unroll 16
    for (int t = kDgBlock - 1; t >= 0; --t) {
        if (tb + t < len) {
            acc += a.e[lbase + t * step];
            a.dg[gbase + t * step] = acc;
        }
    }
    if (jb == 0) a.gc_out[bhv * a.K + kk] = acc;
}

template <int K>
hipError_t launch_passes(const BwdArgs &a, hipStream_t stream) {
    const unsigned grid = static_cast<unsigned>(a.B) * a.HV * (a.V / kCols);
    if (a.bf16)
        hipLaunchKernelGGL((bwd_state_kernel<K, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((bwd_state_kernel<K, false>), dim3(grid), dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.T == 0) return e;
    // the forward gradient pass's LDS (see bwd_grad_kernel)
    constexpr int grad_lds = (2 * kTG * K + 2 * kTG * kWaves * K + 3 * kTG * kCols + kTG) * 4;
    const void *kern = a.bf16 ? reinterpret_cast<const void *>(bwd_grad_kernel<K, true>)
                              : reinterpret_cast<const void *>(bwd_grad_kernel<K, false>);
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, grad_lds);
    if (e != hipSuccess) return e;
    if (a.bf16)
        hipLaunchKernelGGL((bwd_grad_kernel<K, true>), dim3(grid), dim3(kThreads), grad_lds, stream, a);
    else
        hipLaunchKernelGGL((bwd_grad_kernel<K, false>), dim3(grid), dim3(kThreads), grad_lds, stream, a);
    return hipGetLastError();
}

unsigned blocks_of(long n, int per) { return static_cast<unsigned>((n + per - 1) / per); }

// One slab: the reverse and forward gradient passes over its tokens, then
// its reductions.
hipError_t launch_slab(const BwdArgs &a, hipStream_t stream) {
    hipError_t e = a.K == 32 ? launch_passes<32>(a, stream)
                 : a.K == 64 ? launch_passes<64>(a, stream)
                 : a.K == 128 ? launch_passes<128>(a, stream) : hipErrorInvalidValue;
    if (e != hipSuccess || a.T == 0) return e;
    const int len = a.t_end - a.t_begin;
    const long rows = static_cast<long>(a.B) * len * a.HV;
    const unsigned qk_blocks = blocks_of(static_cast<long>(a.B) * len * a.H * a.K, 256);
    if (a.bf16) {
        hipLaunchKernelGGL(bwd_sum_kernel<true>, dim3(blocks_of(rows, 256 / a.K)), dim3(256), 0, stream, a);
        if (a.H != a.HV) hipLaunchKernelGGL(bwd_qk_kernel<true>, dim3(qk_blocks), dim3(256), 0, stream, a);
    } else {
        hipLaunchKernelGGL(bwd_sum_kernel<false>, dim3(blocks_of(rows, 256 / a.K)), dim3(256), 0, stream, a);
        if (a.H != a.HV) hipLaunchKernelGGL(bwd_qk_kernel<false>, dim3(qk_blocks), dim3(256), 0, stream, a);
    }
    const long nb = static_cast<long>(a.B) * a.HV * ((len + kDgBlock - 1) / kDgBlock) * a.K;
    hipLaunchKernelGGL(bwd_dg_blocks_kernel, dim3(blocks_of(nb, 256)), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(bwd_dg_kernel, dim3(blocks_of(nb, 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BwdArgs &a0, hipStream_t stream) {
    if (a0.B == 0) return hipSuccess;
    if (a0.T == 0) {   // only dS0 = dL/dS_T (or zeros): the reverse pass over no tokens
        BwdArgs a = a0;
        a.t_begin = a.t_end = 0;
        return a.K == 32 ? launch_passes<32>(a, stream)
             : a.K == 64 ? launch_passes<64>(a, stream)
             : a.K == 128 ? launch_passes<128>(a, stream) : hipErrorInvalidValue;
    }
    // slabs of Ls tokens, the last one first; the dg carry alternates between
    // the two halves of gc (gc_out of one slab is gc_in of the next)
    const int ns = (a0.T + a0.Ls - 1) / a0.Ls;
    float *gc[2] = {const_cast<float *>(a0.gc_in), a0.gc_out};
    for (int s = ns - 1, j = 0; s >= 0; --s, ++j) {
        BwdArgs a = a0;
        a.t_begin = s * a0.Ls;
        a.t_end = min(a0.T, a.t_begin + a0.Ls);
        a.gc_in = gc[j & 1];
        a.gc_out = gc[(j + 1) & 1];
        const hipError_t e = launch_slab(a, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kda
