// KDA chunk-parallel prefill for bf16 inputs on gfx950: one fused, pipelined kernel.
//
// The chunk form follows delta_recurrence on the page
// "src/tinycenn_lm/research_layers.py" (chunk-local cumulative decay, a
// unit-lower-triangular solve inside each chunk, the state carried from chunk
// to chunk), specialised to KDA (write key k, erase beta*k, value beta*v,
// readout scale on q).  Every exponent is a difference of chunk-local
// cumulative sums G (base 2) around a reference row r = 15, so no factor
// exceeds 2^116 for g >= -5 and every kept product is <= 1:
//     e1 = 2^{G_i - G_r},  e2 = 2^{G_r - G_i},  Gamma_i = 2^{G_i}
//     A_kk = diag(beta) (k e1)(k e2)^T    strictly lower  (the page's tril(., -1))
//     A_qk =            (q e1)(k e2)^T    lower incl. diagonal
//     R = diag(beta) (v - (k Gamma) M)    right-hand side of the in-chunk solve
//     U = (I + A_kk)^-1 R                 (the page's unit-lower-triangular solve)
//     O = scale ((q Gamma) M + A_qk U)
//     M <- Gamma_last (.) M + (k 2^{G_last - G})^T U
// with M the [K x V] state at the chunk start.
//
// The solve is blocked on 16 rows: U1 = T11 R1, U2 = T22 (R2 - A21 U1), where
// T11, T22 are the inverses of the two 16x16 diagonal blocks of I + A_kk
// (formed in fp32 from 8x8 forward substitutions and one block merge).  It runs
// in the carry waves on v_mfma_f32_16x16x16_bf16, whose B operand layout (four
// consecutive reduction rows per lane group) is exactly the accumulator layout
// of the previous product, so the three products chain without leaving
// registers.
//
// Organisation: one workgroup of 8 waves per (b, hv, V-tile of VT columns).
//  * State: carry wave w < VT/16 owns 16 columns of M (all K rows) in MFMA
//    accumulators for the whole sequence.  M is also used directly as the B
//    operand of the 32-deep MFMAs: the reduction index may be permuted as long
//    as both operands agree, so lane group g takes rows {4g..4g+3} of one
//    16-row tile and of the next; A operands are read from LDS in that order.
//  * Pipeline (per iteration n; four barriers):
//      A  P = (q Gamma) M for chunk n       | first operand pass of chunk n+1
//      B  second operand pass of chunk n+1 (exponentials, split operands)
//      C  A_qk, A_kk of chunk n+1 (MFMA)    | prefetch of chunk n+2
//      D  T11, T22 of chunk n+1 (one wave)  | rest of the carry of chunk n
//    Operands produced for chunk n+1 before D and read by the carry of chunk n
//    in D are double-buffered in LDS.
//  * Precision: operands whose bf16 rounding would matter are split into
//    hi + lo bf16 and multiplied as hi*hi + hi*lo + lo*hi: A_qk, (q Gamma) M,
//    the three solve products, A_qk U and k_bar^T U.  A_kk and (k Gamma) M use
//    single bf16 operands.  Emulating this policy against the fp64 oracle over
//    decay ranges from g ~ -5 to g ~ -0.05 and initial states up to
//    N(0, 0.3^2) keeps the output within 3e-3 RMS beyond its own bf16 rounding
//    and the final state within 3e-3 RMS.

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kC = 32;
constexpr int kNW = 8;
constexpr int kNT = kNW * 64;
constexpr int kRef = 15;
constexpr int kTWave = kNW - 1;    // wave that forms T11, T22
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x4 &a, const bf16x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ __bf16 bf(float x) { return static_cast<__bf16>(x); }
__device__ __forceinline__ float fl(__bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 ld8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ bf16x4 ld4(const __bf16 *p) { return *reinterpret_cast<const bf16x4 *>(p); }
__device__ __forceinline__ bf16x8 cat(const bf16x4 &a, const bf16x4 &b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// rows {p[0..3], p[16..19]} as one fragment (the permuted reduction order)
__device__ __forceinline__ bf16x8 ld4x2(const __bf16 *p) { return cat(ld4(p), ld4(p + 16)); }
__device__ __forceinline__ void split4(const f32x4 &x, bf16x4 &hi, bf16x4 &lo) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        hi[r] = bf(x[r]);
        lo[r] = bf(x[r] - fl(hi[r]));
    }
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Raw buffer resource over `bytes` bytes from `p`: out-of-range loads read 0
// and out-of-range stores are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, static_cast<int>(bytes), 0x00020000);
}
// RPG consecutive bf16 values as one LDS store (RPG in {1, 2, 4}).
template <int RPG>
__device__ __forceinline__ void store_rows(__bf16 *dst, const __bf16 (&x)[RPG]) {
    if constexpr (RPG == 4) {
        *reinterpret_cast<bf16x4 *>(dst) = bf16x4{x[0], x[1], x[2], x[3]};
    } else if constexpr (RPG == 2) {
        *reinterpret_cast<bf16x2 *>(dst) = bf16x2{x[0], x[1]};
    } else {
        dst[0] = x[0];
    }
}
// The thread index behind an empty asm: values derived from it inside the
// chunk loop are recomputed per use instead of being hoisted out of the loop
// and kept live (which would push the kernel past its register budget).
__device__ __forceinline__ int opaque_tid() {
    int t = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(t));
    return t;
}
// Workgroup barrier for LDS hand-offs.  Unlike __syncthreads() it does not
// wait for outstanding global loads, so prefetches stay in flight across it
// (each register is waited for at its first use).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Wait for this wave's LDS accesses (cross-lane exchange inside one wave).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int K>
struct Plan {
    static constexpr int LDK = K + 8;    // bf16 rows over K
    static constexpr int LDC = kC + 8;   // bf16 rows over C
    static constexpr int LDF = kC + 4;   // fp32 C x C
    static constexpr int L16 = 16 + 8;   // bf16 rows of a 16x16 block
    static constexpr int CP = K / 2;     // column pairs in the operand phase
    static constexpr int NRG = kNT / CP; // row groups
    static constexpr int RPG = kC / NRG; // rows per group
    static constexpr int B16 = 16 * L16 * 2;  // bytes of one 16x16 bf16 block
    // region A: operands of the A matrices (operand pass -> A phase); the T
    // phase reuses it for fp32 scratch
    static constexpr int oLk = 0;                                // [C][LDK]
    static constexpr int oLq = oLk + kC * LDK * 2;               // [2][C][LDK] hi, lo
    static constexpr int oR = oLq + 2 * kC * LDK * 2;            // [2][C][LDK] hi, lo
    static constexpr int endA = oR + 2 * kC * LDK * 2;
    static constexpr int oTf = 0;                                // fp32 [C][LDF]
    static constexpr int oX = oTf + kC * LDF * 4;                // fp32 [C][LDF]
    static_assert(oX + kC * LDF * 4 <= endA, "T scratch must fit in region A");
    static constexpr int oQh = endA;                             // [2][C][LDK]  q Gamma hi, lo
    static constexpr int oKGr = oQh + 2 * kC * LDK * 2;          // [2 buf][C][LDK]  k Gamma
    static constexpr int oKbarT = oKGr + 2 * kC * LDK * 2;       // [2 buf][2][K][LDC]  k_bar^T hi, lo
    static constexpr int oAqk = oKbarT + 4 * K * LDC * 2;        // [2 buf][2][C][LDC]  hi, lo
    static constexpr int oA21 = oAqk + 4 * kC * LDC * 2;         // [2 buf][2][16][L16]  -A21 hi, lo
    static constexpr int oTi = oA21 + 4 * B16;                   // [2 buf][2 blk][2][16][L16]  T11, T22
    static constexpr int oAkk = oTi + 8 * B16;                   // fp32 [C][LDF]
    static constexpr int oGam = oAkk + kC * LDF * 4;             // fp32 [2 buf][K]
    static constexpr int oBeta = oGam + 2 * K * 4;               // fp32 [2 buf][C]
    static constexpr int oGtot = oBeta + 2 * kC * 4;             // fp32 [NRG][K]
    static constexpr int bytes = oGtot + NRG * K * 4;
};

template <int K, int VT>
__global__ __launch_bounds__(kNT, 1) void prefill_bf16_kernel(PrefillArgs a) {
    using L = Plan<K>;
    static_assert(L::bytes <= 160 * 1024, "LDS plan exceeds 160 KB");
    constexpr int LDK = L::LDK, LDC = L::LDC, LDF = L::LDF, L16 = L::L16;
    constexpr int CP = L::CP, NRG = L::NRG, RPG = L::RPG;
    constexpr int KT = K / 16, KS = K / 32;
    constexpr int NCW = VT / 16;                 // carry waves
    static_assert(RPG >= 1 && (kRef + 1) % RPG == 0, "row groups must align with the reference row");
    static_assert(NCW <= kNW, "too many V columns per workgroup");

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __bf16 *sLk = reinterpret_cast<__bf16 *>(smem + L::oLk);
    __bf16 *sLq = reinterpret_cast<__bf16 *>(smem + L::oLq);
    __bf16 *sR = reinterpret_cast<__bf16 *>(smem + L::oR);
    float *sTf = reinterpret_cast<float *>(smem + L::oTf);
    float *sX = reinterpret_cast<float *>(smem + L::oX);
    __bf16 *sQh = reinterpret_cast<__bf16 *>(smem + L::oQh);
    __bf16 *sKGr = reinterpret_cast<__bf16 *>(smem + L::oKGr);
    __bf16 *sKbarT = reinterpret_cast<__bf16 *>(smem + L::oKbarT);
    __bf16 *sAqk = reinterpret_cast<__bf16 *>(smem + L::oAqk);
    __bf16 *sA21 = reinterpret_cast<__bf16 *>(smem + L::oA21);
    __bf16 *sTi = reinterpret_cast<__bf16 *>(smem + L::oTi);
    float *sAkk = reinterpret_cast<float *>(smem + L::oAkk);
    float *sGam = reinterpret_cast<float *>(smem + L::oGam);
    float *sBeta = reinterpret_cast<float *>(smem + L::oBeta);
    float *sGtot = reinterpret_cast<float *>(smem + L::oGtot);

    const int wave = threadIdx.x >> 6;
    const int nvt = a.V / VT;
    const int vt_idx = blockIdx.x % nvt;
    const int bhv = blockIdx.x / nvt;
    const int b = bhv / a.HV, hv = bhv % a.HV;
    const int h = hv / (a.HV / a.H);
    const int v0 = vt_idx * VT;
    const int T = a.T;
    const int HV = a.HV, V = a.V;
    const int NC = (T + kC - 1) / kC;
    const bool carry = wave < NCW;

    const uint16_t *qg = static_cast<const uint16_t *>(a.q);
    const uint16_t *kg = static_cast<const uint16_t *>(a.k);
    const uint16_t *vg = static_cast<const uint16_t *>(a.v);
    uint16_t *og = static_cast<uint16_t *>(a.out);

    // ---- global memory: per-chunk buffer resources (base in SGPRs, 32-bit lane
    // offsets).  A resource covers exactly the valid rows of the chunk, so rows
    // past the end of the sequence load as zero and their stores are dropped.
    const size_t tok_b = static_cast<size_t>(b) * T;
    const int g_stride = HV * K;             // elements per token
    const int qk_stride = a.H * K;
    const int v_stride = HV * V;
    auto rows_bytes = [&](int t0, int stride, int rowlen, int esz) -> uint32_t {
        const int nv = min(kC, T - t0);
        return static_cast<uint32_t>(((nv - 1) * stride + rowlen) * esz);
    };

    // operand-pass inputs of one chunk: thread owns columns f, f+1 of RPG rows
    float2 pf_g[RPG];
    uint32_t pf_q[RPG], pf_k[RPG];
    float pf_b[RPG];
    auto load_prep = [&](int ch) {
        const int tid = opaque_tid(), rg = tid / CP, f0 = 2 * (tid % CP);
        const int t0 = ch * kC;
        const size_t tb = tok_b + t0;
        const auto rgr = make_rsrc(a.g + (tb * HV + hv) * K, rows_bytes(t0, g_stride, K, 4));
        const auto rq = make_rsrc(qg + (tb * a.H + h) * K, rows_bytes(t0, qk_stride, K, 2));
        const auto rk = make_rsrc(kg + (tb * a.H + h) * K, rows_bytes(t0, qk_stride, K, 2));
        const auto rb = make_rsrc(a.beta + tb * HV + hv, rows_bytes(t0, HV, 1, 4));
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            const int i = rg * RPG + r;
            const auto gg = __builtin_amdgcn_raw_buffer_load_b64(rgr, (i * g_stride + f0) * 4, 0, 0);
            pf_g[r] = make_float2(__uint_as_float(gg[0]), __uint_as_float(gg[1]));
            pf_q[r] = __builtin_amdgcn_raw_buffer_load_b32(rq, (i * qk_stride + f0) * 2, 0, 0);
            pf_k[r] = __builtin_amdgcn_raw_buffer_load_b32(rk, (i * qk_stride + f0) * 2, 0, 0);
            pf_b[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, i * HV * 4, 0, 0));
        }
    };

    // carry inputs: v of the wave's 16 columns, rows in accumulator order
    // (row tile rt, rows 4*lg + r)
    uint16_t pf_v[2][4];
    auto load_v = [&](int ch) {
        const int lane = opaque_tid() & 63, lr = lane & 15, lg = lane >> 4;
        const int vcol = v0 + 16 * wave + lr;
        const int t0 = ch * kC;
        const auto rv = make_rsrc(vg + ((tok_b + t0) * HV + hv) * V, rows_bytes(t0, v_stride, V, 2));
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                pf_v[rt][r] = __builtin_amdgcn_raw_buffer_load_b16(
                    rv, ((rt * 16 + 4 * lg + r) * v_stride + vcol) * 2, 0, 0);
    };

    f32x4 m[KT];
    if (carry) {
        const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
        const int vcol = v0 + 16 * wave + lr;
        const float *S0 = a.S0 ? a.S0 + (static_cast<size_t>(b) * HV + hv) * K * V : nullptr;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                m[kt][r] = S0 ? S0[static_cast<size_t>(kt * 16 + lg * 4 + r) * V + vcol] : 0.f;
    }

    // registers carried from the first to the second operand pass
    float gl[RPG][2], qv[RPG][2], kv[RPG][2];

    // ======================= operand pass 1: cumulative decay within row groups
    auto op1 = [&](int buf) {
        const int tid = opaque_tid(), cp = tid % CP, rg = tid / CP, f0 = 2 * cp;
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            gl[r][0] = pf_g[r].x * kLog2e;
            gl[r][1] = pf_g[r].y * kLog2e;
            qv[r][0] = bf_lo(pf_q[r]);
            qv[r][1] = bf_hi(pf_q[r]);
            kv[r][0] = bf_lo(pf_k[r]);
            kv[r][1] = bf_hi(pf_k[r]);
        }
#pragma unroll
        for (int r = 1; r < RPG; ++r) {
            gl[r][0] += gl[r - 1][0];
            gl[r][1] += gl[r - 1][1];
        }
        *reinterpret_cast<float2 *>(sGtot + rg * K + f0) = make_float2(gl[RPG - 1][0], gl[RPG - 1][1]);
        if (cp == 0)
#pragma unroll
            for (int r = 0; r < RPG; ++r) sBeta[buf * kC + rg * RPG + r] = pf_b[r];
    };

    // ======================= operand pass 2: exponentials and MFMA operands
    auto op2 = [&](int buf) {
        const int tid = opaque_tid(), cp = tid % CP, rg = tid / CP, f0 = 2 * cp;
        float off[2] = {0.f, 0.f}, Gr[2] = {0.f, 0.f}, Gl[2] = {0.f, 0.f};
#pragma unroll
        for (int g2 = 0; g2 < NRG; ++g2) {
            const float2 t = *reinterpret_cast<const float2 *>(sGtot + g2 * K + f0);
            if (g2 < rg) { off[0] += t.x; off[1] += t.y; }
            if (g2 * RPG <= kRef) { Gr[0] += t.x; Gr[1] += t.y; }
            Gl[0] += t.x;
            Gl[1] += t.y;
        }
        float pr[2], pl[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            pr[c] = ex2(Gr[c]);             // 2^{G_r}         >= 2^-116
            pl[c] = ex2(Gl[c] - Gr[c]);     // 2^{G_last - G_r} in [2^-116, 1]
        }
        if (rg == 0)
            *reinterpret_cast<float2 *>(sGam + buf * K + f0) = make_float2(ex2(Gl[0]), ex2(Gl[1]));
        __bf16 kbT[2][RPG], kbTl[2][RPG];
        __bf16 *kgr = sKGr + buf * kC * LDK;
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            const int i = rg * RPG + r;
            bf16x2 lk, lqh, lql, rh, rl, qh, ql, kgm;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const float d = off[c] + gl[r][c] - Gr[c];
                const float e1 = ex2(d), e2 = ex2(-d);
                const float xlk = kv[r][c] * e1, xlq = qv[r][c] * e1, xr = kv[r][c] * e2;
                const float xqh = xlq * pr[c];   // q 2^{G_i}
                const float xkb = xr * pl[c];    // k 2^{G_last - G_i}
                lk[c] = bf(xlk);
                lqh[c] = bf(xlq);
                lql[c] = bf(xlq - fl(lqh[c]));
                rh[c] = bf(xr);
                rl[c] = bf(xr - fl(rh[c]));
                qh[c] = bf(xqh);
                ql[c] = bf(xqh - fl(qh[c]));
                kgm[c] = bf(xlk * pr[c]);        // k 2^{G_i}
                kbT[c][r] = bf(xkb);
                kbTl[c][r] = bf(xkb - fl(kbT[c][r]));
            }
            *reinterpret_cast<bf16x2 *>(sLk + i * LDK + f0) = lk;
            *reinterpret_cast<bf16x2 *>(sLq + i * LDK + f0) = lqh;
            *reinterpret_cast<bf16x2 *>(sLq + kC * LDK + i * LDK + f0) = lql;
            *reinterpret_cast<bf16x2 *>(sR + i * LDK + f0) = rh;
            *reinterpret_cast<bf16x2 *>(sR + kC * LDK + i * LDK + f0) = rl;
            *reinterpret_cast<bf16x2 *>(sQh + i * LDK + f0) = qh;
            *reinterpret_cast<bf16x2 *>(sQh + kC * LDK + i * LDK + f0) = ql;
            *reinterpret_cast<bf16x2 *>(kgr + i * LDK + f0) = kgm;
        }
        __bf16 *kb_buf = sKbarT + buf * 2 * K * LDC;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            store_rows<RPG>(kb_buf + (f0 + c) * LDC + rg * RPG, kbT[c]);
            store_rows<RPG>(kb_buf + K * LDC + (f0 + c) * LDC + rg * RPG, kbTl[c]);
        }
    };

    // ======================= A_qk (3-term split) and A_kk on MFMA
    auto phaseA = [&](int buf) {
        const int lane = opaque_tid() & 63, lr = lane & 15, lg = lane >> 4;
        const int rt = (wave % 3) == 0 ? 0 : 1;
        const int ct = (wave % 3) == 2 ? 1 : 0;
        __bf16 *aq = sAqk + buf * 2 * kC * LDC;
        if (wave < 3) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int kk = ks * 32 + lg * 8;
                const bf16x8 ah = ld8(sLq + (rt * 16 + lr) * LDK + kk);
                const bf16x8 al = ld8(sLq + kC * LDK + (rt * 16 + lr) * LDK + kk);
                const bf16x8 bh = ld8(sR + (ct * 16 + lr) * LDK + kk);
                const bf16x8 bl = ld8(sR + kC * LDK + (ct * 16 + lr) * LDK + kk);
                acc = mfma(ah, bh, acc);
                acc = mfma(ah, bl, acc);
                acc = mfma(al, bh, acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = rt * 16 + lg * 4 + r, j = ct * 16 + lr;
                const float x = (j <= i) ? acc[r] : 0.f;
                const __bf16 hi = bf(x);
                aq[i * LDC + j] = hi;
                aq[kC * LDC + i * LDC + j] = bf(x - fl(hi));
            }
        } else if (wave < 6) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int kk = ks * 32 + lg * 8;
                acc = mfma(ld8(sLk + (rt * 16 + lr) * LDK + kk), ld8(sR + (ct * 16 + lr) * LDK + kk), acc);
            }
            __bf16 *a21 = sA21 + buf * 2 * 16 * L16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = rt * 16 + lg * 4 + r, j = ct * 16 + lr;
                const float x = (j < i) ? sBeta[buf * kC + i] * acc[r] : 0.f;
                sAkk[i * LDF + j] = x;
                if (rt == 1 && ct == 0) {   // -A21, the off-diagonal block of the solve
                    const __bf16 hi = bf(-x);
                    a21[(lg * 4 + r) * L16 + lr] = hi;
                    a21[16 * L16 + (lg * 4 + r) * L16 + lr] = bf(-x - fl(hi));
                }
            }
        } else if (wave == 6) {
            // the all-upper tile (rows 0-15, cols 16-31) of both matrices is zero
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = lg * 4 + r, j = 16 + lr;
                sAkk[i * LDF + j] = 0.f;
                aq[i * LDC + j] = bf(0.f);
                aq[kC * LDC + i * LDC + j] = bf(0.f);
            }
        }
    };

    // ======================= T11, T22: inverses of the 16x16 diagonal blocks of
    // I + A_kk, in fp32 on one wave (8x8 forward substitutions, one merge each)
    auto phaseT = [&](int buf) {
        const int lane = opaque_tid() & 63;
        // (a) 8x8 diagonal blocks (lanes 0-31: block, column); lanes 32-63 clear
        //     the upper 8x8 block of each 16x16 block.
        if (lane < 32) {
            const int d = lane >> 3, c = lane & 7, o = d * 8;
            float x[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                float acc = (r == c) ? 1.f : 0.f;
                if (r > 0) {
                    const f32x4 a0 = *reinterpret_cast<const f32x4 *>(sAkk + (o + r) * LDF + o);
                    const f32x4 a1 = *reinterpret_cast<const f32x4 *>(sAkk + (o + r) * LDF + o + 4);
                    const float ar[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
                    for (int j = 0; j < r; ++j) acc -= ar[j] * x[j];
                }
                x[r] = (r < c) ? 0.f : acc;
            }
#pragma unroll
            for (int r = 0; r < 8; ++r) sTf[(o + r) * LDF + o + c] = x[r];
        } else {
            const int e = lane - 32;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int idx = e * 4 + qq, p = idx >> 6, w = idx & 63;
                sTf[(p * 16 + (w >> 3)) * LDF + p * 16 + 8 + (w & 7)] = 0.f;
            }
        }
        wave_lds_sync();
        // (b) merges: lower-left 8x8 block of each 16x16 block, -T22 (A21 T11)
        {
            const int p = lane >> 5, e = lane & 31, r = e >> 2, c0 = (e & 3) * 2, o = p * 16;
            float x0 = 0.f, x1 = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float av = sAkk[(o + 8 + r) * LDF + o + j];
                x0 += av * sTf[(o + j) * LDF + o + c0];
                x1 += av * sTf[(o + j) * LDF + o + c0 + 1];
            }
            sX[(o + r) * LDF + c0] = x0;
            sX[(o + r) * LDF + c0 + 1] = x1;
            wave_lds_sync();
            float y0 = 0.f, y1 = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float tv = sTf[(o + 8 + r) * LDF + o + 8 + j];
                y0 += tv * sX[(o + j) * LDF + c0];
                y1 += tv * sX[(o + j) * LDF + c0 + 1];
            }
            sTf[(o + 8 + r) * LDF + o + c0] = -y0;
            sTf[(o + 8 + r) * LDF + o + c0 + 1] = -y1;
        }
        wave_lds_sync();
        // (c) T11, T22 as split bf16: lane = (block, row, half row)
        {
            const int blk = lane >> 5, i = (lane & 31) >> 1, j0 = (lane & 1) * 8, o = blk * 16;
            bf16x8 hi, lo;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const float x = sTf[(o + i) * LDF + o + j0 + jj];
                hi[jj] = bf(x);
                lo[jj] = bf(x - fl(hi[jj]));
            }
            __bf16 *dst = sTi + ((buf * 2 + blk) * 2) * 16 * L16 + i * L16 + j0;
            *reinterpret_cast<bf16x8 *>(dst) = hi;
            *reinterpret_cast<bf16x8 *>(dst + 16 * L16) = lo;
        }
    };

    // ======================= carry: state products, solve, output, state update
    f32x4 pq[2];
    bf16x8 mh[KS];
    auto carryP = [&]() {   // P = (q Gamma) M, three terms (M split)
        const int lane = opaque_tid() & 63, lr = lane & 15, lg = lane >> 4;
        bf16x8 ml[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            bf16x4 h0, l0, h1, l1;
            split4(m[2 * s], h0, l0);
            split4(m[2 * s + 1], h1, l1);
            mh[s] = cat(h0, h1);
            ml[s] = cat(l0, l1);
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
            const int base = (rt * 16 + lr) * LDK + lg * 4;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const bf16x8 qf = ld4x2(sQh + base + s * 32);
                const bf16x8 qfl = ld4x2(sQh + kC * LDK + base + s * 32);
                p = mfma(qf, mh[s], p);
                p = mfma(qf, ml[s], p);
                p = mfma(qfl, mh[s], p);
            }
            pq[rt] = p;
        }
    };

    auto carryRest = [&](int buf, int t0) {
        const int lane = opaque_tid() & 63, lr = lane & 15, lg = lane >> 4;
        const int vcol = v0 + 16 * wave + lr;
        // R = diag(beta) (v - (k Gamma) M), accumulator layout per 16-row tile
        const __bf16 *kgr = sKGr + buf * kC * LDK;
        const float *beta = sBeta + buf * kC;
        f32x4 rr[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            const int base = (rt * 16 + lr) * LDK + lg * 4;
#pragma unroll
            for (int s = 0; s < KS; ++s) x = mfma(ld4x2(kgr + base + s * 32), mh[s], x);
            const f32x4 bt = *reinterpret_cast<const f32x4 *>(beta + rt * 16 + lg * 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float vv = __uint_as_float(static_cast<uint32_t>(pf_v[rt][r]) << 16);
                rr[rt][r] = bt[r] * (vv - x[r]);
            }
        }
        // U1 = T11 R1;  Y = R2 - A21 U1;  U2 = T22 Y   (16x16x16 MFMAs, 3 terms each)
        const __bf16 *t11 = sTi + (buf * 2 + 0) * 2 * 16 * L16 + lr * L16 + lg * 4;
        const __bf16 *t22 = sTi + (buf * 2 + 1) * 2 * 16 * L16 + lr * L16 + lg * 4;
        const __bf16 *a21 = sA21 + buf * 2 * 16 * L16 + lr * L16 + lg * 4;
        f32x4 u[2];
        bf16x4 xh, xl, uh0, ul0;
        split4(rr[0], xh, xl);
        {
            const bf16x4 th = ld4(t11), tl = ld4(t11 + 16 * L16);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mfma16(th, xh, acc);
            acc = mfma16(th, xl, acc);
            acc = mfma16(tl, xh, acc);
            u[0] = acc;
        }
        split4(u[0], uh0, ul0);
        {
            const bf16x4 ah = ld4(a21), al = ld4(a21 + 16 * L16);
            f32x4 y = rr[1];
            y = mfma16(ah, uh0, y);
            y = mfma16(ah, ul0, y);
            y = mfma16(al, uh0, y);
            split4(y, xh, xl);
            const bf16x4 th = ld4(t22), tl = ld4(t22 + 16 * L16);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mfma16(th, xh, acc);
            acc = mfma16(th, xl, acc);
            acc = mfma16(tl, xh, acc);
            u[1] = acc;
        }
        bf16x4 uh1, ul1;
        split4(u[1], uh1, ul1);
        const bf16x8 ub_hi = cat(uh0, uh1), ub_lo = cat(ul0, ul1);

        // O = scale (P + A_qk U) -> HBM
        const __bf16 *aq = sAqk + buf * 2 * kC * LDC;
        const auto ro = make_rsrc(og + ((tok_b + t0) * HV + hv) * V, rows_bytes(t0, v_stride, V, 2));
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int off = (rt * 16 + lr) * LDC + lg * 4;
            const bf16x8 ah = ld4x2(aq + off), al = ld4x2(aq + kC * LDC + off);
            f32x4 o = pq[rt];
            o = mfma(ah, ub_hi, o);
            o = mfma(ah, ub_lo, o);
            o = mfma(al, ub_hi, o);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = rt * 16 + lg * 4 + r;
                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, bf(o[r] * a.scale)), ro,
                                                      (i * v_stride + vcol) * 2, 0, 0);
            }
        }
        // M <- Gamma_last (.) M + k_bar^T U
        const __bf16 *kb_buf = sKbarT + buf * 2 * K * LDC + lr * LDC + lg * 4;
        const float *gam = sGam + buf * K + lg * 4;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            const f32x4 gm = *reinterpret_cast<const f32x4 *>(gam + kt * 16);
            const bf16x8 kf = ld4x2(kb_buf + kt * 16 * LDC);
            const bf16x8 kfl = ld4x2(kb_buf + K * LDC + kt * 16 * LDC);
            f32x4 x = m[kt] * gm;
            x = mfma(kf, ub_hi, x);
            x = mfma(kf, ub_lo, x);
            x = mfma(kfl, ub_hi, x);
            m[kt] = x;
        }
    };

    // ---------------------------------------------------------------- prologue: chunk 0
    load_prep(0);
    op1(0);
    lds_barrier();
    op2(0);
    if (NC > 1) load_prep(1);
    lds_barrier();
    phaseA(0);
    lds_barrier();
    if (wave == kTWave) phaseT(0);
    if (carry) load_v(0);
    lds_barrier();

    // ---------------------------------------------------------------- main loop
    for (int n = 0; n < NC; ++n) {
        const bool next = n + 1 < NC;
        const int cur = n & 1, nxt = cur ^ 1;
        // A: P of chunk n reads (q Gamma) before the operand pass overwrites it
        if (carry) carryP();
        if (next) op1(nxt);
        lds_barrier();
        // B
        if (next) op2(nxt);
        lds_barrier();
        // C
        if (next) {
            phaseA(nxt);
            if (n + 2 < NC) load_prep(n + 2);
        }
        lds_barrier();
        // D
        if (next && wave == kTWave) phaseT(nxt);
        if (carry) {
            carryRest(cur, n * kC);
            if (next) load_v(n + 1);
        }
        lds_barrier();
    }

    if (a.ST && carry) {
        const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
        const int vcol = v0 + 16 * wave + lr;
        float *ST = a.ST + (static_cast<size_t>(b) * HV + hv) * K * V;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ST[static_cast<size_t>(kt * 16 + lg * 4 + r) * V + vcol] = m[kt][r];
    }
}

template <int K, int VT>
hipError_t launch_kvt(const PrefillArgs &a, hipStream_t stream) {
    using L = Plan<K>;
    auto kern = prefill_bf16_kernel<K, VT>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, L::bytes);
    if (e != hipSuccess) return e;
    const unsigned grid = static_cast<unsigned>(a.B) * a.HV * (a.V / VT);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kNT), L::bytes, stream, a);
    return hipGetLastError();
}

template <int K>
hipError_t launch_k(const PrefillArgs &a, hipStream_t stream) {
    // Split V across two workgroups when there are too few (b, hv) chains to
    // occupy the GPU; each chain is otherwise one workgroup.
    const long chains = static_cast<long>(a.B) * a.HV;
    const bool split = a.V >= 64 && chains < 160;
    if (a.V == 128) return split ? launch_kvt<K, 64>(a, stream) : launch_kvt<K, 128>(a, stream);
    if (a.V == 64) return split ? launch_kvt<K, 32>(a, stream) : launch_kvt<K, 64>(a, stream);
    return launch_kvt<K, 32>(a, stream);
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs &a, hipStream_t stream) {
    if (a.K == 32) return launch_k<32>(a, stream);
    if (a.K == 64) return launch_k<64>(a, stream);
    if (a.K == 128) return launch_k<128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
