// KDA chunk-parallel prefill for gfx950, fp32 inputs: one fused kernel.
// (bf16 inputs use the pipelined kernel in kda_prefill_bf16.hip.)
//
// The chunk form follows delta_recurrence on the page
// "src/tinycenn_lm/research_layers.py" (chunk-local cumulative decay, a
// unit-lower-triangular solve inside each chunk, the state carried from chunk
// to chunk), specialised to KDA (write key k, erase beta*k, value beta*v,
// readout scale on q) and re-factored for fp32/bf16 hardware:
//
//  * Exponents are only ever taken of differences of CHUNK-LOCAL cumulative
//    sums G (base 2).  The page divides k by the cumulative decay, which at
//    g >= -5 and C = 32 reaches e^160 and overflows fp32.  Here the
//    within-chunk products are factored around a reference row r (row 15):
//        A[i][j] = sum_f (x_if 2^{G_if - G_rf}) (k_jf 2^{G_rf - G_jf})
//    Each factor is at most 2^(5*16*log2 e) ~ 2^116 for g >= -5, and every
//    product that is kept (j <= i) is <= 1.  Entries above the diagonal can be
//    inf/NaN inside the MFMA accumulator and are removed with a select.
//  * By linearity the solve is applied to the M-independent right-hand sides:
//        T = (I + A_kk)^-1,  W = T (beta k Gamma),  U0 = T (beta v)
//    so the state-dependent residual is U = U0 - W M, and the triangular solve
//    never sits on the chunk-to-chunk carry.
//  * Per chunk, with M the [K x VT] state slice at the chunk start:
//        O = (s q Gamma) M + A_qk U                       (A_qk incl. diagonal)
//        M <- Gamma_last (.) M + (k 2^{G_last - G})^T U    (all factors <= 1)
//
// Work decomposition: one workgroup (4 waves) per (b, hv, V-tile of VT
// columns); the chunks of a sequence are processed in order inside it.  The
// state slice lives in MFMA accumulators (fp32) for the whole sequence.  All
// contractions use v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  Operands
// whose rounding to bf16 would cost accuracy are split into a bf16 high part
// and a bf16 low part and multiplied as hi*hi + hi*lo + lo*hi.  With bf16
// inputs the split is used where it matters (A_qk, U0, U in both of its
// products); with fp32 inputs every product is split, which keeps the fp32
// path at ~1e-5 relative error.  The triangular inverse T is formed on the
// VALU in fp32 (8x8 diagonal blocks by forward substitution, then two
// block-merge levels, T21 = -T22 A21 T11).

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kC = 32;          // chunk size
constexpr int kThreads = 256;   // 4 waves
constexpr int kRef = 15;        // reference row of the in-chunk factorisation
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __bf16 to_bf(float x) { return static_cast<__bf16>(x); }
__device__ __forceinline__ float from_bf(__bf16 x) { return static_cast<float>(x); }

__device__ __forceinline__ bf16x8 lds8(const __bf16 *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

// 8 consecutive fp32 from LDS -> bf16 fragment (hi) and its rounding residue (lo).
__device__ __forceinline__ void lds8_split(const float *p, bf16x8 &hi, bf16x8 &lo) {
    const f32x4 x0 = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 x1 = *reinterpret_cast<const f32x4 *>(p + 4);
    const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        hi[i] = to_bf(x[i]);
        lo[i] = to_bf(x[i] - from_bf(hi[i]));
    }
}

__device__ __forceinline__ float load_in(const void *p, size_t i, bool bf16) {
    return bf16 ? bf16_bits_to_float(static_cast<const uint16_t *>(p)[i])
                : static_cast<const float *>(p)[i];
}

// Shared-memory plan.  Region A holds the phase-1/2 operands; later phases of
// the same chunk reuse it for the T-merge scratch, W and the output staging.
template <int K, int VT, bool PREC>
struct Smem {
    static constexpr int LDK = K + 8;    // bf16 rows over K (16 B pad: no bank conflicts)
    static constexpr int LDC = kC + 8;   // bf16 rows over C
    static constexpr int LDF = kC + 4;   // fp32 C x C matrices
    static constexpr int LDO = VT + 4;   // fp32 output staging
    static constexpr int NS = PREC ? 2 : 1;   // hi (+ lo) copies of operands split only in PREC

    // region A (phase 1 -> 2)
    static constexpr int oLk = 0;                                   // [NS][C][LDK]
    static constexpr int oLq = oLk + NS * kC * LDK * 2;             // [2][C][LDK]
    static constexpr int oR = oLq + 2 * kC * LDK * 2;               // [2][C][LDK]
    static constexpr int endA = oR + 2 * kC * LDK * 2;
    // aliases inside region A (phase 3 -> 6)
    static constexpr int oX = 0;                                    // fp32 [C][LDF]
    static constexpr int oW = oX + kC * LDF * 4;                    // [NS][C][LDK]
    static constexpr int oO = oW + NS * kC * LDK * 2;               // fp32 [C][LDO]
    static constexpr int endAlias = oO + kC * LDO * 4;
    // persistent
    static constexpr int oKbT = (endA > endAlias ? endA : endAlias);  // [NS][K][LDC]
    static constexpr int oVbT = oKbT + NS * K * LDC * 2;            // [2][VT][LDC]
    static constexpr int oQh = oVbT + 2 * VT * LDC * 2;             // [NS][C][LDK]
    static constexpr int oKbarT = oQh + NS * kC * LDK * 2;          // [NS][K][LDC]
    static constexpr int oMT = oKbarT + NS * K * LDC * 2;           // [NS][VT][LDK]
    static constexpr int oAqk = oMT + NS * VT * LDK * 2;            // [2][C][LDC]
    static constexpr int oUT = oAqk + 2 * kC * LDC * 2;             // [2][VT][LDC]
    static constexpr int oAkk = oUT + 2 * VT * LDC * 2;             // fp32 [C][LDF]
    static constexpr int oT = oAkk + kC * LDF * 4;                  // fp32 [C][LDF]
    static constexpr int oGam = oT + kC * LDF * 4;                  // fp32 [K]
    static constexpr int oGtot = oGam + K * 4;                      // fp32 [NRG][K]
    static constexpr int NRG = kThreads / (K / 2);
    static constexpr int oBeta = oGtot + NRG * K * 4;               // fp32 [C]
    static constexpr int bytes = oBeta + kC * 4;
};

template <int K, int VT, bool BF16IO>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a) {
    constexpr bool PREC = !BF16IO;
    using L = Smem<K, VT, PREC>;
    static_assert(L::bytes <= 160 * 1024, "LDS plan exceeds 160 KB");
    constexpr int LDK = L::LDK, LDC = L::LDC, LDF = L::LDF, LDO = L::LDO;
    constexpr int NRG = L::NRG;          // row groups in phase 1
    constexpr int RPG = kC / NRG;        // rows per group
    constexpr int KT = K / 16, VTT = VT / 16;
    constexpr int NMT = KT * VTT / 4;    // state tiles per wave
    constexpr int NUT = (2 * VTT + 3) / 4;  // U/P/O tiles per wave
    static_assert(kC % NRG == 0 && (kRef + 1) % RPG == 0, "row groups must align with the reference row");
    static_assert((KT * VTT) % 4 == 0, "state tiles must split over 4 waves");

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __bf16 *sLk = reinterpret_cast<__bf16 *>(smem + L::oLk);
    __bf16 *sLq = reinterpret_cast<__bf16 *>(smem + L::oLq);
    __bf16 *sR = reinterpret_cast<__bf16 *>(smem + L::oR);
    float *sX = reinterpret_cast<float *>(smem + L::oX);
    __bf16 *sW = reinterpret_cast<__bf16 *>(smem + L::oW);
    float *sO = reinterpret_cast<float *>(smem + L::oO);
    __bf16 *sKbT = reinterpret_cast<__bf16 *>(smem + L::oKbT);
    __bf16 *sVbT = reinterpret_cast<__bf16 *>(smem + L::oVbT);
    __bf16 *sQh = reinterpret_cast<__bf16 *>(smem + L::oQh);
    __bf16 *sKbarT = reinterpret_cast<__bf16 *>(smem + L::oKbarT);
    __bf16 *sMT = reinterpret_cast<__bf16 *>(smem + L::oMT);
    __bf16 *sAqk = reinterpret_cast<__bf16 *>(smem + L::oAqk);
    __bf16 *sUT = reinterpret_cast<__bf16 *>(smem + L::oUT);
    float *sAkk = reinterpret_cast<float *>(smem + L::oAkk);
    float *sT = reinterpret_cast<float *>(smem + L::oT);
    float *sGam = reinterpret_cast<float *>(smem + L::oGam);
    float *sGtot = reinterpret_cast<float *>(smem + L::oGtot);
    float *sBeta = reinterpret_cast<float *>(smem + L::oBeta);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15;          // row (A) / column (B, D) index inside a 16x16 tile
    const int lg = lane >> 4;          // lane group: k-slice for A/B, row quad for D

    // blockIdx.x -> (b, hv, vt); the V-tiles of one head are adjacent.
    const int nvt = a.V / VT;
    const int vt_idx = blockIdx.x % nvt;
    const int bhv = blockIdx.x / nvt;
    const int b = bhv / a.HV, hv = bhv % a.HV;
    const int h = hv / (a.HV / a.H);
    const int v0 = vt_idx * VT;
    const float scale = a.scale;

    const size_t HVK = static_cast<size_t>(a.HV) * K;
    const size_t HVV = static_cast<size_t>(a.HV) * a.V;

    // ---------------------------------------------------------------- state
    f32x4 macc[NMT];
    {
        const float *S0 = a.S0 ? a.S0 + (static_cast<size_t>(b) * a.HV + hv) * K * a.V : nullptr;
#pragma unroll
        for (int s = 0; s < NMT; ++s) {
            const int t = wave * NMT + s;
            const int kt = t / VTT, vtt = t % VTT;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int f = kt * 16 + lg * 4 + r, v = vtt * 16 + lr;
                macc[s][r] = S0 ? S0[static_cast<size_t>(f) * a.V + v0 + v] : 0.f;
            }
        }
    }
    // M (bf16 hi/lo) -> sMT[v][f] for use as the B operand of W M and q^ M.
    auto store_MT = [&]() {
#pragma unroll
        for (int s = 0; s < NMT; ++s) {
            const int t = wave * NMT + s;
            const int kt = t / VTT, vtt = t % VTT;
            const int f = kt * 16 + lg * 4, v = vtt * 16 + lr;
            bf16x4 hi, lo;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hi[r] = to_bf(macc[s][r]);
                lo[r] = to_bf(macc[s][r] - from_bf(hi[r]));
            }
            *reinterpret_cast<bf16x4 *>(sMT + v * LDK + f) = hi;
            if (PREC) *reinterpret_cast<bf16x4 *>(sMT + VT * LDK + v * LDK + f) = lo;
        }
    };
    store_MT();
    // M -> dst[K][V] (the state slice of this workgroup's columns)
    auto store_state = [&](float *dst) {
#pragma unroll
        for (int s = 0; s < NMT; ++s) {
            const int t = wave * NMT + s;
            const int kt = t / VTT, vtt = t % VTT;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int f = kt * 16 + lg * 4 + r, v = vtt * 16 + lr;
                dst[static_cast<size_t>(f) * a.V + v0 + v] = macc[s][r];
            }
        }
    };
    // prefix snapshots: the state after every snap_chunks whole chunks
    int snap_left = a.snap_chunks, snap_j = 0;

    const int nchunks = (a.T + kC - 1) / kC;
    for (int ch = 0; ch < nchunks; ++ch) {
        const int t0 = ch * kC;
        const int n = min(kC, a.T - t0);

        // ============ phase 1: chunk-local cumulative decay and operands (VALU)
        {
            const int f = 2 * (tid % (K / 2));
            const int rg = tid / (K / 2);
            float gl[RPG][2], qv[RPG][2], kv[RPG][2], bv[RPG];
#pragma unroll
            for (int r = 0; r < RPG; ++r) {
                const int i = rg * RPG + r;
                if (i < n) {
                    const size_t tok = static_cast<size_t>(b) * a.T + t0 + i;
                    const size_t qi = (tok * a.H + h) * K + f;
                    const float2 gg = *reinterpret_cast<const float2 *>(a.g + tok * HVK + static_cast<size_t>(hv) * K + f);
                    gl[r][0] = gg.x * kLog2e;
                    gl[r][1] = gg.y * kLog2e;
                    qv[r][0] = load_in(a.q, qi, BF16IO) * scale;
                    qv[r][1] = load_in(a.q, qi + 1, BF16IO) * scale;
                    kv[r][0] = load_in(a.k, qi, BF16IO);
                    kv[r][1] = load_in(a.k, qi + 1, BF16IO);
                    bv[r] = a.beta[tok * a.HV + hv];
                } else {
                    gl[r][0] = gl[r][1] = qv[r][0] = qv[r][1] = kv[r][0] = kv[r][1] = bv[r] = 0.f;
                }
            }
            // local inclusive prefix over this group's rows
#pragma unroll
            for (int r = 1; r < RPG; ++r) {
                gl[r][0] += gl[r - 1][0];
                gl[r][1] += gl[r - 1][1];
            }
            sGtot[rg * K + f] = gl[RPG - 1][0];
            sGtot[rg * K + f + 1] = gl[RPG - 1][1];
            if (f == 0)
#pragma unroll
                for (int r = 0; r < RPG; ++r) sBeta[rg * RPG + r] = bv[r];
            __syncthreads();
            float off[2] = {0.f, 0.f}, Gr[2] = {0.f, 0.f}, Gl[2] = {0.f, 0.f};
#pragma unroll
            for (int g2 = 0; g2 < NRG; ++g2)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const float tot = sGtot[g2 * K + f + c];
                    if (g2 < rg) off[c] += tot;
                    if (g2 * RPG <= kRef) Gr[c] += tot;
                    Gl[c] += tot;
                }
            float pr[2], pl[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                pr[c] = exp2f(Gr[c]);           // 2^{G_r}      >= 2^-116
                pl[c] = exp2f(Gl[c] - Gr[c]);   // 2^{G_l - G_r} in [2^-116, 1]
                if (rg == 0) sGam[f + c] = exp2f(Gl[c]);
            }
            __bf16 kbT[2][RPG], kbarT[2][RPG];
            __bf16 kbTl[2][RPG], kbarTl[2][RPG];
#pragma unroll
            for (int r = 0; r < RPG; ++r) {
                const int i = rg * RPG + r;
                __bf16 lk[2], lkl[2], lqh[2], lql[2], rh[2], rl[2], qh[2], qhl[2];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const float G = off[c] + gl[r][c];
                    const float e1 = exp2f(G - Gr[c]);      // 2^{G_i - G_r}
                    const float e2 = exp2f(Gr[c] - G);      // 2^{G_r - G_i}
                    const float gam = pr[c] * e1;           // 2^{G_i} (may underflow to 0)
                    const float kb = pl[c] * e2;            // 2^{G_l - G_i} <= 1
                    const float bk = bv[r] * kv[r][c];
                    const float x_lk = bk * e1, x_lq = qv[r][c] * e1, x_r = kv[r][c] * e2;
                    const float x_kb = bk * gam, x_qh = qv[r][c] * gam, x_kbar = kv[r][c] * kb;
                    lk[c] = to_bf(x_lk);   lkl[c] = to_bf(x_lk - from_bf(lk[c]));
                    lqh[c] = to_bf(x_lq);  lql[c] = to_bf(x_lq - from_bf(lqh[c]));
                    rh[c] = to_bf(x_r);    rl[c] = to_bf(x_r - from_bf(rh[c]));
                    qh[c] = to_bf(x_qh);   qhl[c] = to_bf(x_qh - from_bf(qh[c]));
                    kbT[c][r] = to_bf(x_kb);     kbTl[c][r] = to_bf(x_kb - from_bf(kbT[c][r]));
                    kbarT[c][r] = to_bf(x_kbar); kbarTl[c][r] = to_bf(x_kbar - from_bf(kbarT[c][r]));
                }
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    sLk[i * LDK + f + c] = lk[c];
                    if (PREC) sLk[kC * LDK + i * LDK + f + c] = lkl[c];
                    sLq[i * LDK + f + c] = lqh[c];
                    sLq[kC * LDK + i * LDK + f + c] = lql[c];
                    sR[i * LDK + f + c] = rh[c];
                    sR[kC * LDK + i * LDK + f + c] = rl[c];
                    sQh[i * LDK + f + c] = qh[c];
                    if (PREC) sQh[kC * LDK + i * LDK + f + c] = qhl[c];
                }
            }
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int r = 0; r < RPG; ++r) {
                    const int i = rg * RPG + r;
                    sKbT[(f + c) * LDC + i] = kbT[c][r];
                    sKbarT[(f + c) * LDC + i] = kbarT[c][r];
                    if (PREC) {
                        sKbT[K * LDC + (f + c) * LDC + i] = kbTl[c][r];
                        sKbarT[K * LDC + (f + c) * LDC + i] = kbarTl[c][r];
                    }
                }
            // beta * v of this V-tile, transposed, split hi/lo
            for (int e = tid; e < kC * VT; e += kThreads) {
                const int v = e % VT, i = e / VT;
                float x = 0.f;
                if (i < n) {
                    const size_t tok = static_cast<size_t>(b) * a.T + t0 + i;
                    x = sBeta[i] * load_in(a.v, tok * HVV + static_cast<size_t>(hv) * a.V + v0 + v, BF16IO);
                }
                const __bf16 hi = to_bf(x);
                sVbT[v * LDC + i] = hi;
                sVbT[VT * LDC + v * LDC + i] = to_bf(x - from_bf(hi));
            }
        }
        __syncthreads();

        // ============ phase 2: A_qk (j <= i) and A_kk (j < i) on MFMA
        {
            // tiles (row tile, col tile) of the lower triangle of a 32x32 matrix
            const int rts[3] = {0, 1, 1}, cts[3] = {0, 0, 1};
            if (wave < 3) {
                const int rt = rts[wave], ct = cts[wave];
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < K / 32; ++ks) {
                    const int kk = ks * 32 + lg * 8;
                    const bf16x8 ah = lds8(sLq + (rt * 16 + lr) * LDK + kk);
                    const bf16x8 al = lds8(sLq + kC * LDK + (rt * 16 + lr) * LDK + kk);
                    const bf16x8 bh = lds8(sR + (ct * 16 + lr) * LDK + kk);
                    const bf16x8 bl = lds8(sR + kC * LDK + (ct * 16 + lr) * LDK + kk);
                    acc = mfma(ah, bh, acc);
                    acc = mfma(ah, bl, acc);
                    acc = mfma(al, bh, acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = rt * 16 + lg * 4 + r, j = ct * 16 + lr;
                    const float x = (j <= i) ? acc[r] : 0.f;
                    const __bf16 hi = to_bf(x);
                    sAqk[i * LDC + j] = hi;
                    sAqk[kC * LDC + i * LDC + j] = to_bf(x - from_bf(hi));
                }
            } else {
#pragma unroll
                for (int tt = 0; tt < 3; ++tt) {
                    const int rt = rts[tt], ct = cts[tt];
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < K / 32; ++ks) {
                        const int kk = ks * 32 + lg * 8;
                        const bf16x8 ah = lds8(sLk + (rt * 16 + lr) * LDK + kk);
                        const bf16x8 bh = lds8(sR + (ct * 16 + lr) * LDK + kk);
                        acc = mfma(ah, bh, acc);
                        if (PREC) {
                            const bf16x8 al = lds8(sLk + kC * LDK + (rt * 16 + lr) * LDK + kk);
                            const bf16x8 bl = lds8(sR + kC * LDK + (ct * 16 + lr) * LDK + kk);
                            acc = mfma(ah, bl, acc);
                            acc = mfma(al, bh, acc);
                        }
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = rt * 16 + lg * 4 + r, j = ct * 16 + lr;
                        sAkk[i * LDF + j] = (j < i) ? acc[r] : 0.f;
                    }
                }
                // the all-upper tile (rows 0-15, cols 16-31) is zero in both matrices
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = lg * 4 + r, j = 16 + lr;
                    sAkk[i * LDF + j] = 0.f;
                    sAqk[i * LDC + j] = to_bf(0.f);
                    sAqk[kC * LDC + i * LDC + j] = to_bf(0.f);
                }
            }
        }
        __syncthreads();

        // ============ phase 3: T = (I + A_kk)^-1 in fp32 on the VALU
        {
            // (a) 8x8 diagonal blocks by forward substitution; lane = (block, column).
            if (tid < 32) {
                const int d = tid >> 3, c = tid & 7, o = d * 8;
                float x[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
                    for (int j = 0; j < r; ++j) acc -= sAkk[(o + r) * LDF + o + j] * x[j];
                    x[r] = (r < c) ? 0.f : acc;
                }
#pragma unroll
                for (int r = 0; r < 8; ++r) sT[(o + r) * LDF + o + c] = x[r];
            } else {
                // zero the blocks above the diagonal: (0,1),(2,3) 8x8 and the upper 16x16
                for (int e = tid - 32; e < 128 + 256; e += kThreads - 32) {
                    int i, j;
                    if (e < 128) {
                        const int p = e >> 6, w = e & 63;
                        i = p * 16 + (w >> 3);
                        j = p * 16 + 8 + (w & 7);
                    } else {
                        const int w = e - 128;
                        i = w >> 4;
                        j = 16 + (w & 15);
                    }
                    sT[i * LDF + j] = 0.f;
                }
            }
            __syncthreads();
            // (b) 16x16 merges: T21 = -T22 A21 T11 for both 16-blocks
            if (tid < 128) {
                const int p = tid >> 6, w = tid & 63, r = w >> 3, c = w & 7, o = p * 16;
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) acc += sAkk[(o + 8 + r) * LDF + o + j] * sT[(o + j) * LDF + o + c];
                sX[(o + r) * LDF + c] = acc;
            }
            __syncthreads();
            if (tid < 128) {
                const int p = tid >> 6, w = tid & 63, r = w >> 3, c = w & 7, o = p * 16;
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) acc += sT[(o + 8 + r) * LDF + o + 8 + j] * sX[(o + j) * LDF + c];
                sT[(o + 8 + r) * LDF + o + c] = -acc;
            }
            __syncthreads();
            // (c) 32x32 merge
            {
                const int r = tid >> 4, c = tid & 15;
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < 16; ++j) acc += sAkk[(16 + r) * LDF + j] * sT[j * LDF + c];
                sX[r * LDF + c] = acc;
            }
            __syncthreads();
            {
                const int r = tid >> 4, c = tid & 15;
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < 16; ++j) acc += sT[(16 + r) * LDF + 16 + j] * sX[j * LDF + c];
                sT[(16 + r) * LDF + c] = -acc;
            }
            __syncthreads();
        }

        // ============ phase 4: W = T (beta k Gamma) -> LDS; U0 = T (beta v) -> registers
        f32x4 uacc[NUT], pacc[NUT];
        {
            // T rows of both row tiles, as split bf16 A fragments
            bf16x8 th[2], tl[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) lds8_split(sT + (rt * 16 + lr) * LDF + lg * 8, th[rt], tl[rt]);
            for (int t = wave; t < 2 * KT; t += 4) {
                const int rt = t & 1, ft = t >> 1;
                const bf16x8 bh = lds8(sKbT + (ft * 16 + lr) * LDC + lg * 8);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mfma(th[rt], bh, acc);
                if (PREC) {
                    const bf16x8 bl = lds8(sKbT + K * LDC + (ft * 16 + lr) * LDC + lg * 8);
                    acc = mfma(th[rt], bl, acc);
                    acc = mfma(tl[rt], bh, acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = rt * 16 + lg * 4 + r, ff = ft * 16 + lr;
                    const __bf16 hi = to_bf(acc[r]);
                    sW[i * LDK + ff] = hi;
                    if (PREC) sW[kC * LDK + i * LDK + ff] = to_bf(acc[r] - from_bf(hi));
                }
            }
#pragma unroll
            for (int s = 0; s < NUT; ++s) {
                const int t = wave + 4 * s;
                uacc[s] = {0.f, 0.f, 0.f, 0.f};
                if (t < 2 * VTT) {
                    const int rt = t & 1, vtt = t >> 1;
                    const bf16x8 bh = lds8(sVbT + (vtt * 16 + lr) * LDC + lg * 8);
                    const bf16x8 bl = lds8(sVbT + VT * LDC + (vtt * 16 + lr) * LDC + lg * 8);
                    uacc[s] = mfma(th[rt], bh, uacc[s]);
                    uacc[s] = mfma(th[rt], bl, uacc[s]);
                    uacc[s] = mfma(tl[rt], bh, uacc[s]);
                }
            }
        }
        __syncthreads();

        // ============ phase 5: U = U0 - W M, P = (s q Gamma) M
#pragma unroll
        for (int s = 0; s < NUT; ++s) {
            const int t = wave + 4 * s;
            pacc[s] = {0.f, 0.f, 0.f, 0.f};
            if (t < 2 * VTT) {
                const int rt = t & 1, vtt = t >> 1;
                f32x4 wm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < K / 32; ++ks) {
                    const int kk = ks * 32 + lg * 8;
                    const bf16x8 mh = lds8(sMT + (vtt * 16 + lr) * LDK + kk);
                    const bf16x8 wh = lds8(sW + (rt * 16 + lr) * LDK + kk);
                    const bf16x8 qh = lds8(sQh + (rt * 16 + lr) * LDK + kk);
                    wm = mfma(wh, mh, wm);
                    pacc[s] = mfma(qh, mh, pacc[s]);
                    if (PREC) {
                        const bf16x8 ml = lds8(sMT + VT * LDK + (vtt * 16 + lr) * LDK + kk);
                        const bf16x8 wl = lds8(sW + kC * LDK + (rt * 16 + lr) * LDK + kk);
                        const bf16x8 ql = lds8(sQh + kC * LDK + (rt * 16 + lr) * LDK + kk);
                        wm = mfma(wh, ml, wm);
                        wm = mfma(wl, mh, wm);
                        pacc[s] = mfma(qh, ml, pacc[s]);
                        pacc[s] = mfma(ql, mh, pacc[s]);
                    }
                }
                bf16x4 hi, lo;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float u = uacc[s][r] - wm[r];
                    uacc[s][r] = u;
                    hi[r] = to_bf(u);
                    lo[r] = to_bf(u - from_bf(hi[r]));
                }
                const int v = vtt * 16 + lr, i = rt * 16 + lg * 4;
                *reinterpret_cast<bf16x4 *>(sUT + v * LDC + i) = hi;
                *reinterpret_cast<bf16x4 *>(sUT + VT * LDC + v * LDC + i) = lo;
            }
        }
        __syncthreads();

        // ============ phase 6: O = P + A_qk U -> staging;  M <- Gamma_last M + kbar^T U
#pragma unroll
        for (int s = 0; s < NUT; ++s) {
            const int t = wave + 4 * s;
            if (t < 2 * VTT) {
                const int rt = t & 1, vtt = t >> 1;
                const bf16x8 ah = lds8(sAqk + (rt * 16 + lr) * LDC + lg * 8);
                const bf16x8 al = lds8(sAqk + kC * LDC + (rt * 16 + lr) * LDC + lg * 8);
                const bf16x8 uh = lds8(sUT + (vtt * 16 + lr) * LDC + lg * 8);
                const bf16x8 ul = lds8(sUT + VT * LDC + (vtt * 16 + lr) * LDC + lg * 8);
                f32x4 o = pacc[s];
                o = mfma(ah, uh, o);
                o = mfma(ah, ul, o);
                o = mfma(al, uh, o);
#pragma unroll
                for (int r = 0; r < 4; ++r) sO[(rt * 16 + lg * 4 + r) * LDO + vtt * 16 + lr] = o[r];
            }
        }
#pragma unroll
        for (int s = 0; s < NMT; ++s) {
            const int t = wave * NMT + s;
            const int kt = t / VTT, vtt = t % VTT;
#pragma unroll
            for (int r = 0; r < 4; ++r) macc[s][r] *= sGam[kt * 16 + lg * 4 + r];
            const bf16x8 kh = lds8(sKbarT + (kt * 16 + lr) * LDC + lg * 8);
            const bf16x8 uh = lds8(sUT + (vtt * 16 + lr) * LDC + lg * 8);
            const bf16x8 ul = lds8(sUT + VT * LDC + (vtt * 16 + lr) * LDC + lg * 8);
            macc[s] = mfma(kh, uh, macc[s]);
            macc[s] = mfma(kh, ul, macc[s]);
            if (PREC) {
                const bf16x8 kl = lds8(sKbarT + K * LDC + (kt * 16 + lr) * LDC + lg * 8);
                macc[s] = mfma(kl, uh, macc[s]);
            }
        }
        store_MT();
        if (a.snap && --snap_left == 0) {
            snap_left = a.snap_chunks;
            if (snap_j < a.NS)
                store_state(a.snap + ((static_cast<size_t>(b) * a.NS + snap_j) * a.HV + hv) * K * a.V);
            ++snap_j;
        }
        __syncthreads();

        // ============ output: staging -> global, 16-byte stores along V
        {
            constexpr int EPS = BF16IO ? 8 : 4;            // elements per 16-byte store
            constexpr int SEG = VT / EPS;
            for (int e = tid; e < kC * SEG; e += kThreads) {
                const int i = e / SEG, sg = e % SEG;
                if (i < n) {
                    const size_t tok = static_cast<size_t>(b) * a.T + t0 + i;
                    const size_t base = tok * HVV + static_cast<size_t>(hv) * a.V + v0 + sg * EPS;
                    const float *src = sO + i * LDO + sg * EPS;
                    if (BF16IO) {
                        bf16x8 y;
#pragma unroll
                        for (int c = 0; c < 8; ++c) y[c] = to_bf(src[c]);
                        *reinterpret_cast<bf16x8 *>(static_cast<__bf16 *>(a.out) + base) = y;
                    } else {
                        *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + base) =
                            *reinterpret_cast<const f32x4 *>(src);
                    }
                }
            }
        }
        __syncthreads();   // staging aliases the next chunk's phase-1 operands
    }

    // ---------------------------------------------------------------- final state
    if (a.ST) store_state(a.ST + (static_cast<size_t>(b) * a.HV + hv) * K * a.V);
}

template <int K, int VT, bool BF16IO>
hipError_t launch_one(const PrefillArgs &a, hipStream_t stream) {
    using L = Smem<K, VT, !BF16IO>;
    auto kern = prefill_kernel<K, VT, BF16IO>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, L::bytes);
    if (e != hipSuccess) return e;
    const int nvt = a.V / VT;
    const unsigned grid = static_cast<unsigned>(a.B) * a.HV * nvt;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), L::bytes, stream, a);
    return hipGetLastError();
}

// V-tile width: 64 columns for bf16 inputs with V >= 64, else 32.  The fp32
// path splits every operand, which needs the smaller tile to fit in LDS.
template <int K, bool BF16IO>
hipError_t launch_k(const PrefillArgs &a, hipStream_t stream) {
    if constexpr (BF16IO) {
        if (a.V >= 64) return launch_one<K, 64, BF16IO>(a, stream);
    }
    return launch_one<K, 32, BF16IO>(a, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
    if (a.B == 0 || a.T == 0) return hipSuccess;
    if (a.bf16) return launch_prefill_bf16(a, stream);
    if (a.K == 32) return launch_k<32, false>(a, stream);
    if (a.K == 64) return launch_k<64, false>(a, stream);
    if (a.K == 128) return launch_k<128, false>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
