// KDA chunked backward for bf16 inputs on gfx950 (kda_chunk_bwd).
//
// The gradients of the chunk form of the bf16 prefill (kda_prefill_bf16.hip:
// chunk-local cumulative decay G in base 2 around reference row r = 15, the
// unit-lower-triangular in-chunk solve, the carried state M), derived chunk by
// chunk in reverse.  With, per chunk,
//     e1 = 2^{G_i - G_r}, e2 = 2^{G_r - G_i}, Gamma_i = 2^{G_i},
//     Lambda'_i = 2^{G_last - G_i}, Pq = q e1, Pk = k e1, Rk = k e2,
//     A_qk = L(Pq Rk^T), A_kk = diag(beta) SL(Pk Rk^T), T = (I + A_kk)^-1,
//     W = v - (k Gamma) M, U = T diag(beta) W,
//     O = s ((q Gamma) M + A_qk U),  M' = Gamma_last (.) M + (k Lambda')^T U,
// and dM' = dL/dM' entering from the chunk after (dL/dS_T for the last):
//     dU = (k Lambda') dM' + s A_qk^T dO
//     dR = T^T dU                      (blocked: dR2 = T22^T dU2,
//                                       dR1 = T11^T (dU1 - A21^T dR2))
//     dM = Gamma_last (.) dM' + s (q Gamma)^T dO - (beta k Gamma)^T dR
//     dA_qk = s L(dO U^T),  dA_kk = -SL(dR U^T)
//     dq       = s Gamma (.) (dO M^T) + e1 (.) (dA_qk Rk)
//     dk_read  = beta (.) (-Gamma (.) (dR M^T) + e1 (.) (dA_kk Rk))
//     dk_write = Lambda' (.) (U dM'^T) + e2 (.) (dA_qk^T Pq + (beta dA_kk)^T Pk)
//     dk = dk_read + dk_write,  dv = beta dR,
//     dbeta = rowsum(dR (.) W) + rowsum(dA_kk (.) SL(Pk Rk^T)), where
//     rowsum(dR (.) W) = rowsum(dR (.) v) - rowsum((k Gamma) (.) dR M^T)
// and dg from the same identity the token-recurrent backward uses: a change
// of g_u scales every read at t >= u against every write before u, so
//     dg_u = sum_{t >= u} (q (.) dq + k (.) dk_read - k (.) dk_write)_t
//            + sum_V S_T (.) dL/dS_T.
// This is the backward of KDAFunction on the "K3/kda/ops/reference/recurrent.py"
// page restated for the chunk form of delta_recurrence on the
// "src/tinycenn_lm/research_layers.py" page (its forward quantities as the
// prefill computes them).
//
// Passes, one slab of Ls tokens at a time from the last (the state gradient
// and the dg sum carried between slabs):
//  0. a forward pass over the whole sequence keeps S_T and the states at the
//     slab starts; per slab, the forward kernel's backward instantiation runs
//     the slab again from its start state, keeping the state at every chunk
//     start and U (kda_prefill_bf16.hip);
//  1. prep (chunk-parallel): every chunk's operands of the reverse chain --
//     k Lambda', s (q Gamma)^T, -(beta k Gamma)^T, s A_qk^T, T11^T, T22^T,
//     -A21^T, Gamma_last -- as the exact LDS image the chain kernel reads
//     (bf16 hi/lo pairs);
//  2. chain (one workgroup per (b, hv, V tile), chunks in reverse): dU, dR,
//     the dM update, on the matrix cores; keeps dR and every chunk's dM';
//  3. grad (chunk-parallel, one workgroup per (b, q/k head, chunk), summing
//     over the head's value heads): the rest of the formulas above;
//  4. dg: a reverse sum over the chunks' sums of the dg terms (which the
//     grad pass leaves), then over each chunk's tokens.
// The chain's products take both operands as bf16 pairs x = hi + lo and sum
// hi.hi + hi.lo + lo.hi (two terms where dO, exact in bf16, is one operand),
// the forward's policy; the image holds its operands that way, and dM' and dR
// are split from their fp32 accumulators each chunk.  Every other product is
// an fp32 MFMA (v_mfma_f32_16x16x4_f32) on fp32 operands.
//
// fp32 16x16x4 MFMA lane layout (lane l, x = l % 16, kq = l / 16): A[x][kq],
// B[kq][x]; the result holds D[4 kq + j][x] in element j.  Every product
// D[m][n] = sum_k X[m][k] Y[n][k] below reads, for reduction block k0, the
// float4 X[m0 + x][k0 + 4 kq .. + 3] and Y[n0 + x][k0 + 4 kq .. + 3] and issues
// four MFMAs (element j of both): the reduction index inside a block of 16 is
// permuted (step j takes k0 + 4 kq + j), which both operands share.  A result
// used as the B operand of the next product (dm, dU, dR) is already in that
// order: its element j is row 4 kq + j.

#include <algorithm>
#include <mutex>

#include "kda_internal.h"
#include "kda_lanes.h"

namespace kda {
namespace {

using lanes::ex2;
using lanes::group_sum;
using lanes::kLog2e;
using lanes::make_rsrc;

constexpr int kC = 32;     // tokens per chunk
constexpr int kR = 15;     // reference row
constexpr int kThr = 512;  // threads per workgroup of the prep and chain kernels (8 waves)
constexpr int kThrG = 512;  // of the grad kernel

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma4(float a, float b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// bf16 products of the reverse chain: 16x16 tiles over 32 and 16 reduction
// indices (A: row = lane % 16, 8 or 4 consecutive reduction indices of lane
// group lane / 16; B: the same indices of column lane % 16)
__device__ __forceinline__ f32x4 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x4 &a, const bf16x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
}
__device__ __forceinline__ bf16x8 ld8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ bf16x4 ld4h(const __bf16 *p) { return *reinterpret_cast<const bf16x4 *>(p); }
__device__ __forceinline__ bf16x8 cat(const bf16x4 &a, const bf16x4 &b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// x = hi + lo with hi = bf16(x) (round to nearest even) and lo = bf16(x - hi)
__device__ __forceinline__ void split1(float x, __bf16 &hi, __bf16 &lo) {
    hi = static_cast<__bf16>(x);
    lo = static_cast<__bf16>(x - static_cast<float>(hi));
}
__device__ __forceinline__ void split4(const f32x4 &x, bf16x4 &hi, bf16x4 &lo) {
    const bf16x2 h0 = __builtin_convertvector(f32x2{x[0], x[1]}, bf16x2);
    const bf16x2 h1 = __builtin_convertvector(f32x2{x[2], x[3]}, bf16x2);
    hi = bf16x4{h0[0], h0[1], h1[0], h1[1]};
    const bf16x2 l0 = __builtin_convertvector(
        f32x2{x[0] - static_cast<float>(h0[0]), x[1] - static_cast<float>(h0[1])}, bf16x2);
    const bf16x2 l1 = __builtin_convertvector(
        f32x2{x[2] - static_cast<float>(h1[0]), x[3] - static_cast<float>(h1[1])}, bf16x2);
    lo = bf16x4{l0[0], l0[1], l1[0], l1[1]};
}
// Position of reduction index x within its block of 32: 16 h + 4 g + e goes to
// 8 g + 4 h + e, so that lane group g's 8 indices (rows 4g..4g+3 of two
// 16-row accumulator tiles) are contiguous.
__device__ __forceinline__ int perm32(int x) {
    return (x & ~31) | (((x >> 2) & 3) << 3) | (((x >> 4) & 1) << 2) | (x & 3);
}
__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }
// x of lane 4 (lane / 4) + p (DPP quad broadcast)
template <int P>
__device__ __forceinline__ float quad_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), P | (P << 2) | (P << 4) | (P << 6), 0xf, 0xf, false));
}
__device__ __forceinline__ float quad_bcast(float x, int p) {
    switch (p) {
    case 0: return quad_bcast<0>(x);
    case 1: return quad_bcast<1>(x);
    case 2: return quad_bcast<2>(x);
    default: return quad_bcast<3>(x);
    }
}
// a 16x16 tile product over reduction length L (a multiple of 16):
// D[m][n] += sum_k X[m][k] Y[n][k], X and Y row pointers of this lane's row x
template <int L>
__device__ __forceinline__ void tile_nt(const float *xrow, const float *yrow, int kq, f32x4 &acc) {
#pragma unroll
    for (int k0 = 0; k0 < L; k0 += 16) {
        const f32x4 xa = ld4(xrow + k0 + 4 * kq), yb = ld4(yrow + k0 + 4 * kq);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mma4(xa[j], yb[j], acc);
    }
}

// ---------------------------------------------------------------- operand image
// One chunk's operands of the reverse chain, as the chain kernel's LDS holds
// them: bf16 hi/lo pairs (x = hi + lo), offsets and pitches in bf16 elements.
// The reduction index of each product (K of k Lambda', the chunk's tokens of
// the others) is stored in perm32 order within each block of 32, so that one
// 16-byte read gives a lane its 8 indices; Gamma_last is fp32.
template <int K>
struct Img {
    static constexpr int LK = K + 8;     // [C][K] rows
    static constexpr int LC = kC + 8;    // [K][C], [C][C] rows
    static constexpr int L16 = 20;       // [16][16] rows
    static constexpr int oKb = 0;                      // [2][C][LK]  k Lambda' (hi, lo)
    static constexpr int oA1 = oKb + 2 * kC * LK;      // [2][K][LC]  s (q Gamma)^T
    static constexpr int oA2 = oA1 + 2 * K * LC;       // [2][K][LC]  -(beta k Gamma)^T
    static constexpr int oAq = oA2 + 2 * K * LC;       // [2][C][LC]  s A_qk^T
    static constexpr int oT1 = oAq + 2 * kC * LC;      // [2][16][L16] T11^T (natural order)
    static constexpr int oT2 = oT1 + 2 * 16 * L16;     // [2][16][L16] T22^T
    static constexpr int oNA = oT2 + 2 * 16 * L16;     // [2][16][L16] -A21^T
    static constexpr int oGl = (oNA + 2 * 16 * L16 + 7) / 8 * 8;   // [K] Gamma_last, fp32
    static constexpr int used = oGl + 2 * K;           // bf16 elements
    // floats per chunk in HBM and per LDS buffer: whole rounds of the chain
    // kernel's copy (256 lanes x 16 bytes)
    static constexpr int floats = (used / 2 + 1023) / 1024 * 1024;
    static_assert(oKb % 8 == 0 && oA1 % 8 == 0 && oA2 % 8 == 0 && oAq % 8 == 0 && oT1 % 4 == 0,
                  "16-byte fragment reads");
};

// Per-slab arguments of the three kernels.
struct SlabArgs {
    ChunkBwdArgs a;
    int t_begin, len, NCs;      // tokens [t_begin, t_begin + len), NCs chunks
    const float *Sstart;        // state at the slab start for (b, hv): Sstart + b * s_bstride + hv K V; null = 0
    long long s_bstride;
    const float *dm_in;         // [B,HV,K,V] dL/dS at the slab end, or null (0)
    float *dm_out;              // [B,HV,K,V] dL/dS at the slab start, or null
};

// Base-2 cumulative sums of g over the chunk (per column), for rows < nv
// (rows past the end get g = 0): sG[i][c] = log2(e) sum_{t <= i} g_t[c].
// All 512 threads: column c = tid % K, a run of kC / (512 / K) rows each.
template <int K, int NTHR>
__device__ __forceinline__ void chunk_cumsum(const float *g, int nv, int row_stride, float *sG, int LK,
                                             float *sTot) {
    constexpr int NP = NTHR / K, RP = kC / NP;
    static_assert(RP >= 1, "at least one row per thread");
    const int tid = threadIdx.x, c = tid % K, p = tid / K;
    float acc = 0.f, gv[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) {
        const int i = p * RP + r;
        acc += i < nv ? g[static_cast<size_t>(i) * row_stride + c] : 0.f;
        gv[r] = acc;
    }
    sTot[p * K + c] = acc;
    __syncthreads();
    float off = 0.f;
    for (int pp = 0; pp < p; ++pp) off += sTot[pp * K + c];
#pragma unroll
    for (int r = 0; r < RP; ++r) sG[(p * RP + r) * LK + c] = (gv[r] + off) * kLog2e;
}

// ---------------------------------------------------------------- 1. prep
// One workgroup per (b, hv, chunk of the slab).  The element-wise parts of
// the image (k Lambda', s (q Gamma)^T, -(beta k Gamma)^T, Gamma_last) go
// straight to HBM, each thread a 16-byte hi and lo piece of 8 reduction
// indices that perm32 keeps together; the products (A_qk, Pk Rk^T) form
// their scaled operands as the MFMAs read them, from q and k in LDS as bf16
// and G.  Only the image's in-chunk matrices (s A_qk^T, T11^T, T22^T,
// -A21^T) are staged in LDS and copied out: about 48 KB of LDS, so that
// several workgroups share a CU and hide each other's latency.
template <int K>
struct PrepPlan {
    using I = Img<K>;
    static constexpr int LK = K + 4;           // fp32 [C][K] G
    static constexpr int LQ = K + 8;           // bf16 [C][K] q, k
    static constexpr int tail = I::oAq;        // image elements staged in LDS: [oAq, oGl)
    static constexpr int ntail = I::oGl - I::oAq;
    static constexpr int bytes = (kC * LK + kThr + kC + 2 * 16 * 20) * 4 + 2 * kC * LQ * 2 + ntail * 2;
    static_assert(ntail % 8 == 0, "16-byte copy of the staged part");
};

// (at least 6 waves per SIMD: three workgroups per CU, 80 VGPRs at K = 128)
template <int K>
__global__ __launch_bounds__(kThr, 6) void cbwd_prep_kernel(SlabArgs s) {
    using I = Img<K>;
    using P = PrepPlan<K>;
    constexpr int LK = P::LK, LQ = P::LQ;
    constexpr int IK = I::LK, IC = I::LC, L16 = I::L16;   // image pitches (bf16)
    const ChunkBwdArgs &a = s.a;
    extern __shared__ __attribute__((aligned(16))) float sm[];
    float *sG = sm;                         // [C][LK] base-2 cumulative sums
    float *sTot = sG + kC * LK;             // [kThr] partial column sums
    float *sB = sTot + kThr;                // [C] beta
    float *sAb = sB + kC;                   // [2][16][L16] diagonal blocks of A_kk
    uint16_t *sQ = reinterpret_cast<uint16_t *>(sAb + 2 * 16 * L16);   // [C][LQ] bf16 q, k
    uint16_t *sK = sQ + kC * LQ;
    __bf16 *st = reinterpret_cast<__bf16 *>(sK + kC * LQ);   // image elements [oAq, oGl)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 15, lg = lane >> 4;
    const int n = blockIdx.x % s.NCs;
    const int bhv = blockIdx.x / s.NCs;
    const int b = bhv / a.HV, hv = bhv % a.HV, h = hv / (a.HV / a.H);
    const int t0 = s.t_begin + n * kC;
    const int nv = min(kC, s.t_begin + s.len - t0);
    const size_t tok = static_cast<size_t>(b) * a.T + t0;
    const uint16_t *qg = static_cast<const uint16_t *>(a.q);
    const uint16_t *kg = static_cast<const uint16_t *>(a.k);
    // this chunk's image in HBM, as bf16 elements
    __bf16 *gim = reinterpret_cast<__bf16 *>(a.img + ((static_cast<size_t>(b) * s.NCs + n) * a.HV + hv) * I::floats);
    // x as its bf16 pair in the staged part: hi at image element at, lo at + half
    auto put = [&](int at, int half, float x) {
        __bf16 hi, lo;
        split1(x, hi, lo);
        st[at - P::tail] = hi;
        st[at - P::tail + half] = lo;
    };
    // 8 values as bf16 pairs, to image elements at (hi) and at + half (lo) in HBM
    auto put8 = [&](int at, int half, const float (&x)[8]) {
        bf16x4 h0, l0, h1, l1;
        split4(f32x4{x[0], x[1], x[2], x[3]}, h0, l0);
        split4(f32x4{x[4], x[5], x[6], x[7]}, h1, l1);
        *reinterpret_cast<bf16x8 *>(gim + at) = cat(h0, h1);
        *reinterpret_cast<bf16x8 *>(gim + at + half) = cat(l0, l1);
    };

    // q, k of the chunk as bf16 rows, 16 bytes per unit (rows past the end 0)
    for (int u = tid; u < kC * K / 8; u += kThr) {
        const int i = u / (K / 8), c = (u % (K / 8)) * 8;
        uint4 wq = make_uint4(0u, 0u, 0u, 0u), wk = wq;
        if (i < nv) {
            const size_t qi = ((tok + i) * a.H + h) * K + c;
            wq = *reinterpret_cast<const uint4 *>(qg + qi);
            wk = *reinterpret_cast<const uint4 *>(kg + qi);
        }
        *reinterpret_cast<uint4 *>(sQ + i * LQ + c) = wq;
        *reinterpret_cast<uint4 *>(sK + i * LQ + c) = wk;
    }
    chunk_cumsum<K, kThr>(a.g + (tok * a.HV + hv) * K, nv, a.HV * K, sG, LK, sTot);
    if (tid < kC) sB[tid] = tid < nv ? a.beta[(tok + tid) * a.HV + hv] : 0.f;
    __syncthreads();
    auto qat = [&](int i, int c) { return bf2f(sQ[i * LQ + c]); };
    auto kat = [&](int i, int c) { return bf2f(sK[i * LQ + c]); };
    // index e of the 8 that perm32 places at 8 g .. 8 g + 7 of a block of 32
    auto pidx = [](int g, int e) { return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4); };

    // k Lambda' [token i][channels of group m], 16 bytes per piece
    for (int u = tid; u < kC * K / 8; u += kThr) {
        const int i = u / (K / 8), m = u % (K / 8), c0 = (m / 4) * 32, g = m % 4;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = c0 + pidx(g, e);
            x[e] = kat(i, c) * ex2(sG[(kC - 1) * LK + c] - sG[i * LK + c]);
        }
        put8(I::oKb + i * IK + c0 + 8 * g, kC * IK, x);
    }
    // s (q Gamma)^T and -(beta k Gamma)^T [channel c][tokens of group g]
    for (int u = tid; u < K * 4; u += kThr) {
        const int c = u / 4, g = u % 4;
        float x1[8], x2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = pidx(g, e);
            const float gam = ex2(sG[i * LK + c]);
            x1[e] = a.scale * qat(i, c) * gam;
            x2[e] = -sB[i] * kat(i, c) * gam;
        }
        put8(I::oA1 + c * IC + 8 * g, K * IC, x1);
        put8(I::oA2 + c * IC + 8 * g, K * IC, x2);
    }
    // Gamma_last, fp32
    for (int c = tid; c < K; c += kThr)
        reinterpret_cast<float *>(gim + I::oGl)[c] = ex2(sG[(kC - 1) * LK + c]);

    // A_qk (waves 0-2) and Pk Rk^T (waves 3-5), lower tiles (0,0), (1,0), (1,1):
    // rows X e1 (X = q or k) against columns k e2, e1 = 2^{G_i - G_r} and
    // e2 = 2^{G_r - G_j} formed per operand element
    if (wave < 6) {
        const int t = wave % 3, rt = t == 0 ? 0 : 1, ct = t == 2 ? 1 : 0;
        const uint16_t *X = wave < 3 ? sQ : sK;
        const int xr = rt * 16 + lr, yr = ct * 16 + lr;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int k0 = 0; k0 < K; k0 += 16) {
            const int c = k0 + 4 * lg;
            const f32x4 gx = ld4(sG + xr * LK + c), gy = ld4(sG + yr * LK + c), gr = ld4(sG + kR * LK + c);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float xa = bf2f(X[xr * LQ + c + j]) * ex2(gx[j] - gr[j]);
                const float yb = kat(yr, c + j) * ex2(gr[j] - gy[j]);
                acc = mma4(xa, yb, acc);
            }
        }
        if (wave < 3) {
            // s A_qk^T: element (col, row) of A_qk, lower including the diagonal
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = rt * 16 + 4 * lg + j, col = ct * 16 + lr;
                put(I::oAq + col * IC + perm32(row), kC * IC, col <= row ? a.scale * acc[j] : 0.f);
            }
            if (wave == 0) {
                // rows 16-31 of A_qk^T, columns 0-15: above A_qk's diagonal
#pragma unroll
                for (int j = 0; j < 4; ++j) put(I::oAq + (16 + lr) * IC + perm32(4 * lg + j), kC * IC, 0.f);
            }
        } else if (t != 1) {
            // diagonal block of A_kk = diag(beta) SL(Pk Rk^T)
            const int blk = rt;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 4 * lg + j;
                sAb[blk * 16 * L16 + i * L16 + lr] = lr < i ? sB[16 * blk + i] * acc[j] : 0.f;
            }
        } else {
            // -A21^T: element (m, j) = -beta_{16+j} (Pk Rk^T)[16 + j][m]
#pragma unroll
            for (int j = 0; j < 4; ++j) put(I::oNA + lr * L16 + 4 * lg + j, 16 * L16, -sB[16 + 4 * lg + j] * acc[j]);
        }
    }
    __syncthreads();
    // T_blk = (I + A_blk)^-1 by rows: row i solves x^T (I + A_blk) = e_i^T,
    // swept k = 15 .. 1 (x_k final, removed from every earlier column; the
    // strictly lower A_blk makes the update uniform).  Lane = (row i, quarter
    // q) holds x_{4q..4q+3}.  Stored transposed: T^T[m][i] = x_m.
    if (wave < 2) {
        const int blk = wave;
        const float *A = sAb + blk * 16 * L16;
        const int i = lane >> 2, q = lane & 3;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (4 * q + e == i) ? 1.f : 0.f;
#pragma unroll
        for (int k = 15; k >= 1; --k) {
            const f32x4 av = ld4(A + k * L16 + 4 * q);
            const float xk = quad_bcast(x[k % 4], k / 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] -= av[e] * xk;
        }
        const int oT = blk == 0 ? I::oT1 : I::oT2;
#pragma unroll
        for (int e = 0; e < 4; ++e) put(oT + (4 * q + e) * L16 + i, 16 * L16, x[e]);
    }
    __syncthreads();
    // the staged in-chunk matrices to HBM, 16 bytes per thread
    for (int u = tid; u < P::ntail / 8; u += kThr)
        *reinterpret_cast<bf16x8 *>(gim + P::tail + 8 * u) = *reinterpret_cast<const bf16x8 *>(st + 8 * u);
}

// ---------------------------------------------------------------- 2. chain
// One workgroup per (b, hv, V tile of VT columns); chunks of the slab in
// reverse.  Waves 0 .. NCW-1 hold dM (NG blocks of 16 columns each, all K rows,
// in MFMA accumulators); waves 4-7 bring the next chunk's operand image and dO
// tile into the other LDS buffer.
template <int K, int VT>
__global__ __launch_bounds__(kThr, 1) void cbwd_chain_kernel(SlabArgs s) {
    using I = Img<K>;
    constexpr int LK = I::LK, LC = I::LC, L16 = I::L16;
    constexpr int KT = K / 16;
    constexpr int NCW = VT / 16 < 4 ? VT / 16 : 4;
    constexpr int NG = VT / (16 * NCW);
    constexpr int LDO = VT + 8;                                  // bf16 pitch of the dO tile
    constexpr int BUF = I::floats + (kC * LDO * 2 + 15) / 16 * 4;   // floats per buffer
    const ChunkBwdArgs &a = s.a;
    extern __shared__ __attribute__((aligned(16))) float sm[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 15, lg = lane >> 4;
    const int nvt = a.V / VT;
    const int vt = blockIdx.x % nvt, bhv = blockIdx.x / nvt;
    const int b = bhv / a.HV, hv = bhv % a.HV;
    const int v0 = vt * VT;
    const int HV = a.HV, V = a.V;
    const bool carry = wave < NCW;
    const uint16_t *dog = static_cast<const uint16_t *>(a.dout);

    // operand image and dO tile of chunk n into buffer n & 1 (waves 4-7)
    auto load = [&](int n) {
        const int hl = tid - 256;
        float *buf = sm + (n & 1) * BUF;
        const float4 *src = reinterpret_cast<const float4 *>(a.img + ((static_cast<size_t>(b) * s.NCs + n) * HV + hv) * I::floats);
        float4 *dst = reinterpret_cast<float4 *>(buf);
        // every load in flight before the first LDS store: one round trip
        constexpr int NJ = I::floats / 1024;
        constexpr int UPR = VT / 8, NUO = kC * UPR, NJO = (NUO + 255) / 256;   // dO: 8 bf16 per unit
        const int t0 = s.t_begin + n * kC;
        const int nv = min(kC, s.t_begin + s.len - t0);
        float4 t[NJ];
        uint4 w[NJO];
#pragma unroll
        for (int j = 0; j < NJ; ++j) t[j] = src[hl + 256 * j];
#pragma unroll
        for (int j = 0; j < NJO; ++j) {
            const int u = hl + 256 * j, row = u / UPR, c8 = (u % UPR) * 8;
            w[j] = make_uint4(0u, 0u, 0u, 0u);
            if (u < NUO && row < nv)
                w[j] = *reinterpret_cast<const uint4 *>(dog + ((static_cast<size_t>(b) * a.T + t0 + row) * HV + hv) * V + v0 + c8);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) dst[hl + 256 * j] = t[j];
        __bf16 *sdo = reinterpret_cast<__bf16 *>(buf + I::floats);
#pragma unroll
        for (int j = 0; j < NJO; ++j) {
            const int u = hl + 256 * j, row = u / UPR, c8 = (u % UPR) * 8;
            if (u < NUO) *reinterpret_cast<uint4 *>(sdo + row * LDO + c8) = w[j];
        }
    };

    f32x4 dm[NG][KT];
    if (carry) {
        const float *src = s.dm_in ? s.dm_in + (static_cast<size_t>(b) * HV + hv) * K * V : nullptr;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const int col = v0 + 16 * (wave * NG + gi) + lr;
#pragma unroll
            for (int kb = 0; kb < KT; ++kb)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    dm[gi][kb][j] = src ? src[static_cast<size_t>(kb * 16 + 4 * lg + j) * V + col] : 0.f;
        }
    }
    if (wave >= 4) load(s.NCs - 1);
    __syncthreads();

    for (int n = s.NCs - 1; n >= 0; --n) {
        if (wave >= 4 && n > 0) load(n - 1);
        if (carry) {
            const float *img = sm + (n & 1) * BUF;
            const __bf16 *sdo = reinterpret_cast<const __bf16 *>(img + I::floats);
            const int t0 = s.t_begin + n * kC;
            const int nv = min(kC, s.t_begin + s.len - t0);
            // dM' (the gradient at the end of chunk n) for the gradient kernel
            float *dms = a.dMs + ((static_cast<size_t>(b) * s.NCs + n) * HV + hv) * K * V;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const int col = v0 + 16 * (wave * NG + gi) + lr;
#pragma unroll
                for (int kb = 0; kb < KT; ++kb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) dms[static_cast<size_t>(kb * 16 + 4 * lg + j) * V + col] = dm[gi][kb][j];
            }
            // dO fragments (bf16, exact): rows 4 lg + j and 16 + 4 lg + j of the
            // block's column lr -- lane group lg's tokens in perm32 order
            bf16x8 dob[NG];
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                bf16x4 f[2];
#pragma unroll
                for (int b2 = 0; b2 < 2; ++b2) {
                    const int row = b2 * 16 + 4 * (lane >> 4) + ((lane >> 2) & 3);
                    const int col = 16 * (wave * NG + gi) + 4 * (lane & 3);
                    f[b2] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (__attribute__((address_space(3))) bf16x4 *)(sdo + row * LDO + col));
                }
                dob[gi] = cat(f[0], f[1]);
            }
            const __bf16 *im = reinterpret_cast<const __bf16 *>(img);
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            // dU = (k Lambda') dM' + s A_qk^T dO.  dM' (accumulator rows 4 lg + j
            // of two 16-row tiles: lane group lg's 8 rows of a block of 32) split
            // into bf16 pairs is the B operand as it stands; three terms, two
            // where dO (exact in bf16) is the B operand
            f32x4 du[NG][2];
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) du[gi][rt] = zero;
#pragma unroll
            for (int ks = 0; ks < K / 32; ++ks) {
                bf16x8 kh[2], kl[2];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const int at = I::oKb + (rt * 16 + lr) * LK + ks * 32 + 8 * lg;
                    kh[rt] = ld8(im + at);
                    kl[rt] = ld8(im + at + kC * LK);
                }
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    bf16x4 h0, l0, h1, l1;
                    split4(dm[gi][2 * ks], h0, l0);
                    split4(dm[gi][2 * ks + 1], h1, l1);
                    const bf16x8 mh = cat(h0, h1), ml = cat(l0, l1);
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) {
                        du[gi][rt] = mfma32(kh[rt], mh, du[gi][rt]);
                        du[gi][rt] = mfma32(kh[rt], ml, du[gi][rt]);
                        du[gi][rt] = mfma32(kl[rt], mh, du[gi][rt]);
                    }
                }
            }
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int at = I::oAq + (rt * 16 + lr) * LC + 8 * lg;
                const bf16x8 ah = ld8(im + at), al = ld8(im + at + kC * LC);
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    du[gi][rt] = mfma32(ah, dob[gi], du[gi][rt]);
                    du[gi][rt] = mfma32(al, dob[gi], du[gi][rt]);
                }
            }
            // dR2 = T22^T dU2;  Y = dU1 - A21^T dR2;  dR1 = T11^T Y  (16x16x16,
            // three terms; the accumulator rows 4 lg + j are the B operand's)
            const int tq = lr * L16 + 4 * lg, th = 16 * L16;
            const bf16x4 t1h = ld4h(im + I::oT1 + tq), t1l = ld4h(im + I::oT1 + th + tq);
            const bf16x4 t2h = ld4h(im + I::oT2 + tq), t2l = ld4h(im + I::oT2 + th + tq);
            const bf16x4 nah = ld4h(im + I::oNA + tq), nal = ld4h(im + I::oNA + th + tq);
            f32x4 dr[NG][2];
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                bf16x4 xh, xl;
                split4(du[gi][1], xh, xl);
                f32x4 x = mfma16(t2h, xh, zero), x2 = mfma16(t2h, xl, zero);
                x2 = mfma16(t2l, xh, x2);
                x += x2;
                dr[gi][1] = x;
                split4(x, xh, xl);
                f32x4 y = mfma16(nah, xh, du[gi][0]), y2 = mfma16(nah, xl, zero);
                y2 = mfma16(nal, xh, y2);
                y += y2;
                split4(y, xh, xl);
                f32x4 z = mfma16(t1h, xh, zero), z2 = mfma16(t1h, xl, zero);
                z2 = mfma16(t1l, xh, z2);
                dr[gi][0] = z + z2;
            }
            // dR (rows of the chunk inside the sequence) for the gradient kernel
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const int col = v0 + 16 * (wave * NG + gi) + lr;
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int row = rt * 16 + 4 * lg + j;
                        if (row < nv)
                            a.dR[((static_cast<size_t>(b) * a.Ls + n * kC + row) * HV + hv) * V + col] = dr[gi][rt][j];
                    }
            }
            // dM = Gamma_last (.) dM' + s (q Gamma)^T dO - (beta k Gamma)^T dR
            // (dR split into bf16 pairs: three terms; dO two)
            bf16x8 rbh[NG], rbl[NG];
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                bf16x4 h0, l0, h1, l1;
                split4(dr[gi][0], h0, l0);
                split4(dr[gi][1], h1, l1);
                rbh[gi] = cat(h0, h1);
                rbl[gi] = cat(l0, l1);
            }
            const float *glp = reinterpret_cast<const float *>(im + I::oGl);
#pragma unroll
            for (int kb = 0; kb < KT; ++kb) {
                const f32x4 gl = ld4(glp + kb * 16 + 4 * lg);
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) dm[gi][kb] *= gl;
                const int at1 = I::oA1 + (kb * 16 + lr) * LC + 8 * lg, at2 = I::oA2 + (kb * 16 + lr) * LC + 8 * lg;
                const bf16x8 a1h = ld8(im + at1), a1l = ld8(im + at1 + K * LC);
                const bf16x8 a2h = ld8(im + at2), a2l = ld8(im + at2 + K * LC);
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    dm[gi][kb] = mfma32(a1h, dob[gi], dm[gi][kb]);
                    dm[gi][kb] = mfma32(a1l, dob[gi], dm[gi][kb]);
                    dm[gi][kb] = mfma32(a2h, rbh[gi], dm[gi][kb]);
                    dm[gi][kb] = mfma32(a2h, rbl[gi], dm[gi][kb]);
                    dm[gi][kb] = mfma32(a2l, rbh[gi], dm[gi][kb]);
                }
            }
        }        __syncthreads();
    }
    if (carry && s.dm_out) {
        float *dst = s.dm_out + (static_cast<size_t>(b) * HV + hv) * K * V;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const int col = v0 + 16 * (wave * NG + gi) + lr;
#pragma unroll
            for (int kb = 0; kb < KT; ++kb)
#pragma unroll
                for (int j = 0; j < 4; ++j) dst[static_cast<size_t>(kb * 16 + 4 * lg + j) * V + col] = dm[gi][kb][j];
        }
    }
}

// ---------------------------------------------------------------- 3. grad
// One workgroup per (b, q/k head h, chunk of the slab); the value heads of h
// one after another, dq and dk summed over them in registers.  The chunk's
// dO, dR and U are staged in LDS once per head (every wave reads all of their
// rows); each wave's [C x K] tiles share one 16-column block of K, so it loads
// that block's 16 rows of M and dM' once for both, half of V at a time.
template <int K, int V>
__global__ __launch_bounds__(kThrG, 1) void cbwd_grad_kernel(SlabArgs s) {
    constexpr int LK = K + 4, LC = kC + 4, LV = V + 4, LQ = K + 8, LO = V + 8;
    constexpr int KT = K / 16;
    constexpr int NT = 2 * KT;              // 16x16 tiles of a [C][K] result
    constexpr int TPW = (NT + 7) / 8;       // tiles per wave (all of one column block)
    constexpr int VS = V / 16;              // reduction blocks over V
    const ChunkBwdArgs &a = s.a;
    extern __shared__ __attribute__((aligned(16))) float sm[];
    float *sG = sm;                         // [C][LK] base-2 cumulative sums
    float *sPqT = sG + kC * LK;             // [K][LC] (q e1)^T, (k e1)^T, (k e2)^T
    float *sPkT = sPqT + K * LC;
    float *sRkT = sPkT + K * LC;
    float *sDq = sRkT + K * LC;             // [C][LC] dA_qk, dA_qk^T, dA_kk, (beta dA_kk)^T
    float *sDqT = sDq + kC * LC;
    float *sDk = sDqT + kC * LC;
    float *sDkbT = sDk + kC * LC;
    float *sdR = sDkbT + kC * LC;           // [C][LV] dR, U of the chunk and head
    float *sU = sdR + kC * LV;
    float *sTot = sU + kC * LV;             // [kThrG] partial column sums
    float *sB = sTot + kThrG;               // [C] beta
    float *sDb = sB + kC;                   // [4][C] partial dbeta
    float *sCs = sDb + 4 * kC;              // [8][K] partial column sums of the dg terms
    float *sXw = sCs + 8 * K;               // [K/16][C] partial rowsum((k Gamma) (.) dR M^T)
    uint16_t *sQ = reinterpret_cast<uint16_t *>(sXw + 8 * kC);   // [C][LQ] bf16 q, k
    uint16_t *sK = sQ + kC * LQ;
    uint16_t *sdO = sK + kC * LQ;           // [C][LO] bf16 dO

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 15, lg = lane >> 4;
    const int n = blockIdx.x % s.NCs;
    const int bh = blockIdx.x / s.NCs;
    const int b = bh / a.H, h = bh % a.H;
    const int G = a.HV / a.H;
    const int HV = a.HV;
    const int t0 = s.t_begin + n * kC;
    const int nv = min(kC, s.t_begin + s.len - t0);
    const size_t tok = static_cast<size_t>(b) * a.T + t0;
    const uint16_t *qg = static_cast<const uint16_t *>(a.q);
    const uint16_t *kg = static_cast<const uint16_t *>(a.k);
    const uint16_t *dog = static_cast<const uint16_t *>(a.dout);
    const float scale = a.scale;
    const bool has_tiles = wave < NT;
    const int ct = wave % KT;               // this wave's column block of K (every tile of the wave)
    const int yr = ct * 16 + lr;

    // q, k of the chunk as bf16 rows, 16 bytes per unit (rows past the end 0)
    for (int u = tid; u < kC * K / 8; u += kThrG) {
        const int i = u / (K / 8), c = (u % (K / 8)) * 8;
        uint4 wq = make_uint4(0u, 0u, 0u, 0u), wk = wq;
        if (i < nv) {
            const size_t qi = ((tok + i) * a.H + h) * K + c;
            wq = *reinterpret_cast<const uint4 *>(qg + qi);
            wk = *reinterpret_cast<const uint4 *>(kg + qi);
        }
        *reinterpret_cast<uint4 *>(sQ + i * LQ + c) = wq;
        *reinterpret_cast<uint4 *>(sK + i * LQ + c) = wk;
    }
    auto qk_at = [&](const uint16_t *base, int i, int c) { return bf2f(base[i * LQ + c]); };
    auto dO4 = [&](int row, int col) -> f32x4 {
        const uint2 w = *reinterpret_cast<const uint2 *>(sdO + row * LO + col);
        return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
    };

    f32x4 dqa[TPW], dka[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) dqa[u] = dka[u] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int gv = 0; gv < G; ++gv) {
        const int hv = h * G + gv;
        // slab-local rows of this chunk in the [B, Ls, HV, V] arrays
        const size_t lrow0 = static_cast<size_t>(b) * a.Ls + n * kC;
        const float *Ug = a.U + (lrow0 * HV + hv) * V;
        const uint16_t *vg = static_cast<const uint16_t *>(a.v) + (tok * HV + hv) * V;
        const float *dRg = a.dR + (lrow0 * HV + hv) * V;
        const uint16_t *dOg = dog + (tok * HV + hv) * V;
        const size_t rs = static_cast<size_t>(HV) * V;   // row stride of those arrays
        // dO (8 bf16 per unit), dR and U (4 floats per unit) of the chunk: every
        // load in flight before the first wait (rows past the end are 0)
        constexpr int NUO = kC * V / 8, NUF = kC * V / 4;
        constexpr int JO = (NUO + kThrG - 1) / kThrG, JF = (NUF + kThrG - 1) / kThrG;
        uint4 wo[JO];
        f32x4 wr[JF], wu[JF];
#pragma unroll
        for (int j = 0; j < JO; ++j) {
            const int u = tid + kThrG * j, i = u / (V / 8), c = (u % (V / 8)) * 8;
            wo[j] = make_uint4(0u, 0u, 0u, 0u);
            if (u < NUO && i < nv) wo[j] = *reinterpret_cast<const uint4 *>(dOg + i * rs + c);
        }
#pragma unroll
        for (int j = 0; j < JF; ++j) {
            const int u = tid + kThrG * j, i = u / (V / 4), c = (u % (V / 4)) * 4;
            wr[j] = wu[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (u < NUF && i < nv) {
                wr[j] = ld4(dRg + i * rs + c);
                wu[j] = ld4(Ug + i * rs + c);
            }
        }
        __syncthreads();   // the previous head's LDS reads are done
        chunk_cumsum<K, kThrG>(a.g + (tok * HV + hv) * K, nv, HV * K, sG, LK, sTot);
        if (tid < kC) sB[tid] = tid < nv ? a.beta[(tok + tid) * HV + hv] : 0.f;
#pragma unroll
        for (int j = 0; j < JO; ++j) {
            const int u = tid + kThrG * j, i = u / (V / 8), c = (u % (V / 8)) * 8;
            if (u < NUO) *reinterpret_cast<uint4 *>(sdO + i * LO + c) = wo[j];
        }
#pragma unroll
        for (int j = 0; j < JF; ++j) {
            const int u = tid + kThrG * j, i = u / (V / 4), c = (u % (V / 4)) * 4;
            if (u < NUF) {
                *reinterpret_cast<f32x4 *>(sdR + i * LV + c) = wr[j];
                *reinterpret_cast<f32x4 *>(sU + i * LV + c) = wu[j];
            }
        }
        __syncthreads();
        for (int e = tid; e < kC * K; e += kThrG) {
            const int c = e / kC, i = e % kC;   // consecutive threads: consecutive rows of one column
            const float Gi = sG[i * LK + c], Gr = sG[kR * LK + c];
            const float e1 = ex2(Gi - Gr), e2 = ex2(Gr - Gi);
            const float qv = qk_at(sQ, i, c), kv = qk_at(sK, i, c);
            sPqT[c * LC + i] = qv * e1;
            sPkT[c * LC + i] = kv * e1;
            sRkT[c * LC + i] = kv * e2;
        }
        __syncthreads();

        if (wave < 6) {
            // dA_qk = s L(dO U^T) (waves 0-2), dA_kk = -SL(dR U^T) and the
            // dbeta term with SL(Pk Rk^T) (waves 3-5); lower tiles (0,0), (1,0), (1,1)
            const int t = wave % 3, rt = t == 0 ? 0 : 1, ctt = t == 2 ? 1 : 0;
            const int xr = rt * 16 + lr, jr = ctt * 16 + lr;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < VS; ++st) {
                const int c = st * 16 + 4 * lg;
                const f32x4 xa = wave < 3 ? dO4(xr, c) : ld4(sdR + xr * LV + c);
                const f32x4 yb = ld4(sU + jr * LV + c);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc = mma4(xa[j], yb[j], acc);
            }
            if (wave < 3) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = rt * 16 + 4 * lg + j, col = ctt * 16 + lr;
                    const float x = col <= row ? scale * acc[j] : 0.f;
                    sDq[row * LC + col] = x;
                    sDqT[col * LC + row] = x;
                }
                if (wave == 0) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        sDq[(4 * lg + j) * LC + 16 + lr] = 0.f;
                        sDqT[(16 + lr) * LC + 4 * lg + j] = 0.f;
                    }
                }
            } else {
                // Pk Rk^T of the tile, from the transposed operands
                f32x4 ar = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
                for (int k0 = 0; k0 < K; k0 += 16)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int kk = k0 + 4 * lg + j;
                        ar = mma4(sPkT[kk * LC + xr], sRkT[kk * LC + jr], ar);
                    }
                float part[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = rt * 16 + 4 * lg + j, col = ctt * 16 + lr;
                    const float x = col < row ? -acc[j] : 0.f;
                    sDk[row * LC + col] = x;
                    sDkbT[col * LC + row] = sB[row] * x;
                    part[j] = x * ar[j];
                }
                if (wave == 3) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        sDk[(4 * lg + j) * LC + 16 + lr] = 0.f;
                        sDkbT[(16 + lr) * LC + 4 * lg + j] = 0.f;
                    }
                }
                // row sums over the tile's 16 columns (one DPP row of lanes)
#pragma unroll
                for (int j = 0; j < 4; ++j) part[j] = group_sum<16>(part[j]);
                if (lr == 0) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) sDb[(t == 2 ? 1 : 0) * kC + rt * 16 + 4 * lg + j] = part[j];
                }
            }
        } else if (wave < 8) {
            // waves 6-7: dv = beta dR, and rowsum(dR (.) v); lane = (row, quarter of V)
            const int l = tid - 384, row = l >> 2, qv = l & 3;
            float dot = 0.f;
            if (row < nv) {
                uint16_t *dvg = static_cast<uint16_t *>(a.dv) + ((tok + row) * HV + hv) * V;
                const float bt = sB[row];
                f32x4 ww[VS];
#pragma unroll
                for (int st = 0; st < VS; ++st) {
                    const uint2 w2 = *reinterpret_cast<const uint2 *>(vg + row * rs + st * 16 + qv * 4);
                    ww[st] = f32x4{__uint_as_float(w2.x << 16), __uint_as_float(w2.x & 0xffff0000u),
                                   __uint_as_float(w2.y << 16), __uint_as_float(w2.y & 0xffff0000u)};
                }
#pragma unroll
                for (int st = 0; st < VS; ++st) {
                    const int c = st * 16 + qv * 4;
                    const f32x4 d = ld4(sdR + row * LV + c), w = ww[st];
                    dot += d[0] * w[0] + d[1] * w[1] + d[2] * w[2] + d[3] * w[3];
                    uint2 o;
                    o.x = static_cast<uint32_t>(float_to_bf16_bits(bt * d[0])) | (static_cast<uint32_t>(float_to_bf16_bits(bt * d[1])) << 16);
                    o.y = static_cast<uint32_t>(float_to_bf16_bits(bt * d[2])) | (static_cast<uint32_t>(float_to_bf16_bits(bt * d[3])) << 16);
                    *reinterpret_cast<uint2 *>(dvg + c) = o;
                }
            }
            dot += lanes::dpp<0xb1>(dot);
            dot += lanes::dpp<0x4e>(dot);
            if (qv == 0) sDb[2 * kC + row] = dot;
        }
        __syncthreads();

        // [C x K] results: tiles (rt, ct) of this wave.  Its rows of M (the
        // state at the chunk start) and dM' (the gradient at its end) are
        // loaded once for both tiles, half of V at a time (all in flight together)
        const float *Mn = n == 0 ? (s.Sstart ? s.Sstart + b * s.s_bstride + static_cast<size_t>(hv) * K * V : nullptr)
                                 : a.snapc + ((static_cast<size_t>(b) * (s.NCs - 1) + n - 1) * HV + hv) * K * V;
        const float *dMn = a.dMs + ((static_cast<size_t>(b) * s.NCs + n) * HV + hv) * K * V;
        constexpr int VH = VS > 4 ? 4 : VS;     // reduction blocks per half
        f32x4 x1[TPW], x2[TPW], x3[TPW];
#pragma unroll
        for (int u = 0; u < TPW; ++u) x1[u] = x2[u] = x3[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (has_tiles) {
#pragma unroll
            for (int s0 = 0; s0 < VS; s0 += VH) {
                f32x4 mrow[VH], dmrow[VH];
#pragma unroll
                for (int st = 0; st < VH; ++st) {
                    const int c = (s0 + st) * 16 + 4 * lg;
                    mrow[st] = Mn ? ld4(Mn + static_cast<size_t>(yr) * V + c) : f32x4{0.f, 0.f, 0.f, 0.f};
                    dmrow[st] = ld4(dMn + static_cast<size_t>(yr) * V + c);
                }
#pragma unroll
                for (int u = 0; u < TPW; ++u) {
                    const int tile = wave + 8 * u;
                    if (tile < NT) {
                        const int xr = (tile / KT) * 16 + lr;
                        // dO M^T, dR M^T, U dM'^T over this half of V; dO, dR, U rows from LDS
#pragma unroll
                        for (int st = 0; st < VH; ++st) {
                            const int c = (s0 + st) * 16 + 4 * lg;
                            const f32x4 o4 = dO4(xr, c), r4 = ld4(sdR + xr * LV + c), u4 = ld4(sU + xr * LV + c);
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                x1[u] = mma4(o4[j], mrow[st][j], x1[u]);
                                x2[u] = mma4(r4[j], mrow[st][j], x2[u]);
                                x3[u] = mma4(u4[j], dmrow[st][j], x3[u]);
                            }
                        }
                    }
                    // one tile at a time: both tiles' operand reads would not fit the registers
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        float *eg = a.e + ((static_cast<size_t>(b) * a.Ls + n * kC) * HV + hv) * K;
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int tile = wave + 8 * u;
            if (tile < NT) {
                const int rt = tile / KT;
                const int xr = rt * 16 + lr;
                f32x4 y1 = {0.f, 0.f, 0.f, 0.f}, y2 = y1, y3 = y1;
                // dA_qk Rk, dA_kk Rk, dA_qk^T Pq + (beta dA_kk)^T Pk over the chunk's rows
                tile_nt<kC>(sDq + xr * LC, sRkT + yr * LC, lg, y1);
                tile_nt<kC>(sDk + xr * LC, sRkT + yr * LC, lg, y2);
                tile_nt<kC>(sDqT + xr * LC, sPqT + yr * LC, lg, y3);
                tile_nt<kC>(sDkbT + xr * LC, sPkT + yr * LC, lg, y3);
                const int c = ct * 16 + lr;
                const float Gr = sG[kR * LK + c], Gl = sG[(kC - 1) * LK + c];
                float csum = 0.f, wx[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = rt * 16 + 4 * lg + j;
                    const float Gi = sG[i * LK + c];
                    const float gam = ex2(Gi), e1 = ex2(Gi - Gr), e2 = ex2(Gr - Gi), lam = ex2(Gl - Gi);
                    const float bt = sB[i];
                    const float dq = scale * gam * x1[u][j] + e1 * y1[j];
                    const float dkr = bt * (e1 * y2[j] - gam * x2[u][j]);
                    const float dkw = lam * x3[u][j] + e2 * y3[j];
                    const float q = qk_at(sQ, i, c), k = qk_at(sK, i, c);
                    const float term = q * dq + k * (dkr - dkw);   // 0 on rows past the end (q = k = 0)
                    if (i < nv) eg[static_cast<size_t>(i) * HV * K + c] = term;
                    csum += term;
                    dqa[u][j] += dq;
                    dka[u][j] += dkr + dkw;
                    wx[j] = k * gam * x2[u][j];
                }
                sCs[(rt * 4 + lg) * K + c] = csum;
                // this column block's part of rowsum((k Gamma) (.) dR M^T)
#pragma unroll
                for (int j = 0; j < 4; ++j) wx[j] = group_sum<16>(wx[j]);
                if (lr == 0) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) sXw[ct * kC + rt * 16 + 4 * lg + j] = wx[j];
                }
            }
        }
        // the chunk's sum of the dg terms per column, for the reverse sum over chunks
        __syncthreads();
        if (tid < K) {
            float cs = 0.f;
#pragma unroll
            for (int r = 0; r < 8; ++r) cs += sCs[r * K + tid];
            a.cs[((static_cast<size_t>(b) * HV + hv) * s.NCs + n) * K + tid] = cs;
        }
        if (tid < nv) {
            // dbeta: rowsum(dR (.) v) - rowsum((k Gamma) (.) dR M^T) (= rowsum(dR (.) W))
            // and the A_kk tile terms (rows 0-15 one, rows 16-31 two)
            float wx = 0.f;
#pragma unroll
            for (int cb = 0; cb < KT; ++cb) wx += sXw[cb * kC + tid];
            const float dA = sDb[tid] + (tid >= 16 ? sDb[kC + tid] : 0.f);
            a.dbeta[(tok + tid) * HV + hv] = (sDb[2 * kC + tid] - wx) + dA;
        }
    }
    // dq, dk (bf16) of the chunk's rows inside the sequence
    uint16_t *dqg = static_cast<uint16_t *>(a.dq), *dkg = static_cast<uint16_t *>(a.dk);
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int tile = wave + 8 * u;
        if (tile < NT) {
            const int rt = tile / KT;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = rt * 16 + 4 * lg + j;
                if (i < nv) {
                    const size_t o = ((tok + i) * a.H + h) * K + ct * 16 + lr;
                    dqg[o] = float_to_bf16_bits(dqa[u][j]);
                    dkg[o] = float_to_bf16_bits(dka[u][j]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------- 4. dg
// dg_u = sum over V of S_T (.) dL/dS_T + sum over t >= u of the dg terms e_t
// (the identity in the header).  The final-state term starts the carry:
// gc[b, hv, k] = sum_v S_T[k][v] dL/dS_T[k][v].
__global__ __launch_bounds__(256) void cbwd_dg_final_kernel(ChunkBwdArgs a, float *gc) {
    const long n = static_cast<long>(a.B) * a.HV * a.K;
    const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    float c = 0.f;
    if (a.dST) {
        const f32x4 *st = reinterpret_cast<const f32x4 *>(a.ST + i * a.V);
        const f32x4 *ds = reinterpret_cast<const f32x4 *>(a.dST + i * a.V);
        for (int v = 0; v < a.V / 4; ++v) {
            const f32x4 x = st[v], y = ds[v];
            c += (x[0] * y[0] + x[1] * y[1]) + (x[2] * y[2] + x[3] * y[3]);
        }
    }
    gc[i] = c;
}

// T = 0: dS0 = dL/dS_T, or zeros without it (a kernel rather than a memset or
// copy node, so that the call records only kernels when captured).
__global__ __launch_bounds__(256) void cbwd_ds0_kernel(float *dS0, const float *dST, long n) {
    const long stride = static_cast<long>(gridDim.x) * 256;
    for (long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride)
        dS0[i] = dST ? dST[i] : 0.f;
}

// One slab: thread = (b, hv, chunk j, k).  The carry in (the final-state term
// and every later slab's terms) plus the later chunks' sums, then the chunk's
// 32 tokens from the last; the thread of chunk 0 leaves the carry for the
// slab before.
__global__ __launch_bounds__(256) void cbwd_dg_kernel(SlabArgs s, const float *gc_in, float *gc_out) {
    const ChunkBwdArgs &a = s.a;
    const long n = static_cast<long>(a.B) * a.HV * s.NCs * a.K;
    const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    const int k = static_cast<int>(i % a.K);
    const long r = i / a.K;
    const int j = static_cast<int>(r % s.NCs);
    const long bhv = r / s.NCs;
    const int b = static_cast<int>(bhv / a.HV), hv = static_cast<int>(bhv % a.HV);
    float acc = gc_in[bhv * a.K + k];
    for (int jj = s.NCs - 1; jj > j; --jj) acc += a.cs[(bhv * s.NCs + jj) * a.K + k];
    const int nv = min(kC, s.len - j * kC);
    const size_t step = static_cast<size_t>(a.HV) * a.K;
    const float *e = a.e + ((static_cast<size_t>(b) * a.Ls + j * kC) * a.HV + hv) * a.K + k;
    float *dg = a.dg + ((static_cast<size_t>(b) * a.T + s.t_begin + j * kC) * a.HV + hv) * a.K + k;
    float ev[kC];
#pragma unroll
    for (int t = 0; t < kC; ++t) ev[t] = t < nv ? e[t * step] : 0.f;
#pragma unroll
    for (int t = kC - 1; t >= 0; --t) {
        acc += ev[t];
        if (t < nv) dg[t * step] = acc;
    }
    if (j == 0) gc_out[bhv * a.K + k] = acc;
}

template <int K>
constexpr int prep_lds() { return PrepPlan<K>::bytes; }
template <int K, int VT>
constexpr int chain_lds() { return 2 * (Img<K>::floats + (kC * (VT + 8) * 2 + 15) / 16 * 4) * 4; }
template <int K, int V>
constexpr int grad_lds() {
    return (kC * (K + 4) + 3 * K * (kC + 4) + 4 * kC * (kC + 4) + 2 * kC * (V + 4) + kThrG + kC + 4 * kC + 8 * K + 8 * kC) * 4
         + (2 * kC * (K + 8) + kC * (V + 8)) * 2;
}

template <typename F>
hipError_t launch_dyn(F kern, unsigned grid, int lds, hipStream_t stream, const SlabArgs &s, int threads = kThr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, stream, s);
    return hipGetLastError();
}

template <int K>
hipError_t launch_prep_k(const SlabArgs &s, hipStream_t stream) {
    static_assert(prep_lds<K>() <= 160 * 1024, "LDS plan exceeds 160 KB");
    return launch_dyn(cbwd_prep_kernel<K>, static_cast<unsigned>(s.a.B) * s.a.HV * s.NCs, prep_lds<K>(), stream, s);
}
// One workgroup per (b, hv) with all of V: the chain is bound by bringing in
// each chunk's operand image, not by its matrix work, and a head split over
// two workgroups reads the image twice (measured 0.3 ms slower per call on the
// HV96 shape, where the forward does split V).
template <int K, int V>
hipError_t launch_chain_kv(const SlabArgs &s, hipStream_t stream) {
    static_assert(chain_lds<K, V>() <= 160 * 1024, "LDS plan exceeds 160 KB");
    return launch_dyn(cbwd_chain_kernel<K, V>, static_cast<unsigned>(s.a.B) * s.a.HV, chain_lds<K, V>(), stream, s);
}
template <int K, int V>
hipError_t launch_grad_kv(const SlabArgs &s, hipStream_t stream) {
    static_assert(grad_lds<K, V>() <= 160 * 1024, "LDS plan exceeds 160 KB");
    return launch_dyn(cbwd_grad_kernel<K, V>, static_cast<unsigned>(s.a.B) * s.a.H * s.NCs, grad_lds<K, V>(), stream, s,
                      kThrG);
}
enum class Pass { prep, chain, grad };
template <int K, int V>
hipError_t launch_pass_kv(Pass p, const SlabArgs &s, hipStream_t stream) {
    switch (p) {
    case Pass::prep: return launch_prep_k<K>(s, stream);
    case Pass::chain: return launch_chain_kv<K, V>(s, stream);
    default: return launch_grad_kv<K, V>(s, stream);
    }
}
template <int K>
hipError_t launch_pass_k(Pass p, const SlabArgs &s, hipStream_t stream) {
    switch (s.a.V) {
    case 32: return launch_pass_kv<K, 32>(p, s, stream);
    case 64: return launch_pass_kv<K, 64>(p, s, stream);
    case 128: return launch_pass_kv<K, 128>(p, s, stream);
    default: return hipErrorInvalidValue;
    }
}
hipError_t launch_pass(Pass p, const SlabArgs &s, hipStream_t stream) {
    switch (s.a.K) {
    case 32: return launch_pass_k<32>(p, s, stream);
    case 64: return launch_pass_k<64>(p, s, stream);
    case 128: return launch_pass_k<128>(p, s, stream);
    default: return hipErrorInvalidValue;
    }
}

// The three further streams of the backward (one set per device, default
// priority, created on first use) and the events that order them against the
// caller's.  The mutex makes one call's enqueue sequence atomic, so calls from
// several host threads on one device do not interleave their event records.
struct SideStream {
    std::mutex mu;
    hipStream_t y = nullptr, z = nullptr, w = nullptr;
    hipEvent_t start = nullptr, st = nullptr, p0[2] = {}, prep[2] = {}, chain[2] = {}, grad[2] = {};
    hipEvent_t zdone = nullptr;
    bool ready = false;   // every stream and event above created
};
constexpr int kMaxDev = 64;
SideStream g_side[kMaxDev];

hipError_t side_stream(hipStream_t stream, SideStream **out) {
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    SideStream &ss = g_side[dev];
    *out = &ss;
    std::lock_guard<std::mutex> lock(ss.mu);   // one creation per device, whichever thread comes first
    if (ss.ready) return hipSuccess;
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    e = hipStreamCreateWithFlags(&ss.y, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&ss.z, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&ss.w, hipStreamNonBlocking);
    hipEvent_t *evs[] = {&ss.start, &ss.st, &ss.p0[0], &ss.p0[1], &ss.prep[0], &ss.prep[1],
                         &ss.chain[0], &ss.chain[1], &ss.grad[0], &ss.grad[1], &ss.zdone};
    for (hipEvent_t *ev : evs)
        if (e == hipSuccess) e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
    ss.ready = e == hipSuccess;
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    return e != hipSuccess ? e : e2;
}

}  // namespace

int chunk_bwd_image_floats(int K) {
    return K == 32 ? Img<32>::floats : K == 64 ? Img<64>::floats : K == 128 ? Img<128>::floats : 0;
}

// Slab by slab from the last, on four streams.  The caller's stream X runs
// the chain of state gradients, slab after slab.  A second stream Y runs the
// forward passes the chain's consumers need -- the whole sequence, then each
// slab -- and a third, P, the operand images, which depend on the inputs
// alone, both ahead of X; a fourth, Z, runs each slab's gradient pass and dg
// sums once its chain is done, beside the chain of the slab before.  Y, P and
// Z use the CUs the chain leaves idle (one workgroup per head).  Per-slab
// buffers that one stream writes while another may still read the previous
// slab's (chunk-start states and U from Y; images from P; dR and every
// chunk's dM' from X) are double-buffered by slab parity, and each is
// overwritten only after the pass of the slab two before that reads it is
// done.  X waits for Z's last work before the call's enqueue ends, so work
// enqueued on X afterwards runs after all of it.
//
// While the caller's stream is being captured into a graph, every pass runs
// in the same order on that stream alone: no side streams, events or stream
// queries are recorded (the enqueue order below satisfies every dependency
// the events express, so the results are the same bits).
hipError_t launch_chunk_backward(const ChunkBwdArgs &a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    const size_t sKV = static_cast<size_t>(a.HV) * a.K * a.V;
    if (a.T == 0) {
        // only dS0 = dL/dS_T (or zeros)
        if (!a.dS0) return hipSuccess;
        const long n = static_cast<long>(a.B) * static_cast<long>(sKV);
        const long blocks = std::min<long>((n + 255) / 256, 4096);
        hipLaunchKernelGGL(cbwd_ds0_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a.dS0,
                           a.dST, n);
        return hipGetLastError();
    }
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    const bool serial = cap != hipStreamCaptureStatusNone;
    SideStream none, *ss = &none;   // none: events never used (serial)
    std::unique_lock<std::mutex> lock;
    hipStream_t X = stream, Y = stream, Z = stream, P = stream;
    if (!serial) {
        e = side_stream(stream, &ss);
        if (e != hipSuccess) return e;
        lock = std::unique_lock<std::mutex>(ss->mu);
        Y = ss->y;
        Z = ss->z;
        P = ss->w;
    }
    auto rec = [&](hipEvent_t ev, hipStream_t s) { return serial ? hipSuccess : hipEventRecord(ev, s); };
    auto wait = [&](hipStream_t s, hipEvent_t ev) { return serial ? hipSuccess : hipStreamWaitEvent(s, ev, 0); };
#define KDA_TRY(x) do { const hipError_t e_ = (x); if (e_ != hipSuccess) return e_; } while (0)
    KDA_TRY(rec(ss->start, X));
    KDA_TRY(wait(Y, ss->start));
    KDA_TRY(wait(Z, ss->start));
    KDA_TRY(wait(P, ss->start));
    const int ns = (a.T + a.Ls - 1) / a.Ls;
    // 0. the whole sequence once: S_T and the states at the slab starts
    // (given by the caller in the saved variant)
    if (!a.saved) {
        PrefillArgs f{};
        f.q = a.q; f.k = a.k; f.v = a.v; f.g = a.g; f.beta = a.beta; f.S0 = a.S0;
        f.ST = a.ST;
        f.snap = ns > 1 ? a.snap1 : nullptr;
        f.snap_chunks = a.Ls / kC; f.NS = ns - 1;
        f.B = a.B; f.T = a.T; f.H = a.H; f.HV = a.HV; f.K = a.K; f.V = a.V;
        f.scale = a.scale; f.bf16 = true; f.bwd = true;
        KDA_TRY(launch_prefill_bf16(f, Y));
        KDA_TRY(rec(ss->st, Y));
    }
    float *gc[2] = {a.gc, a.gc + static_cast<size_t>(a.B) * a.HV * a.K};
    {
        if (!a.saved) KDA_TRY(wait(Z, ss->st));
        const long nk = static_cast<long>(a.B) * a.HV * a.K;
        hipLaunchKernelGGL(cbwd_dg_final_kernel, dim3(static_cast<unsigned>((nk + 255) / 256)), dim3(256), 0,
                           Z, a, gc[0]);
        KDA_TRY(hipGetLastError());
    }
    for (int si = ns - 1, j = 0; si >= 0; --si, ++j) {
        const int p = si & 1;
        SlabArgs s{};
        s.a = a;
        if (p) {
            s.a.snapc = a.snapc2; s.a.U = a.U2; s.a.img = a.img2;
            s.a.dR = a.dR2; s.a.dMs = a.dMs2;
        }
        s.t_begin = si * a.Ls;
        s.len = min(a.T, s.t_begin + a.Ls) - s.t_begin;
        s.NCs = (s.len + kC - 1) / kC;
        if (si == 0) {
            s.Sstart = a.S0;
            s.s_bstride = static_cast<long long>(sKV);
        } else {
            s.Sstart = a.snap1 + static_cast<size_t>(si - 1) * sKV;
            s.s_bstride = static_cast<long long>(a.saved ? a.NSsaved : a.NS1) * sKV;
        }
        s.dm_in = si == ns - 1 ? a.dST : a.Dc;
        s.dm_out = si == 0 ? a.dS0 : a.Dc;
        // Y: the slab's forward pass (states at its chunk starts, U) once the
        // gradient pass of slab si + 2 has read these buffers
        if (j >= 2) KDA_TRY(wait(Y, ss->grad[p]));
        PrefillArgs f{};
        f.q = a.q; f.k = a.k; f.v = a.v; f.g = a.g; f.beta = a.beta;
        f.S0 = s.Sstart; f.s0_bstride = s.s_bstride;
        f.snap = s.NCs > 1 ? s.a.snapc : nullptr;
        f.snap_chunks = 1; f.NS = s.NCs - 1;
        f.u_out = s.a.U; f.Lw = a.Ls;
        f.t_off = s.t_begin; f.Tseq = a.T;
        f.B = a.B; f.T = s.len; f.H = a.H; f.HV = a.HV; f.K = a.K; f.V = a.V;
        f.scale = a.scale; f.bf16 = true; f.bwd = true;
        KDA_TRY(launch_prefill_bf16(f, Y));
        KDA_TRY(rec(ss->p0[p], Y));
        // P: the operand images (from the inputs alone), once the chain of
        // slab si + 2 has read this parity's
        if (j >= 2) KDA_TRY(wait(P, ss->chain[p]));
        KDA_TRY(launch_pass(Pass::prep, s, P));
        KDA_TRY(rec(ss->prep[p], P));
        // X: the chain, once the images are there and the gradient pass of
        // slab si + 2 has read this parity's dR and dM'
        KDA_TRY(wait(X, ss->prep[p]));
        if (j >= 2) KDA_TRY(wait(X, ss->grad[p]));
        KDA_TRY(launch_pass(Pass::chain, s, X));
        KDA_TRY(rec(ss->chain[p], X));
        // Z: the gradient pass and dg (carried to the slab before)
        KDA_TRY(wait(Z, ss->chain[p]));
        KDA_TRY(wait(Z, ss->p0[p]));
        KDA_TRY(launch_pass(Pass::grad, s, Z));
        KDA_TRY(rec(ss->grad[p], Z));
        const long nd = static_cast<long>(a.B) * a.HV * s.NCs * a.K;
        hipLaunchKernelGGL(cbwd_dg_kernel, dim3(static_cast<unsigned>((nd + 255) / 256)), dim3(256), 0, Z, s,
                           gc[j & 1], gc[(j + 1) & 1]);
        KDA_TRY(hipGetLastError());
    }
    // everything on Y and P ends in work X or Z waited for; Z's end joins X
    KDA_TRY(rec(ss->zdone, Z));
    KDA_TRY(wait(X, ss->zdone));
#undef KDA_TRY
    return hipSuccess;
}

}  // namespace kda
