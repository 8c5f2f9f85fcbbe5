// In-chunk matrices of the KDA chunk form for gates with no lower bound
// (kda_chunk_fwd_unbounded): a chunk-parallel pass ahead of the bf16 chunk
// kernel's unbounded instantiation (kda_prefill_bf16.hip, UNB).
//
// The chunk form (delta_recurrence on the page
// "src/tinycenn_lm/research_layers.py", specialised to KDA) needs, per chunk
// of 32 tokens and key channel c, the decay between tokens j <= i of the
// chunk, 2^{G_i - G_j}, G the chunk-local cumulative sum of g (base 2):
//     A_qk[i][j] = sum_c q_ic k_jc 2^{G_ic - G_jc}      j <= i
//     A_kk[i][j] = beta_i sum_c k_ic k_jc 2^{G_ic - G_jc}  j < i
// As a matrix product the factor splits around a reference row r,
// 2^{G_i - G_r} 2^{G_r - G_j}.  The bounded prefill takes one r for the whole
// chunk, which keeps both factors in fp32 only while the decay over 15 tokens
// stays below about 2^116 (g >= -5).  Here the lower triangle is covered by
// blocks that each have a reference row of their own:
//   F1  rows 16..31 x columns 0..15, r = 15: both factors <= 1;
//   F2  rows 8..15 x 0..7 and 24..31 x 16..23, r = 7 and 23: both <= 1;
//   F3  j <= i inside each block of 8 tokens, r = its fourth token (3, 11,
//       19, 27): at most 3 tokens before r and 4 after it.
// Each token's log-decay is floored at kUnbFloor = -17 (2^-24.5) first, so
// an F3 factor lies in [2^-98, 2^98]: no overflow, and no operand above
// 2^-126 |q| flushes.  The floor changes a token's decay only where it keeps
// less than e^-17 (4e-8) of the state: such a token then keeps 4e-8 of it.
// The chunk kernel applies the same floor to its own cumulative sums.
//
// One workgroup of 4 waves per (b, hv, chunk).  q, k and G go to LDS as fp32;
// wave w forms the fp32 MFMA products (v_mfma_f32_16x16x4_f32) of family
// F1, F2 (both 16-blocks in one 16x16 tile), F3 of rows 0..15, F3 of rows
// 16..31, for A_qk and the raw A_kk at once; the factors are formed per
// operand element as the products read them.  Then wave 0 and 1 invert the
// two diagonal 16x16 blocks of I + A_kk (T11, T22; fp32 forward
// substitution), wave 2 forms -A21 and wave 3 rounds A_qk.  The result is one
// image per chunk in HBM, in the chunk kernel's LDS layouts, bf16 hi/lo pairs
// (x = hi + lo to about 2^-16 relative):
//     [0, 2048)     A_qk hi, lo        [32][32], columns in the MFMA's
//                                      permuted order (c -> perm(c))
//     [2048, 2560)  -A21 hi, lo        [16][16]  (rows 16..31, columns 0..15)
//     [2560, 3584)  T11 hi, lo, T22 hi, lo  [16][16] each
// kUnbImgElems bf16 per chunk, [B][HV][NC][kUnbImgElems].

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kC = 32;
constexpr int kThrU = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLA = 36;   // fp32 row pitch of the A arrays in LDS

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma4(float a, float b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
// (a, b) -> packed bf16 pair, round to nearest even
__device__ __forceinline__ uint32_t pk(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// hi = bf16(a, b), lo = bf16 of the remainders (exact differences)
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = pk(a, b);
    lo = pk(a - bf_lo(hi), b - bf_hi(hi));
}
// x of lane 4 (lane / 4) + p (DPP quad broadcast; p must fold to a constant)
__device__ __forceinline__ float quad_bcast(float x, int p) {
    const int v = __float_as_int(x);
    switch (p) {
    case 0: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x00, 0xf, 0xf, false));
    case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x55, 0xf, 0xf, false));
    case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xaa, 0xf, 0xf, false));
    default: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xff, 0xf, 0xf, false));
    }
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, static_cast<int>(bytes), 0x00020000);
}

struct UnbPrepArgs {
    const uint16_t *q, *k;      // [B,T,H,K] bf16
    const float *g, *beta;      // [B,T,HV,K], [B,T,HV]
    uint16_t *img;              // [B,HV,NC,kUnbImgElems] bf16
    int T, H, HV, NC;
};

template <int K>
struct UPlan {
    static constexpr int LK = K + 4;
    static constexpr int oQ = 0;                    // fp32 [C][LK] q
    static constexpr int oK = oQ + kC * LK;         // fp32 [C][LK] k
    static constexpr int oG = oK + kC * LK;         // fp32 [C][LK] G (base 2, floored g)
    static constexpr int oAq = oG + kC * LK;        // fp32 [C][kLA] A_qk
    static constexpr int oAk = oAq + kC * kLA;      // fp32 [C][kLA] A_kk without beta
    static constexpr int oB = oAk + kC * kLA;       // fp32 [C] beta
    static constexpr int floats = oB + kC;
};

template <int K>
__global__ __launch_bounds__(kThrU) void unb_prep_kernel(UnbPrepArgs a) {
    using P = UPlan<K>;
    constexpr int LK = P::LK;
    __shared__ __attribute__((aligned(16))) float sm[P::floats];
    float *sQ = sm + P::oQ, *sK = sm + P::oK, *sG = sm + P::oG;
    float *sAq = sm + P::oAq, *sAk = sm + P::oAk, *sB = sm + P::oB;

    const int tid = static_cast<int>(threadIdx.x);
    const int ch = static_cast<int>(blockIdx.x) % a.NC;
    const int bhv = static_cast<int>(blockIdx.x) / a.NC;
    const int b = bhv / a.HV, hv = bhv % a.HV;
    const int h = hv / (a.HV / a.H);
    const int t0 = ch * kC;
    const int nv = min(kC, a.T - t0);   // valid tokens (>= 1)
    const size_t tb = static_cast<size_t>(b) * a.T + t0;

    // ---- loads: rows past the sequence end read 0 (an exact no-op token)
    {
        const int gs = a.HV * K, qs = a.H * K;
        const auto rg = make_rsrc(a.g + (tb * a.HV + hv) * K, static_cast<uint32_t>(((nv - 1) * gs + K) * 4));
        const auto rq = make_rsrc(a.q + (tb * a.H + h) * K, static_cast<uint32_t>(((nv - 1) * qs + K) * 2));
        const auto rk = make_rsrc(a.k + (tb * a.H + h) * K, static_cast<uint32_t>(((nv - 1) * qs + K) * 2));
        constexpr int G4 = kC * K / 4;
#pragma unroll
        for (int u = tid; u < G4; u += kThrU) {
            const int row = u / (K / 4), c = (u % (K / 4)) * 4;
            const auto w = __builtin_amdgcn_raw_buffer_load_b128(rg, (row * gs + c) * 4, 0, 0);
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = fmaxf(__uint_as_float(w[e]), kUnbFloor) * kLog2e;
            *reinterpret_cast<f32x4 *>(sG + row * LK + c) = x;
        }
        constexpr int Q8 = kC * K / 8;
#pragma unroll
        for (int u = tid; u < Q8; u += kThrU) {
            const int row = u / (K / 8), c = (u % (K / 8)) * 8;
            const auto wq = __builtin_amdgcn_raw_buffer_load_b128(rq, (row * qs + c) * 2, 0, 0);
            const auto wk = __builtin_amdgcn_raw_buffer_load_b128(rk, (row * qs + c) * 2, 0, 0);
            f32x4 q0, q1, k0, k1;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                q0[2 * e] = bf_lo(wq[e]); q0[2 * e + 1] = bf_hi(wq[e]);
                q1[2 * e] = bf_lo(wq[e + 2]); q1[2 * e + 1] = bf_hi(wq[e + 2]);
                k0[2 * e] = bf_lo(wk[e]); k0[2 * e + 1] = bf_hi(wk[e]);
                k1[2 * e] = bf_lo(wk[e + 2]); k1[2 * e + 1] = bf_hi(wk[e + 2]);
            }
            *reinterpret_cast<f32x4 *>(sQ + row * LK + c) = q0;
            *reinterpret_cast<f32x4 *>(sQ + row * LK + c + 4) = q1;
            *reinterpret_cast<f32x4 *>(sK + row * LK + c) = k0;
            *reinterpret_cast<f32x4 *>(sK + row * LK + c + 4) = k1;
        }
        if (tid < kC) {
            const auto rb = make_rsrc(a.beta + tb * a.HV + hv, static_cast<uint32_t>(((nv - 1) * a.HV + 1) * 4));
            sB[tid] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, tid * a.HV * 4, 0, 0));
        }
        for (int u = tid; u < 2 * kC * kLA; u += kThrU) sAq[u] = 0.f;   // sAq, sAk are adjacent
    }
    __syncthreads();
    // ---- G: inclusive sums over the chunk's tokens, one key channel per thread
    for (int c = tid; c < K; c += kThrU) {
        float col[kC];
#pragma unroll
        for (int i = 0; i < kC; ++i) col[i] = sG[i * LK + c];
#pragma unroll
        for (int i = 1; i < kC; ++i) col[i] += col[i - 1];
#pragma unroll
        for (int i = 0; i < kC; ++i) sG[i * LK + c] = col[i];
    }
    __syncthreads();

    // ---- products.  Lane (x, kq): A operand row ri (reference rr), B operand
    // row cj (reference rc); reduction steps k0 + 4 kq + j.
    const int wave = tid >> 6, lane = tid & 63, x = lane & 15, kq = lane >> 4;
    {
        int ri, rr, cj, rc;
        if (wave == 0) {
            ri = 16 + x; rr = 15; cj = x; rc = 15;
        } else if (wave == 1) {
            ri = x < 8 ? 8 + x : 16 + x; rr = x < 8 ? 7 : 23;
            cj = x < 8 ? x : 8 + x; rc = rr;
        } else {
            const int o = 16 * (wave - 2);
            ri = o + x; rr = o + (x < 8 ? 3 : 11);
            cj = ri; rc = rr;
        }
        f32x4 aq = {0.f, 0.f, 0.f, 0.f}, ak = aq;
#pragma unroll 2
        for (int k0 = 0; k0 < K; k0 += 16) {
            const int c = k0 + 4 * kq;
            const f32x4 q4 = ld4(sQ + ri * LK + c), k4 = ld4(sK + ri * LK + c);
            const f32x4 g4 = ld4(sG + ri * LK + c), gr4 = ld4(sG + rr * LK + c);
            const f32x4 kc4 = ld4(sK + cj * LK + c), gc4 = ld4(sG + cj * LK + c), gcr4 = ld4(sG + rc * LK + c);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float er = ex2(g4[j] - gr4[j]), ec = ex2(gcr4[j] - gc4[j]);
                const float bk = kc4[j] * ec;
                aq = mma4(q4[j] * er, bk, aq);
                ak = mma4(k4[j] * er, bk, ak);
            }
        }
        // element j: tile row r = 4 kq + j, tile column x
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * kq + j;
            if (wave == 0) {
                sAq[(16 + r) * kLA + x] = aq[j];
                sAk[(16 + r) * kLA + x] = ak[j];
            } else if ((r < 8) == (x < 8)) {
                if (wave == 1) {
                    const int i = r < 8 ? 8 + r : 16 + r, jj = x < 8 ? x : 8 + x;
                    sAq[i * kLA + jj] = aq[j];
                    sAk[i * kLA + jj] = ak[j];
                } else {
                    const int o = 16 * (wave - 2);
                    if (x <= r) sAq[(o + r) * kLA + o + x] = aq[j];
                    if (x < r) sAk[(o + r) * kLA + o + x] = ak[j];
                }
            }
        }
    }
    __syncthreads();

    // ---- outputs
    uint16_t *img = a.img + (static_cast<size_t>(bhv) * a.NC + ch) * kUnbImgElems;
    if (wave < 2) {
        // T_blk = (I + diag(beta) A_blk)^-1, A_blk the strictly lower diagonal
        // block `wave` of A_kk.  Row i of T solves x^T (I + A_blk) = e_i^T,
        // swept k = 15 .. 1: once x_k is final it is removed from every earlier
        // column.  Lane = (row i, quarter q) holds x_{4q..4q+3}; x_k comes from
        // its row's lane k / 4.
        const int o = 16 * wave, i = lane >> 2, q = lane & 3;
        float xv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) xv[e] = (4 * q + e == i) ? 1.f : 0.f;
#pragma unroll
        for (int kk = 15; kk >= 1; --kk) {
            const f32x4 av = ld4(sAk + (o + kk) * kLA + o + 4 * q);
            const float xk = quad_bcast(xv[kk % 4], kk / 4) * sB[o + kk];
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[e] -= av[e] * xk;
        }
        uint32_t hw[2], lw[2];
        split2(xv[0], xv[1], hw[0], lw[0]);
        split2(xv[2], xv[3], hw[1], lw[1]);
        uint16_t *dst = img + 2560 + wave * 512 + i * 16 + 4 * q;
        *reinterpret_cast<uint2 *>(dst) = make_uint2(hw[0], hw[1]);
        *reinterpret_cast<uint2 *>(dst + 256) = make_uint2(lw[0], lw[1]);
    } else if (wave == 2) {
        // -A21 = -diag(beta) A_kk(rows 16..31, columns 0..15)
        const int i = lane >> 2, q = lane & 3;
        const f32x4 av = ld4(sAk + (16 + i) * kLA + 4 * q);
        const float nb = -sB[16 + i];
        uint32_t hw[2], lw[2];
        split2(nb * av[0], nb * av[1], hw[0], lw[0]);
        split2(nb * av[2], nb * av[3], hw[1], lw[1]);
        uint16_t *dst = img + 2048 + i * 16 + 4 * q;
        *reinterpret_cast<uint2 *>(dst) = make_uint2(hw[0], hw[1]);
        *reinterpret_cast<uint2 *>(dst + 256) = make_uint2(lw[0], lw[1]);
    } else {
        // A_qk row i, positions 16 hh .. 16 hh + 15: position p = 8 g + 4 h' + e
        // holds column 16 h' + 4 g + e
        const int i = lane >> 1, hh = lane & 1;
        uint32_t hw[8], lw[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            float v2[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int p = 16 * hh + 2 * w + s;
                const int c = 16 * ((p >> 2) & 1) + 4 * (p >> 3) + (p & 3);
                v2[s] = sAq[i * kLA + c];
            }
            split2(v2[0], v2[1], hw[w], lw[w]);
        }
        uint16_t *dst = img + i * 32 + 16 * hh;
        *reinterpret_cast<uint4 *>(dst) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4 *>(dst + 8) = make_uint4(hw[4], hw[5], hw[6], hw[7]);
        *reinterpret_cast<uint4 *>(dst + 1024) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        *reinterpret_cast<uint4 *>(dst + 1032) = make_uint4(lw[4], lw[5], lw[6], lw[7]);
    }
}

template <int K>
hipError_t launch_prep_k(const UnbPrepArgs &u, long blocks, hipStream_t stream) {
    hipLaunchKernelGGL(unb_prep_kernel<K>, dim3(static_cast<unsigned>(blocks)), dim3(kThrU), 0, stream, u);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_unbounded_prefill(const PrefillArgs &a, uint16_t *img, hipStream_t stream) {
    if (!a.bf16 || a.snap || a.A_log || a.bwd || a.t_off || a.Tseq) return hipErrorInvalidValue;
    if (a.B == 0 || a.T == 0) return hipSuccess;
    UnbPrepArgs u{};
    u.q = static_cast<const uint16_t *>(a.q);
    u.k = static_cast<const uint16_t *>(a.k);
    u.g = a.g; u.beta = a.beta; u.img = img;
    u.T = a.T; u.H = a.H; u.HV = a.HV; u.NC = (a.T + kC - 1) / kC;
    const long blocks = static_cast<long>(a.B) * a.HV * u.NC;
    hipError_t e = a.K == 32 ? launch_prep_k<32>(u, blocks, stream)
                 : a.K == 64 ? launch_prep_k<64>(u, blocks, stream)
                 : a.K == 128 ? launch_prep_k<128>(u, blocks, stream)
                              : hipErrorInvalidValue;
    if (e != hipSuccess) return e;
    PrefillArgs m = a;
    m.unb = true;
    m.img = img;
    return launch_prefill_bf16(m, stream);
}

}  // namespace kda
