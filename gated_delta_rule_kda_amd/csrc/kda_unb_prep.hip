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
// Workgroups of 4 waves, each taking chunks in turn with the next chunk's
// loads in flight.  q, k go to LDS as loaded, G as fp32;
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
// Workgroup barrier for LDS hand-offs that, unlike __syncthreads(), does not
// wait for outstanding global loads: the next chunk's prefetch stays in flight
// across it (each register is waited for at its first use).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, static_cast<int>(bytes), 0x00020000);
}

struct UnbPrepArgs {
    const uint16_t *q, *k;      // [B,T,H,K] bf16
    const float *g, *beta;      // [B,T,HV,K], [B,T,HV]
    uint16_t *img;              // [B,HV,NC,kUnbImgElems] bf16
    int B, T, H, HV, NC;
};

template <int K>
struct UPlan {
    static constexpr int LK = K + 4;    // fp32 rows of G
    static constexpr int LKB = K + 8;   // bf16 rows of q, k
    static constexpr int oQ = 0;                    // bf16 [C][LKB] q (as loaded)
    static constexpr int oK = oQ + kC * LKB / 2;    // bf16 [C][LKB] k
    static constexpr int oG = oK + kC * LKB / 2 > 2 * kC * kLA ? oK + kC * LKB / 2 : 2 * kC * kLA;
                                                    // fp32 [C][LK] G (base 2, floored g)
    static constexpr int oB = oG + kC * LK;         // fp32 [C] beta
    static constexpr int floats = oB + kC;          // (offsets in floats)
    // A_qk and A_kk (without beta), fp32 [C][kLA] each, over q and k (and
    // below G) once the products have read them
    static constexpr int oAq = oQ;
    static constexpr int oAk = oAq + kC * kLA;
    static_assert(2 * kC * kLA <= oG, "A arrays must fit below G");
};

// x of lane l - D within the lane's row of 16 (DPP row_shr:D)
template <int D>
__device__ __forceinline__ float row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + D, 0xf, 0xf, false));
}

// At most 168 VGPRs (three waves per SIMD; the compiler takes 159): three
// workgroups per CU instead of the two that 172 allowed, their LDS 103 KB
// (the pass 3 % faster on the HV96 workload; a budget of 128 spills).
template <int K>
__global__ __launch_bounds__(kThrU, 3) void unb_prep_kernel(UnbPrepArgs a) {
    using P = UPlan<K>;
    constexpr int LK = P::LK, LKB = P::LKB;
    __shared__ __attribute__((aligned(16))) float sm[P::floats];
    uint16_t *sQ = reinterpret_cast<uint16_t *>(sm + P::oQ), *sK = reinterpret_cast<uint16_t *>(sm + P::oK);
    float *sG = sm + P::oG;
    float *sAq = sm + P::oAq, *sAk = sm + P::oAk, *sB = sm + P::oB;

    const int tid = static_cast<int>(threadIdx.x);
    const long total = static_cast<long>(a.B) * a.HV * a.NC;
    const int gs = a.HV * K, qs = a.H * K;
    // Items in the order (b, chunk, value head), so that the workgroups running
    // at a time read whole token rows of every head (DRAM pages stay open).
    // Each workgroup takes items blockIdx.x, + gridDim.x, ...; the next
    // chunk's q, k, g and beta are loaded into registers while the current
    // one is processed.  Rows past the sequence end read 0 (an exact no-op
    // token), and so does everything of an item past the last.
    // g: thread (channel c, part p) holds rows p R .. p R + R - 1 of column c,
    // the NP parts of a column in consecutive lanes.
    constexpr int NP = kThrU / K, R = kC / NP;
    static_assert(NP * K == kThrU && (NP == 2 || NP == 4 || NP == 8), "g parts per column");
    constexpr int Q8 = kC * K / 8, QPT = (Q8 + kThrU - 1) / kThrU;  // 16-byte units of q, k per thread
    const int gc = tid / NP, gp = tid % NP;
    float pg[R];
    u32x4 pq[QPT], pk[QPT];
    uint32_t pb = 0;
    auto load = [&](long item) {
        long it = item < total ? item : 0;
        const int hv = static_cast<int>(it % a.HV), bch = static_cast<int>(it / a.HV);
        const int ch = bch % a.NC, b = bch / a.NC, h = hv / (a.HV / a.H);
        const int t0 = ch * kC;
        const int nv = item < total ? min(kC, a.T - t0) : 0;
        const size_t tb = static_cast<size_t>(b) * a.T + t0;
        const auto rg = make_rsrc(a.g + (tb * a.HV + hv) * K, nv ? static_cast<uint32_t>(((nv - 1) * gs + K) * 4) : 0u);
        const auto rq = make_rsrc(a.q + (tb * a.H + h) * K, nv ? static_cast<uint32_t>(((nv - 1) * qs + K) * 2) : 0u);
        const auto rk = make_rsrc(a.k + (tb * a.H + h) * K, nv ? static_cast<uint32_t>(((nv - 1) * qs + K) * 2) : 0u);
#pragma unroll
        for (int r = 0; r < R; ++r)
            pg[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, ((gp * R + r) * gs + gc) * 4, 0, 0));
#pragma unroll
        for (int j = 0; j < QPT; ++j) {
            const int u = tid + j * kThrU, row = u / (K / 8), c = (u % (K / 8)) * 8;   // u >= Q8: row >= C, reads 0
            pq[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, (row * qs + c) * 2, 0, 0);
            pk[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, (row * qs + c) * 2, 0, 0);
        }
        if (tid < kC) {
            const auto rb = make_rsrc(a.beta + tb * a.HV + hv, nv ? static_cast<uint32_t>(((nv - 1) * a.HV + 1) * 4) : 0u);
            pb = __builtin_amdgcn_raw_buffer_load_b32(rb, tid * a.HV * 4, 0, 0);
        }
    };
    // The loaded registers to LDS: q, k as loaded; G = the inclusive sums of
    // floored g (base 2) over the chunk's tokens (within the thread's rows,
    // then over the parts before it by DPP).
    auto stage = [&]() {
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            run += fmaxf(pg[r], kUnbFloor) * kLog2e;
            pg[r] = run;
        }
        float incl = run;
        if constexpr (NP > 1) { const float y = row_shr<1>(incl); if (gp >= 1) incl += y; }
        if constexpr (NP > 2) { const float y = row_shr<2>(incl); if (gp >= 2) incl += y; }
        if constexpr (NP > 4) { const float y = row_shr<4>(incl); if (gp >= 4) incl += y; }
        const float before = incl - run;
#pragma unroll
        for (int r = 0; r < R; ++r) sG[(gp * R + r) * LK + gc] = pg[r] + before;
#pragma unroll
        for (int j = 0; j < QPT; ++j) {
            const int u = tid + j * kThrU, row = u / (K / 8), c = (u % (K / 8)) * 8;
            if (u < Q8) {
                *reinterpret_cast<u32x4 *>(sQ + row * LKB + c) = pq[j];
                *reinterpret_cast<u32x4 *>(sK + row * LKB + c) = pk[j];
            }
        }
        if (tid < kC) sB[tid] = __uint_as_float(pb);
    };
    // 4 bf16 of a row of q or k as fp32
    auto ldb4 = [](const uint16_t *p) {
        const uint2 w = *reinterpret_cast<const uint2 *>(p);
        return f32x4{bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y)};
    };

    load(blockIdx.x);
    for (long item = blockIdx.x; item < total; item += gridDim.x) {
        lds_barrier();   // the previous item's outputs have read the LDS
        stage();
        load(item + gridDim.x);
        lds_barrier();

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
            if (wave >= 2) {
                // F3: both operands from the same rows and reference rows
#pragma unroll 2
                for (int k0 = 0; k0 < K; k0 += 16) {
                    const int c = k0 + 4 * kq;
                    const f32x4 q4 = ldb4(sQ + ri * LKB + c), k4 = ldb4(sK + ri * LKB + c);
                    const f32x4 g4 = ld4(sG + ri * LK + c), gr4 = ld4(sG + rr * LK + c);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float er = ex2(g4[j] - gr4[j]), ec = ex2(gr4[j] - g4[j]);
                        const float bk = k4[j] * ec;
                        aq = mma4(q4[j] * er, bk, aq);
                        ak = mma4(k4[j] * er, bk, ak);
                    }
                }
            } else {
#pragma unroll 2
                for (int k0 = 0; k0 < K; k0 += 16) {
                    const int c = k0 + 4 * kq;
                    const f32x4 q4 = ldb4(sQ + ri * LKB + c), k4 = ldb4(sK + ri * LKB + c);
                    const f32x4 g4 = ld4(sG + ri * LK + c), gr4 = ld4(sG + rr * LK + c);
                    const f32x4 kc4 = ldb4(sK + cj * LKB + c), gc4 = ld4(sG + cj * LK + c);
                    const f32x4 gcr4 = ld4(sG + rc * LK + c);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float er = ex2(g4[j] - gr4[j]), ec = ex2(gcr4[j] - gc4[j]);
                        const float bk = kc4[j] * ec;
                        aq = mma4(q4[j] * er, bk, aq);
                        ak = mma4(k4[j] * er, bk, ak);
                    }
                }
            }
            // element j: tile row r = 4 kq + j, tile column x.  Every entry of
            // A_qk and of the blocks of A_kk the outputs read is written, zeros
            // included: A_qk's upper right tile by F1, the entries above the
            // diagonal of each 16x16 diagonal block by F3.
            lds_barrier();   // q and k are read: A goes over them
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * kq + j;
                if (wave == 0) {
                    sAq[(16 + r) * kLA + x] = aq[j];
                    sAk[(16 + r) * kLA + x] = ak[j];
                    sAq[r * kLA + 16 + x] = 0.f;
                } else if (wave == 1) {
                    if ((r < 8) == (x < 8)) {
                        const int i = r < 8 ? 8 + r : 16 + r, jj = x < 8 ? x : 8 + x;
                        sAq[i * kLA + jj] = aq[j];
                        sAk[i * kLA + jj] = ak[j];
                    }
                } else {
                    const int o = 16 * (wave - 2), at = (o + r) * kLA + o + x;
                    if ((r < 8) == (x < 8)) {
                        sAq[at] = x <= r ? aq[j] : 0.f;
                        sAk[at] = x < r ? ak[j] : 0.f;
                    } else if (r < 8) {
                        sAq[at] = 0.f;
                        sAk[at] = 0.f;
                    }
                }
            }
        }
        lds_barrier();

        // ---- outputs
        uint16_t *img;
        {
            const int hv = static_cast<int>(item % a.HV), bch = static_cast<int>(item / a.HV);
            img = a.img + ((static_cast<size_t>(bch / a.NC) * a.HV + hv) * a.NC + bch % a.NC) * kUnbImgElems;
        }
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
            // (runs of four: positions 16 hh + 4 m .. + 3 hold columns
            // 8 hh + {0, 16, 4, 20}[m] .. + 3)
            const int i = lane >> 1, hh = lane & 1;
            f32x4 run[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) run[m] = ld4(sAq + i * kLA + 8 * hh + 16 * (m & 1) + 4 * (m >> 1));
            uint32_t hw[8], lw[8];
#pragma unroll
            for (int w = 0; w < 8; ++w) split2(run[w >> 1][2 * (w & 1)], run[w >> 1][2 * (w & 1) + 1], hw[w], lw[w]);
            uint16_t *dst = img + i * 32 + 16 * hh;
            *reinterpret_cast<uint4 *>(dst) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            *reinterpret_cast<uint4 *>(dst + 8) = make_uint4(hw[4], hw[5], hw[6], hw[7]);
            *reinterpret_cast<uint4 *>(dst + 1024) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
            *reinterpret_cast<uint4 *>(dst + 1032) = make_uint4(lw[4], lw[5], lw[6], lw[7]);
        }
    }
}

// Workgroups: as many as are resident on the device at once, at most one per
// chunk.
template <int K>
hipError_t launch_prep_k(const UnbPrepArgs &u, long items, hipStream_t stream) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, unb_prep_kernel<K>, kThrU, 0);
    if (e != hipSuccess) return e;
    const long resident = static_cast<long>(cus) * (per_cu > 0 ? per_cu : 1);
    const long blocks = items < resident ? items : resident;
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
    u.B = a.B; u.T = a.T; u.H = a.H; u.HV = a.HV; u.NC = (a.T + kC - 1) / kC;
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
