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
// with M the [K x V] state at the chunk start.  The state-side products use
// q Gamma = (q e1) 2^{G_r} and k Gamma = (k e1) 2^{G_r}: the per-channel factor
// 2^{G_r} >= 2^-116 scales the rows of M instead, so q e1 and k e1 serve both
// the in-chunk matrices and the state products.
//
// The solve is blocked on 16 rows: U1 = T11 R1, U2 = T22 (R2 - A21 U1), where
// T11, T22 are the inverses of the two 16x16 diagonal blocks of I + A_kk
// (fp32 forward substitution, one column per lane).  It runs in the carry
// waves on v_mfma_f32_16x16x16_bf16, whose B operand layout (four consecutive
// reduction rows per lane group) is exactly the accumulator layout of the
// previous product, so the three products chain without leaving registers.
//
// Organisation: one workgroup of 8 waves per (b, hv, V-tile of VT columns).
// Wave w and wave w + 4 share one SIMD; a single wave issues at most one VALU
// instruction every four cycles, so the VALU-heavy operand pass is spread over
// all eight waves and the MFMA chains of the carry interleave with it.
//  * carry waves 0..3 hold the state: carry wave w owns NG blocks of 16
//    columns of M (all K rows) in MFMA accumulators for the whole sequence.
//    M is also used directly as the B operand of the 32-deep MFMAs: the
//    reduction index may be permuted as long as both operands agree, so lane
//    group g takes rows {4g..4g+3} of one 16-row tile and of the next; A
//    operands are read from LDS in that order.
//  * operand pass: each operand wave owns a slice of K columns and all 32 rows
//    of the chunk (so the cumulative sums never leave the wave) and turns q, k,
//    g, beta of the next chunk into MFMA operands (exponentials, hi/lo splits).
//  * waves 4 and 5 then form A_kk's diagonal-block inverses T11, T22 (fp32,
//    one block per wave, at raised wave priority), wave 6 the diagonal A_qk
//    tiles, wave 7 A_qk(1,0) and -A21.
//  * The carry holds the state as N = 2^{G_r} (.) M, the form the state
//    products read, and the update takes (k e2)^T U with the row factors
//    2^{G_last - G_r} and the next chunk's 2^{G_r} applied after it, so the
//    operand pass stores k e2 once for A_qk, A_kk and the update.
//  * Pipeline (per chunk n; two barriers):
//      P1  carry: R, solve, O (-> HBM) of chunk n (U stays in registers)
//          all:   operand pass of chunk n+1, prefetch of chunk n+2
//      P2  carry: state update of chunk n, (q Gamma) M and (k Gamma) M of chunk n+1
//          waves 4..7: T11, T22, A_qk, -A21 of chunk n+1
//    Operands written in P1 of chunk n+1 while the carry still reads chunk n's
//    ((k e2)^T, 2^{G_last - G_r}, beta) are double-buffered in LDS; everything
//    else is single.
//  * The three terms of a split product accumulate in place where independent
//    products can be issued between them, and operand fragments are read
//    ahead, so chains run at MFMA throughput instead of MFMA and LDS latency.
//  * Precision: operands whose bf16 rounding would matter are split into
//    hi + lo bf16 and multiplied as hi*hi + hi*lo + lo*hi: A_qk, (q Gamma) M
//    (q e1 and 2^{G_r} M both split), the three solve products, A_qk U and
//    (k e2)^T U.  A_kk and (k Gamma) M use single bf16 operands.  Emulating this policy against the fp64 oracle over
//    decay ranges from g ~ -5 to g ~ -0.05 and initial states up to
//    N(0, 0.3^2) keeps the output within 3e-3 RMS beyond its own bf16 rounding
//    and the final state within 3e-3 RMS.

//  * Fused layer stages (GATED, OG instantiations, for kda_chunk_fwd_gated):
//    GATED reads the gate pre-activation z where g would be and beta logits,
//    and the operand pass forms g = lb sigmoid(exp(A_log)(z + dt_bias)) (the
//    bounded_gate of the page "metrale_model_weights/kimi_k3_host/kda.rs") and
//    beta = sigmoid(logit) before the cumulative sums, so g never goes through
//    HBM.  OG (one workgroup per whole V row) applies full_rank_output_gate of
//    the same page, y = sigmoid(gate) o / sqrt(mean(o^2) + eps), to the bf16
//    rows of o as the helper waves store them: the 16 lanes holding a row of
//    128 values sum its squares by DPP within their row of lanes.
//  * The chunked backward's forward pass (BWD, a snapshot instantiation):
//    no o; U of every chunk goes to the workspace from the carry's registers
//    (fp32), and the call may cover a sub-range of the
//    sequences (t_off, Tseq) starting from a state with its own batch stride.
//  * Gates without a lower bound (UNB, for kda_chunk_fwd_unbounded): A_qk,
//    -A21, T11 and T22 come from the chunk-parallel pass of kda_unb_prep.hip
//    (an image per chunk in HBM, the layouts of sAqk, sA21 and sTi), which
//    waves 4..7 copy into LDS where the other instantiations form them.  The
//    operand pass applies the same per-token floor to g (kUnbFloor) and uses
//    forward-only factors, each <= 1: q Gamma and k Gamma with Gamma_i =
//    2^{G_i}, and k Lambda with Lambda_i = 2^{G_last - G_i} for the update.
//    The carry holds M itself: M' = Gamma_last (.) M + (k Lambda)^T U.

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kC = 32;
constexpr int kNW = 8;
constexpr int kNT = kNW * 64;
constexpr int kMaxCW = 4;          // carry waves 0..3 at most
constexpr int kRef = 15;
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// (a, b) -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pk(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// A 32-bit constant the compiler cannot see through, kept in an SGPR.  The bf16
// pairs below go to v_dot2c_f32_bf16 this way: as an inline constant the pair
// (-1, 0) is encoded as the fp32 constant -1.0, whose bits the instruction reads
// as the pair (0, -1).
__device__ __forceinline__ bf16x2 sgpr_pair(uint32_t bits) {
    asm("" : "+s"(bits));
    return __builtin_bit_cast(bf16x2, bits);
}
// a - (low bf16 of w), b - (high bf16 of w) in one v_dot2c_f32_bf16 each: the
// products with -1 and 0 are exact and the difference of a and its own bf16
// rounding is representable, so the result is exact.
__device__ __forceinline__ float minus_lo(uint32_t w, float a) {
    return __builtin_amdgcn_fdot2_f32_bf16(sgpr_pair(0x0000bf80u), __builtin_bit_cast(bf16x2, w), a, false);
}
__device__ __forceinline__ float minus_hi(uint32_t w, float b) {
    return __builtin_amdgcn_fdot2_f32_bf16(sgpr_pair(0xbf800000u), __builtin_bit_cast(bf16x2, w), b, false);
}
// hi = bf16(a, b), lo = bf16(a - hi_a, b - hi_b): four instructions per pair
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = pk(a, b);
    lo = pk(minus_lo(hi, a), minus_hi(hi, b));
}
__device__ __forceinline__ void split4(const f32x4 &x, bf16x4 &hi, bf16x4 &lo) {
    uint32_t h[2], l[2];
    split2(x[0], x[1], h[0], l[0]);
    split2(x[2], x[3], h[1], l[1]);
    hi = __builtin_bit_cast(bf16x4, h);
    lo = __builtin_bit_cast(bf16x4, l);
}
__device__ __forceinline__ void st_word(__bf16 *p, uint32_t w) { *reinterpret_cast<uint32_t *>(p) = w; }
// x of lane l - N within the lane's row of 16 (DPP row_shr:N), 0 for l % 16 < N
template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf, false));
}
// Sum of x over aligned groups of N lanes (N = 2, 4, 8 or 16), in every lane
// of the group: swap neighbours, then pairs, then the two quads of each half
// row, then the halves (DPP; a fixed order, the same result on every run).
template <int N>
__device__ __forceinline__ float rowN_sum(float x) {
    static_assert(N == 2 || N == 4 || N == 8 || N == 16, "DPP groups");
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xb1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
    if constexpr (N >= 4)
        x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4e, 0xf, 0xf, false));  // quad_perm 2,3,0,1
    if constexpr (N >= 8)
        x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false)); // row_half_mirror
    if constexpr (N >= 16)
        x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xf, 0xf, false)); // row_mirror
    return x;
}
// 1 / (1 + 2^t): the logistic function of -t ln 2 (hardware exponential and
// reciprocal; 0 for t -> +inf, 1 for t -> -inf)
__device__ __forceinline__ float inv1p_exp2(float t) { return __builtin_amdgcn_rcpf(1.0f + ex2(t)); }

// x of lane p of the lane's group of four (DPP quad_perm broadcast; p must
// fold to a constant)
__device__ __forceinline__ float quad_bcast(float x, int p) {
    const int v = __float_as_int(x);
    switch (p) {
    case 0: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x00, 0xf, 0xf, false));
    case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x55, 0xf, 0xf, false));
    case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xaa, 0xf, 0xf, false));
    default: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xff, 0xf, 0xf, false));
    }
}
// x of lane `src` (0..63) of the wave (ds_bpermute)
__device__ __forceinline__ float lane_value(int src, float x) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}
// NW consecutive packed words as one LDS store (NW in {1, 2, 4})
template <int NW>
__device__ __forceinline__ void st_words(__bf16 *p, const uint32_t (&w)[NW]) {
    if constexpr (NW == 4) {
        *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if constexpr (NW == 2) {
        *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
    } else {
        *reinterpret_cast<uint32_t *>(p) = w[0];
    }
}

// Raw buffer resource over `bytes` bytes from `p`: out-of-range loads read 0
// and out-of-range stores are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, static_cast<int>(bytes), 0x00020000);
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
// Wait for this wave's LDS accesses (exchange between lanes of one wave).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int K>
struct Plan {
    static constexpr int LDK = K + 16;   // bf16 rows over K
    static constexpr int LDC = kC + 16;  // bf16 rows over C
    static constexpr int L16 = 16 + 8;   // bf16 rows of a 16x16 block
    static constexpr int LDT = 20;       // fp32 rows of a 16x16 block
    static constexpr int CPW = K / 16 > 4 ? K / 16 : 4;   // column pairs per operand wave
    static constexpr int NOW = K / (2 * CPW);             // operand waves (the last NOW waves)
    static constexpr int NRG = 64 / CPW;                  // row groups per operand wave
    static constexpr int RPG = kC / NRG;                  // rows per group
    static constexpr int oLk = 0;                                // [C][LDK]  k e1
    static constexpr int oLq = oLk + kC * LDK * 2;               // [2][C][LDK]  q e1 hi, lo
    static constexpr int oR = oLq + 2 * kC * LDK * 2;            // [2][C][LDK]  k e2 hi, lo
    static constexpr int oKbarT = oR + 2 * kC * LDK * 2;         // [2 buf][2][K][LDC]  (k e2)^T hi, lo
    static constexpr int oAqk = oKbarT + 4 * K * LDC * 2;        // [2][C][LDC]  A_qk hi, lo
    static constexpr int oA21 = oAqk + 2 * kC * LDC * 2;         // [2][16][L16]  -A21 hi, lo
    static constexpr int oTi = oA21 + 2 * 16 * L16 * 2;          // [2 blk][2][16][L16]  T11, T22
    static constexpr int oPl = oTi + 4 * 16 * L16 * 2;           // fp32 [2 buf][K]  2^{G_last - G_r}
    static constexpr int oPr = oPl + 2 * K * 4;                  // fp32 [K]  2^{G_r}
    static constexpr int oBeta = oPr + K * 4;                    // fp32 [2 buf][C]
    static constexpr int oTs = oBeta + 2 * kC * 4;               // fp32 [2 blk][16][LDT]  A_blk
    static constexpr int oStage = oTs + 2 * 16 * LDT * 4;        // bf16 [2][C][VT + 8]  o, v of a chunk
    static constexpr int bytes = oStage;                         // plus stage_bytes(VT)
    static constexpr int stage_bytes(int VT) { return 2 * kC * (VT + 8) * 2; }
};

// SNAP: the variant that also writes prefix snapshots of the state (a
// separate instantiation, so that the plain path carries none of its code).
template <int K, int VT, bool SNAP, bool GATED, bool OG, bool BWD, bool UNB>
__global__ __launch_bounds__(kNT, 1) void prefill_bf16_kernel(PrefillArgs a) {
    static_assert(!OG || !SNAP, "the output gate is built for the plain prefill only");
    static_assert(!BWD || (SNAP && !GATED && !OG), "the backward's forward pass is a snapshot variant");
    static_assert(!UNB || (!SNAP && !GATED && !OG && !BWD), "the unbounded gate is built for the plain prefill");
    using L = Plan<K>;
    static_assert(L::bytes + L::stage_bytes(VT) <= 160 * 1024, "LDS plan exceeds 160 KB");
    constexpr int LDO = VT + 8;   // bf16 rows of the o staging tile
    constexpr int LDK = L::LDK, LDC = L::LDC, L16 = L::L16, LDT = L::LDT;
    constexpr int CPW = L::CPW, NOW = L::NOW, NRG = L::NRG, RPG = L::RPG;
    constexpr int KT = K / 16, KS = K / 32;
    constexpr int NCW = VT / 16 < kMaxCW ? VT / 16 : kMaxCW;   // carry waves
    constexpr int NG = VT / (16 * NCW);                          // 16-column blocks per carry wave
    static_assert(NG * NCW * 16 == VT, "V tile must split evenly over the carry waves");
    static_assert(NOW * 2 * CPW == K && NOW <= kNW && NOW >= 4, "operand waves must cover K");
    static_assert(RPG >= 2 && RPG % 2 == 0 && (kRef + 1) % RPG == 0,
                  "row groups must pair rows and align with the reference row");

    // [C][LDK] operand arrays: element (i, c) sits in 8-column group (c / 8) XOR
    // (XS if i >= 16).  With the K + 16 row pitch the MFMA fragment reads (16
    // consecutive rows x 4 groups) are free of LDS bank conflicts, and the
    // operand pass's 32-bit stores -- whose 32-lane halves hold row groups of
    // both 16-row halves of the chunk, see row_base -- conflict only pairwise,
    // the least their column pattern allows (each measured on the device).
    constexpr int XS = K >= 64 ? 4 : 2;
    auto sw = [](int i, int c) { return i * LDK + ((((c >> 3) ^ (((i >> 4) & 1) * XS)) << 3) | (c & 7)); };
    // Within every block of 32 reduction indices (K columns, or tokens of a
    // chunk) the operands are stored in the MFMA's permuted order: index
    // 16h + 4g + e goes to 8g + 4h + e, so lane group g's fragment (rows
    // {4g..4g+3} of two 16-row tiles) is 16 contiguous bytes, one LDS read.
    auto perm = [](int c) { return (c & ~31) | ((c & 12) << 1) | ((c & 16) >> 2) | (c & 3); };
    // (k e2)^T [K][LDC]: token position p of row kr sits in 8-token group
    // (p / 8) XOR ((kr / 4) % 4); with the C + 16 pitch the update's fragment
    // reads (16 rows x 4 groups) are then free of bank conflicts (measured).
    auto kb_at = [](int kr, int p) { return kr * LDC + ((((p >> 3) ^ ((kr >> 2) & 3)) << 3) | (p & 7)); };
    // First row of operand-pass row group q: the groups' two top index bits are
    // swapped, so that each 32-lane half of a wave (q < NRG / 2, q >= NRG / 2)
    // holds groups from both 16-row halves of the chunk, while the two or four
    // groups of one DPP row of 16 lanes stay consecutive rows.
    auto row_base = [](int q) {
        constexpr int hb = NRG / 2, nb = NRG / 4;
        return RPG * ((q & ~(hb | nb)) | ((q & hb) ? nb : 0) | ((q & nb) ? hb : 0));
    };

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __bf16 *sLk = reinterpret_cast<__bf16 *>(smem + L::oLk);
    __bf16 *sLq = reinterpret_cast<__bf16 *>(smem + L::oLq);
    __bf16 *sR = reinterpret_cast<__bf16 *>(smem + L::oR);
    __bf16 *sKbarT = reinterpret_cast<__bf16 *>(smem + L::oKbarT);
    __bf16 *sAqk = reinterpret_cast<__bf16 *>(smem + L::oAqk);
    __bf16 *sA21 = reinterpret_cast<__bf16 *>(smem + L::oA21);
    __bf16 *sTi = reinterpret_cast<__bf16 *>(smem + L::oTi);
    float *sPl = reinterpret_cast<float *>(smem + L::oPl);
    float *sPr = reinterpret_cast<float *>(smem + L::oPr);
    float *sBeta = reinterpret_cast<float *>(smem + L::oBeta);
    float *sTs = reinterpret_cast<float *>(smem + L::oTs);
    __bf16 *sO = reinterpret_cast<__bf16 *>(smem + L::oStage);
    __bf16 *sV = sO + kC * LDO;

    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int nvt = a.V / VT;
    // Workgroups are handed to the 8 XCDs round-robin (block i -> XCD i % 8),
    // each with its own L2.  Give every XCD a contiguous range of the logical
    // order (b, q/k head, value head, V tile), so the V tiles of one value head
    // (same q, k, g) and the value heads of one q/k head (same q, k) run on one
    // XCD at about the same time and share its L2.
    const int nblk = static_cast<int>(gridDim.x);
    const int blk = (nblk & 7) == 0 ? (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3)
                                    : static_cast<int>(blockIdx.x);
    const int vt_idx = blk % nvt;
    const int bhv = blk / nvt;
    const int b = bhv / a.HV, hv = bhv % a.HV;
    const int h = hv / (a.HV / a.H);
    const int v0 = vt_idx * VT;
    const int T = a.T;
    const int HV = a.HV, V = a.V;
    const int NC = (T + kC - 1) / kC;
    const bool carry = wave < NCW;
    const bool opw = NOW == kNW || wave >= kNW - NOW;
    const int ow = wave - (kNW - NOW);   // operand wave index (valid when opw)
    // GATED: the gate of the lane's two columns as a base-2 exponent,
    // exp(-decay (z + dt_bias)) = 2^(gsl z + gof[c]) with decay = exp(A_log[hv])
    float gsl = 0.f, gof[2] = {0.f, 0.f};
    if constexpr (GATED) {
        if (opw) {
            const int f0 = ow * 2 * CPW + 2 * ((threadIdx.x & 63) % CPW);
            gsl = -expf(a.A_log[hv]) * kLog2e;
            gof[0] = gsl * a.dt_bias[hv * K + f0];
            gof[1] = gsl * a.dt_bias[hv * K + f0 + 1];
        }
    }

    const uint16_t *qg = static_cast<const uint16_t *>(a.q);
    const uint16_t *kg = static_cast<const uint16_t *>(a.k);
    const uint16_t *vg = static_cast<const uint16_t *>(a.v);
    uint16_t *og = static_cast<uint16_t *>(a.out);

    // ---- global memory: per-chunk buffer resources (base in SGPRs, 32-bit lane
    // offsets).  A resource covers exactly the valid rows of the chunk, so rows
    // past the end of the sequence load as zero and their stores are dropped; a
    // chunk past the end has an empty resource.  Prefetches are therefore issued
    // unconditionally, which keeps their registers out of loop-carried copies
    // that would wait for the loads.
    const size_t tok_b = static_cast<size_t>(b) * (a.Tseq ? a.Tseq : T) + a.t_off;
    const int g_stride = HV * K;             // elements per token
    const int qk_stride = a.H * K;
    const int v_stride = HV * V;
    auto rows_bytes = [&](int t0, int stride, int rowlen, int esz) -> uint32_t {
        const int nv = min(kC, T - t0);
        return nv > 0 ? static_cast<uint32_t>(((nv - 1) * stride + rowlen) * esz) : 0u;
    };

    // ======================= operand pass.  Lane = (row group rg, column pair
    // cp): columns f0, f0 + 1 of rows rg*RPG .. rg*RPG + RPG - 1.
    float2 pf_g[RPG];
    uint32_t pf_q[RPG], pf_k[RPG];
    float pf_b;
    auto load_prep = [&](int ch) {
        const int lane = opaque_tid() & 63, cp = lane % CPW, rg = lane / CPW;
        const int f0 = ow * 2 * CPW + 2 * cp;
        const int t0 = ch * kC;
        const size_t tb = tok_b + t0;
        const auto rgr = make_rsrc(a.g + (tb * HV + hv) * K, rows_bytes(t0, g_stride, K, 4));
        const auto rq = make_rsrc(qg + (tb * a.H + h) * K, rows_bytes(t0, qk_stride, K, 2));
        const auto rk = make_rsrc(kg + (tb * a.H + h) * K, rows_bytes(t0, qk_stride, K, 2));
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            const int i = row_base(rg) + r;
            const auto gg = __builtin_amdgcn_raw_buffer_load_b64(rgr, (i * g_stride + f0) * 4, 0, 0);
            pf_g[r] = make_float2(__uint_as_float(gg[0]), __uint_as_float(gg[1]));
            pf_q[r] = __builtin_amdgcn_raw_buffer_load_b32(rq, (i * qk_stride + f0) * 2, 0, 0);
            pf_k[r] = __builtin_amdgcn_raw_buffer_load_b32(rk, (i * qk_stride + f0) * 2, 0, 0);
        }
        if (wave == kNW - 1) {
            const auto rb = make_rsrc(a.beta + tb * HV + hv, rows_bytes(t0, HV, 1, 4));
            pf_b = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, (lane & (kC - 1)) * HV * 4, 0, 0));
        }
    };

    // operand pass 1a: take the prefetched registers, so that the next prefetch
    // can be issued into them before the cross-lane steps of pass 1b
    float gl[RPG][2];
    uint32_t qw[RPG], kw[RPG];
    float pl[2], og2[2];
    float gl2[2];   // UNB: G_last (base 2) of the lane's columns
    auto op1a = [&](int buf, int ch) {
        const int lane = opaque_tid() & 63;
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            gl[r][0] = pf_g[r].x;
            gl[r][1] = pf_g[r].y;
            qw[r] = pf_q[r];
            kw[r] = pf_k[r];
        }
        if (wave == kNW - 1 && lane < kC) {
            float bt = pf_b;
            // GATED: beta = sigmoid(logit); tokens past the end write nothing
            if constexpr (GATED) bt = ch * kC + lane < T ? inv1p_exp2(-bt * kLog2e) : 0.f;
            sBeta[buf * kC + lane] = bt;
        }
    };
    // operand pass 1b: cumulative sums of g (natural log units) within the row
    // group, then across the row groups, and the chunk's exponent offsets; the
    // prefetch and the carry work of the phase cover the cross-lane latency
    auto op1b = [&](int buf, int ch) {
        const int lane = opaque_tid() & 63, cp = lane % CPW, rg = lane / CPW;
        const int f0 = ow * 2 * CPW + 2 * cp;
        if constexpr (GATED) {
            // g = lb sigmoid(decay (z + dt_bias)); 0 (no decay) past the end
#pragma unroll
            for (int r = 0; r < RPG; ++r)
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    gl[r][c] = ch * kC + row_base(rg) + r < T
                                   ? a.lower_bound * inv1p_exp2(__builtin_fmaf(gl[r][c], gsl, gof[c]))
                                   : 0.f;
        }
        if constexpr (UNB) {
#pragma unroll
            for (int r = 0; r < RPG; ++r) {
                gl[r][0] = fmaxf(gl[r][0], kUnbFloor);
                gl[r][1] = fmaxf(gl[r][1], kUnbFloor);
            }
        }
#pragma unroll
        for (int r = 1; r < RPG; ++r) {
            gl[r][0] += gl[r - 1][0];
            gl[r][1] += gl[r - 1][1];
        }
        // sums over the row groups of one column pair (lanes cp, cp + CPW, ..):
        // an inclusive scan within each DPP row of 16 lanes (row_shr by CPW,
        // 2 CPW, ..; its row groups are consecutive rows), then the four row
        // totals in one round of ds_bpermute.  In row order the DPP rows come
        // 0, 2, 1, 3 (row_base); rows 0..15 of the chunk are DPP rows 0 and 2.
        const int drow = lane >> 4;
        float pr[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float sc = gl[RPG - 1][c];
            if constexpr (CPW <= 1) sc += row_shr<1>(sc);
            if constexpr (CPW <= 2) sc += row_shr<2>(sc);
            if constexpr (CPW <= 4) sc += row_shr<4>(sc);
            if constexpr (CPW <= 8) sc += row_shr<8>(sc);
            float rt[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) rt[j] = lane_value(16 * j + 16 - CPW + cp, sc);
            const float Gr = rt[0] + rt[2];
            const float Gl = Gr + (rt[1] + rt[3]);
            const float before = drow == 0 ? 0.f : drow == 2 ? rt[0] : drow == 1 ? Gr : Gr + rt[1];
            const float off = before + (sc - gl[RPG - 1][c]);    // rows before the group
            if constexpr (UNB) {
                pr[c] = 1.f;
                pl[c] = ex2(Gl * kLog2e);          // Gamma_last
                gl2[c] = Gl * kLog2e;
                og2[c] = off * kLog2e;
            } else {
                pr[c] = ex2(Gr * kLog2e);          // 2^{G_r}         >= 2^-116
                pl[c] = ex2((Gl - Gr) * kLog2e);   // 2^{G_last - G_r} in [2^-116, 1]
                og2[c] = (off - Gr) * kLog2e;
            }
        }
        if (rg == 0) {
            *reinterpret_cast<float2 *>(sPl + buf * K + f0) = make_float2(pl[0], pl[1]);
            if constexpr (!UNB) *reinterpret_cast<float2 *>(sPr + f0) = make_float2(pr[0], pr[1]);
        }
    };

    // operand pass 2: exponentials (base 2) and MFMA operands of one chunk
    auto op2 = [&](int buf) {
        const int lane = opaque_tid() & 63, cp = lane % CPW, rg = lane / CPW;
        const int f0 = ow * 2 * CPW + 2 * cp;
        uint32_t rh[RPG], rl[RPG];   // k e2 of the lane's rows, packed bf16 pairs (hi, lo)
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            const int i = row_base(rg) + r;
            const float qf[2] = {bf_lo(qw[r]), bf_hi(qw[r])};
            const float kf[2] = {bf_lo(kw[r]), bf_hi(kw[r])};
            float xlk[2], xlq[2], xr[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                // G_i - G_r (UNB: G_i, and the factors Gamma_i, Lambda_i)
                const float d = __builtin_fmaf(gl[r][c], kLog2e, og2[c]);
                const float e1 = ex2(d), e2 = UNB ? ex2(gl2[c] - d) : ex2(-d);
                xlk[c] = kf[c] * e1;
                xlq[c] = qf[c] * e1;
                xr[c] = kf[c] * e2;
            }
            uint32_t hi, lo;
            const int at = sw(i, perm(f0));
            st_word(sLk + at, pk(xlk[0], xlk[1]));
            split2(xlq[0], xlq[1], hi, lo);
            st_word(sLq + at, hi);
            st_word(sLq + kC * LDK + at, lo);
            split2(xr[0], xr[1], rh[r], rl[r]);
            if constexpr (!UNB) {
                st_word(sR + at, rh[r]);
                st_word(sR + kC * LDK + at, rl[r]);
            }
        }
        // (k e2)^T for the state update: the same bf16 halves, regrouped by
        // column (tokens 2w, 2w + 1 of column f0 + c in one word)
        uint32_t kbh[2][RPG / 2], kbl[2][RPG / 2];
#pragma unroll
        for (int w = 0; w < RPG / 2; ++w) {
            kbh[0][w] = __builtin_amdgcn_perm(rh[2 * w + 1], rh[2 * w], 0x05040100u);
            kbh[1][w] = __builtin_amdgcn_perm(rh[2 * w + 1], rh[2 * w], 0x07060302u);
            kbl[0][w] = __builtin_amdgcn_perm(rl[2 * w + 1], rl[2 * w], 0x05040100u);
            kbl[1][w] = __builtin_amdgcn_perm(rl[2 * w + 1], rl[2 * w], 0x07060302u);
        }
        __bf16 *kb_buf = sKbarT + buf * 2 * K * LDC;
        // runs of four tokens stay contiguous under the permutation
        constexpr int RUN = RPG < 4 ? RPG : 4;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int q = 0; q < RPG / RUN; ++q) {
                const int at = kb_at(f0 + c, perm(row_base(rg) + q * RUN));
                uint32_t wh[RUN / 2], wl[RUN / 2];
#pragma unroll
                for (int w = 0; w < RUN / 2; ++w) {
                    wh[w] = kbh[c][q * RUN / 2 + w];
                    wl[w] = kbl[c][q * RUN / 2 + w];
                }
                st_words<RUN / 2>(kb_buf + at, wh);
                st_words<RUN / 2>(kb_buf + K * LDC + at, wl);
            }
    };

    // ======================= waves 4..7: A_qk (3-term), -A21, T11, T22
    // A_qk tile (rt, ct): independent accumulators for the three terms
    auto aqk_tile = [&](int rt, int ct) {
        const int lane = opaque_tid() & 63, lr = lane & 15, lg = lane >> 4;
        f32x4 hh = {0.f, 0.f, 0.f, 0.f}, hl = hh, lh = hh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int kk = ks * 32 + lg * 8;
            const int pa = sw(rt * 16 + lr, kk), pb = sw(ct * 16 + lr, kk);
            const bf16x8 ah = ld8(sLq + pa);
            const bf16x8 al = ld8(sLq + kC * LDK + pa);
            const bf16x8 bh = ld8(sR + pb);
            const bf16x8 bl = ld8(sR + kC * LDK + pb);
            hh = mfma(ah, bh, hh);
            hl = mfma(ah, bl, hl);
            lh = mfma(al, bh, lh);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = rt * 16 + lg * 4 + r, j = ct * 16 + lr;
            const float x = (j <= i) ? (hh[r] + (hl[r] + lh[r])) : 0.f;
            const __bf16 hi = bf(x);
            sAqk[i * LDC + perm(j)] = hi;
            sAqk[kC * LDC + i * LDC + perm(j)] = bf(x - fl(hi));
        }
    };
    // raw A_kk tile (rt, ct) = (k e1)(k e2)^T with single bf16 operands (beta not applied)
    auto akk_tile = [&](int rt, int ct) {
        const int lane = opaque_tid() & 63, lr = lane & 15, lg = lane >> 4;
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int kk = ks * 32 + lg * 8;
            const bf16x8 x = ld8(sLk + sw(rt * 16 + lr, kk)), y = ld8(sR + sw(ct * 16 + lr, kk));
            if (ks & 1) acc1 = mfma(x, y, acc1);
            else acc0 = mfma(x, y, acc0);
        }
        return acc0 + acc1;
    };
    auto phaseAT = [&](int buf) {
        const int lane = opaque_tid() & 63, lr = lane & 15, lg = lane >> 4;
        const float *beta = sBeta + buf * kC;
        if (wave == 4 || wave == 5) {
            // the inverses are the longest path of this phase: this wave's
            // LDS and VALU instructions go ahead of the others' while it runs
            __builtin_amdgcn_s_setprio(3);
            // T_blk = (I + A_blk)^-1 for diagonal block blk = wave - 4 of A_kk, in
            // fp32.  A_blk goes to LDS row-major; row i of T solves
            // x^T (I + A_blk) = e_i^T, swept k = 15 .. 1: once x_k is final it is
            // removed from every earlier column.  Lane = (row i, quarter q) holds
            // x_{4q..4q+3}; x_k comes from its row's lane k / 4 by DPP, and the
            // strictly lower A_blk (zero for j >= k) makes the update uniform.
            // The finished quarter rows are split and stored as they stand.
            const int blk = wave - 4;
            float *sA = sTs + blk * 16 * LDT;
            {
                const f32x4 acc = akk_tile(blk, blk);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = lg * 4 + r;
                    sA[i * LDT + lr] = (lr < i) ? beta[16 * blk + i] * acc[r] : 0.f;
                }
            }
            wave_lds_sync();
            const int i = lane >> 2, q = lane & 3;
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (4 * q + e == i) ? 1.f : 0.f;
#pragma unroll
            for (int k = 15; k >= 1; --k) {
                const f32x4 av = *reinterpret_cast<const f32x4 *>(sA + k * LDT + 4 * q);
                const float xk = quad_bcast(x[k % 4], k / 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] -= av[e] * xk;
            }
            uint32_t hw[2], lw[2];
            split2(x[0], x[1], hw[0], lw[0]);
            split2(x[2], x[3], hw[1], lw[1]);
            __bf16 *dst = sTi + blk * 2 * 16 * L16 + i * L16 + 4 * q;
            *reinterpret_cast<uint2 *>(dst) = make_uint2(hw[0], hw[1]);
            *reinterpret_cast<uint2 *>(dst + 16 * L16) = make_uint2(lw[0], lw[1]);
            __builtin_amdgcn_s_setprio(0);
        } else if (wave == 6) {
            aqk_tile(0, 0);
            aqk_tile(1, 1);
        } else if (wave == 7) {
            aqk_tile(1, 0);
            // -A21: the off-diagonal block of the solve (rows 16-31, columns 0-15)
            const f32x4 acc = akk_tile(1, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = lg * 4 + r;
                const float x = -beta[16 + i] * acc[r];
                const __bf16 hi = bf(x);
                sA21[i * L16 + lr] = hi;
                sA21[16 * L16 + i * L16 + lr] = bf(x - fl(hi));
            }
        }
    };

    // UNB: the chunk's in-chunk matrices from the image in HBM, 16 bytes per
    // lane, waves 4..7 a quarter each, loaded a phase ahead like v
    constexpr int kImgUnits = kUnbImgElems / 8;
    uint4 pfi[UNB ? 2 : 1];
    auto loadImg = [&](int ch) {
        if constexpr (UNB) {
            const int lane = opaque_tid() & 63;
            const auto ri = make_rsrc(a.img + ((static_cast<size_t>(b) * HV + hv) * NC + ch) * kUnbImgElems,
                                      ch < NC ? kUnbImgElems * 2 : 0);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int u = (4 * j + wave - 4) * 64 + lane;   // past the image: read as 0, not stored
                const auto w = __builtin_amdgcn_raw_buffer_load_b128(ri, u * 16, 0, 0);
                pfi[j] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    };
    auto writeImg = [&]() {
        if constexpr (UNB) {
            const int lane = opaque_tid() & 63;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int u = (4 * j + wave - 4) * 64 + lane;
                if (u < kImgUnits) {
                    const int e = 8 * u;
                    __bf16 *dst;
                    if (e < 2048) {
                        dst = sAqk + (e >> 10) * kC * LDC + ((e >> 5) & 31) * LDC + (e & 31);
                    } else if (e < 2560) {
                        const int f = e - 2048;
                        dst = sA21 + (f >> 8) * 16 * L16 + ((f >> 4) & 15) * L16 + (f & 15);
                    } else {
                        const int f = e - 2560;
                        dst = sTi + (f >> 8) * 16 * L16 + ((f >> 4) & 15) * L16 + (f & 15);
                    }
                    *reinterpret_cast<uint4 *>(dst) = pfi[j];
                }
            }
        }
    };

    // ======================= carry waves
    // v of a chunk: waves 4..7 load whole rows of the V tile (16 bytes per lane)
    // one chunk ahead and write them to the staging tile sV; the carry waves read
    // their accumulator-layout fragments (column lr, rows 4 lg .. 4 lg + 3) with
    // ds_read_b64_tr_b16: in each 16-lane group g, lane 4a + b gets element b
    // of the 8-byte pieces addressed by lanes 16 g + 4 e + a, e = 0..3.
    // The staging work of the o and v tiles goes to waves 7, 4 and 5 (wave 6
    // has the longest list of its own in that phase; 4 and 5 the next): groups
    // of 64 units round-robin, helper index sh.
    constexpr int VUPR = VT / 8;                // 16-byte units per row of the V tile
    constexpr int VU = kC * VUPR;               // units of the tile
    constexpr int VPL = (VU / 64 + 2) / 3;      // unit groups per helper wave (at most)
    const int sh = wave == 7 ? 0 : wave == 4 ? 1 : 2;
    uint4 pfv[VPL];
    auto loadV = [&](int ch) {
        const int lane = opaque_tid() & 63;
        const int t0 = ch * kC;
        const auto rv = make_rsrc(vg + ((tok_b + t0) * HV + hv) * V + v0, rows_bytes(t0, v_stride, VT, 2));
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const int u = (3 * j + sh) * 64 + lane;   // past the tile: rows >= C, dropped by the resource
            const int row = u / VUPR, c8 = (u % VUPR) * 8;
            const auto w = __builtin_amdgcn_raw_buffer_load_b128(rv, (row * v_stride + c8) * 2, 0, 0);
            pfv[j] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    };
    // OG: the output gate's values for the o tile the helper waves store
    // next, loaded a phase ahead (the same addressing as the o stores)
    uint4 pfog[OG ? VPL : 1];
    auto loadOG = [&](int ch) {
        if constexpr (OG) {
            const int lane = opaque_tid() & 63;
            const int t0 = ch * kC;
            const auto rg_ = make_rsrc(static_cast<const uint16_t *>(a.ogate) + ((tok_b + t0) * HV + hv) * V + v0,
                                       rows_bytes(t0, v_stride, VT, 2));
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                const int u = (3 * j + sh) * 64 + lane;
                const int row = u / VUPR, c8 = (u % VUPR) * 8;
                const auto w = __builtin_amdgcn_raw_buffer_load_b128(rg_, (row * v_stride + c8) * 2, 0, 0);
                pfog[j] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    };
    auto writeV = [&]() {
        const int lane = opaque_tid() & 63;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const int u = (3 * j + sh) * 64 + lane;
            if (u < VU) {
                const int row = u / VUPR, c8 = (u % VUPR) * 8;
                *reinterpret_cast<uint4 *>(sV + row * LDO + c8) = pfv[j];
            }
        }
    };
    // v fragment of row tile rt, column block gi of this carry wave: rows
    // rt*16 + 4 lg + e (e = 0..3) of column 16 (wave NG + gi) + lr
    auto readV = [&](int rt, int gi) {
        const int lane = opaque_tid() & 63;
        const int row = rt * 16 + 4 * (lane >> 4) + ((lane >> 2) & 3);
        const int col = 16 * (wave * NG + gi) + 4 * (lane & 3);
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4 *)(sV + row * LDO + col));
    };

    // BWD: one 16-row tile of a chunk's [C][VT] fp32 result (accumulator
    // layout, this carry wave's column block gi) to dst [B, Lw, HV, V], rows
    // past the end dropped by the resource; nothing when dst is null
    auto storeTile = [&](float *dst, int n, int rt, int gi, const f32x4 &x) {
        if (!dst) return;
        const int lane = opaque_tid() & 63, lr = lane & 15, lg = lane >> 4;
        const int t0 = n * kC;
        const auto rs = make_rsrc(dst + ((static_cast<size_t>(b) * a.Lw + t0) * HV + hv) * V + v0,
                                  rows_bytes(t0, v_stride, VT, 4));
        const int col = 16 * (wave * NG + gi) + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float xr = x[r];
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(xr), rs,
                                                  ((rt * 16 + lg * 4 + r) * v_stride + col) * 4, 0, 0);
        }
    };

    f32x4 m[NG][KT];
    f32x4 pq[NG][2], xq[NG][2];
    bf16x8 ubh[NG], ubl[NG];       // U of the chunk between its solve (P1) and the state update (P2)
    // P = (q Gamma) M = (q e1)(2^{G_r} (.) M)  (three terms, both split) and
    // X = (k Gamma) M = (k e1)(2^{G_r} (.) M)  (single terms) of the next chunk.
    // The reference-row factor 2^{G_r} >= 2^-116 moves onto the state, so the
    // operand pass stores q e1 and k e1 once for both these products and A_qk, A_kk.
    auto carryPX = [&]() {
        const int lane = opaque_tid() & 63, lr = lane & 15, lg = lane >> 4;
        bf16x8 mh[NG][KS], ml[NG][KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                bf16x4 h0, l0, h1, l1;
                split4(m[gi][2 * s], h0, l0);
                split4(m[gi][2 * s + 1], h1, l1);
                mh[gi][s] = cat(h0, h1);
                ml[gi][s] = cat(l0, l1);
            }
        }
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                pq[gi][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
                xq[gi][rt] = pq[gi][rt];
            }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            bf16x8 qf[2], qfl[2], kf[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int p0 = sw(rt * 16 + lr, s * 32 + lg * 8);
                qf[rt] = ld8(sLq + p0);
                qfl[rt] = ld8(sLq + kC * LDK + p0);
                kf[rt] = ld8(sLk + p0);
            }
            // the three terms of P accumulate in place (accumulator forwarding
            // between MFMAs of one shape); independent products sit between them
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    pq[gi][rt] = mfma(qf[rt], mh[gi][s], pq[gi][rt]);
                    xq[gi][rt] = mfma(kf[rt], mh[gi][s], xq[gi][rt]);
                }
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) pq[gi][rt] = mfma(qf[rt], ml[gi][s], pq[gi][rt]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) pq[gi][rt] = mfma(qfl[rt], mh[gi][s], pq[gi][rt]);
        }
    };

    // R, solve and output of chunk n (U stays in registers for the state update)
    auto carryMain = [&](int n) {
        const int lane = opaque_tid() & 63, lr = lane & 15, lg = lane >> 4;
        const int cbuf = n & 1;
        // operand fragments that do not depend on this chunk's products
        const __bf16 *t11 = sTi + lr * L16 + lg * 4;
        const __bf16 *t22 = sTi + 2 * 16 * L16 + lr * L16 + lg * 4;
        const __bf16 *a21 = sA21 + lr * L16 + lg * 4;
        const bf16x4 t11h = ld4(t11), t11l = ld4(t11 + 16 * L16);
        const bf16x4 t22h = ld4(t22), t22l = ld4(t22 + 16 * L16);
        const bf16x4 a21h = ld4(a21), a21l = ld4(a21 + 16 * L16);
        bf16x8 aqh[2], aql[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int off = (rt * 16 + lr) * LDC + lg * 8;
            aqh[rt] = ld8(sAqk + off);
            aql[rt] = ld8(sAqk + kC * LDC + off);
        }
        // R = diag(beta) (v - (k Gamma) M), accumulator layout per 16-row tile
        const float *beta = sBeta + cbuf * kC;
        bf16x4 vf[NG][2];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) vf[gi][rt] = readV(rt, gi);
        f32x4 rr[NG][2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const f32x4 bt = *reinterpret_cast<const f32x4 *>(beta + rt * 16 + lg * 4);
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    rr[gi][rt][r] = bt[r] * (fl(vf[gi][rt][r]) - xq[gi][rt][r]);
                }
        }
        // U1 = T11 R1;  Y = R2 - A21 U1;  U2 = T22 Y   (16x16x16 MFMAs, 3 terms each)
        bf16x4 uh0[NG], ul0[NG], uh1[NG], ul1[NG];
        f32x4 acc[NG], acc2[NG];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            bf16x4 xh, xl;
            split4(rr[gi][0], xh, xl);
            acc[gi] = mfma16(t11h, xh, f32x4{0.f, 0.f, 0.f, 0.f});
            acc2[gi] = mfma16(t11h, xl, f32x4{0.f, 0.f, 0.f, 0.f});
            acc2[gi] = mfma16(t11l, xh, acc2[gi]);
        }
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            split4(acc[gi] + acc2[gi], uh0[gi], ul0[gi]);
            if constexpr (BWD) storeTile(a.u_out, n, 0, gi, acc[gi] + acc2[gi]);
            acc[gi] = mfma16(a21h, uh0[gi], rr[gi][1]);
            acc2[gi] = mfma16(a21h, ul0[gi], f32x4{0.f, 0.f, 0.f, 0.f});
            acc2[gi] = mfma16(a21l, uh0[gi], acc2[gi]);
        }
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            bf16x4 xh, xl;
            split4(acc[gi] + acc2[gi], xh, xl);
            acc[gi] = mfma16(t22h, xh, f32x4{0.f, 0.f, 0.f, 0.f});
            acc2[gi] = mfma16(t22h, xl, f32x4{0.f, 0.f, 0.f, 0.f});
            acc2[gi] = mfma16(t22l, xh, acc2[gi]);
        }
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            split4(acc[gi] + acc2[gi], uh1[gi], ul1[gi]);
            if constexpr (BWD) storeTile(a.u_out, n, 1, gi, acc[gi] + acc2[gi]);
            ubh[gi] = cat(uh0[gi], uh1[gi]);
            ubl[gi] = cat(ul0[gi], ul1[gi]);
        }

        // O = scale (P + A_qk U) -> the LDS staging tile (row-major); waves 4..7
        // store it to HBM in whole rows in the next phase
        if constexpr (BWD) return;
        f32x4 o[2][NG];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) o[rt][gi] = mfma(aqh[rt], ubh[gi], pq[gi][rt]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) o[rt][gi] = mfma(aqh[rt], ubl[gi], o[rt][gi]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) o[rt][gi] = mfma(aql[rt], ubh[gi], o[rt][gi]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const int col = 16 * (wave * NG + gi) + lr;
#pragma unroll
                for (int r = 0; r < 4; ++r) sO[(rt * 16 + lg * 4 + r) * LDO + col] = bf(o[rt][gi][r] * a.scale);
            }
    };

    // o of chunk n from the staging tile to HBM, 16 bytes per lane and whole
    // rows of the V tile per lane group (the helper waves, a third each)
    auto storeO = [&](int n) {
        if constexpr (BWD) return;
        const int lane = opaque_tid() & 63;
        const int t0 = n * kC;
        const auto ro = make_rsrc(og + ((tok_b + t0) * HV + hv) * V + v0, rows_bytes(t0, v_stride, VT, 2));
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const int u = (3 * j + sh) * 64 + lane;
            if (u < VU) {
                const int row = u / VUPR, c8 = (u % VUPR) * 8;
                uint4 w = *reinterpret_cast<const uint4 *>(sO + row * LDO + c8);
                if constexpr (OG) {
                    // y = sigmoid(gate) o / sqrt(mean(o^2) + eps) over the row's
                    // VT = V values, held by VUPR consecutive lanes (u < VU is the
                    // same for all of them: VU is a multiple of 64)
                    const uint32_t ow_[4] = {w.x, w.y, w.z, w.w};
                    const uint32_t gw[4] = {pfog[j].x, pfog[j].y, pfog[j].z, pfog[j].w};
                    float o[8], ss = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        o[2 * e] = bf_lo(ow_[e]);
                        o[2 * e + 1] = bf_hi(ow_[e]);
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(o[e], o[e], ss);
                    ss = rowN_sum<VUPR>(ss);
                    const float inv = 1.0f / sqrtf(ss * (1.0f / VT) + a.og_eps);
                    uint32_t yw[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        yw[e] = pk(inv1p_exp2(-bf_lo(gw[e]) * kLog2e) * o[2 * e] * inv,
                                   inv1p_exp2(-bf_hi(gw[e]) * kLog2e) * o[2 * e + 1] * inv);
                    w = make_uint4(yw[0], yw[1], yw[2], yw[3]);
                }
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), ro, (row * v_stride + c8) * 2, 0, 0);
            }
        }
    };

    // State update of chunk n.  The carried state is N = 2^{G_r} (.) M (per K
    // row; G_r of the chunk about to be processed), the form the state products
    // read.  With k_bar = 2^{G_last - G_r} (k e2):
    //     M' = Gamma_last (.) M + k_bar^T U = 2^{G_last - G_r} (.) (N + (k e2)^T U)
    // so (k e2)^T U accumulates into N, then the rows are scaled by
    // 2^{G_last - G_r} and (unless this is the last chunk) by the next chunk's
    // 2^{G_r}: two products, since each factor is >= 2^-116 but theirs may not
    // be representable.  Four row tiles at a time; the three terms accumulate
    // into N in turn, the tiles of a batch between them.
    auto carryUpdate = [&](int n, bool last) {
        const int lane = opaque_tid() & 63, lr = lane & 15, lg = lane >> 4;
        const int cbuf = n & 1;
        const __bf16 *kb_buf = sKbarT + cbuf * 2 * K * LDC + kb_at(lr, lg * 8);
        const float *plp = sPl + cbuf * K + lg * 4;
        const float *prp = sPr + lg * 4;
        constexpr int KB = KT < 4 ? KT : 4;
#pragma unroll
        for (int k0 = 0; k0 < KT; k0 += KB) {
            bf16x8 kf[KB], kfl[KB];
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                kf[u] = ld8(kb_buf + (k0 + u) * 16 * LDC);
                kfl[u] = ld8(kb_buf + K * LDC + (k0 + u) * 16 * LDC);
            }
            if constexpr (UNB) {
                // M' = Gamma_last (.) M + (k Lambda)^T U: the decay first
#pragma unroll
                for (int u = 0; u < KB; ++u) {
                    const f32x4 plv = *reinterpret_cast<const f32x4 *>(plp + (k0 + u) * 16);
#pragma unroll
                    for (int gi = 0; gi < NG; ++gi) m[gi][k0 + u] *= plv;
                }
            }
#pragma unroll
            for (int u = 0; u < KB; ++u)
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) m[gi][k0 + u] = mfma(kf[u], ubh[gi], m[gi][k0 + u]);
#pragma unroll
            for (int u = 0; u < KB; ++u)
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) m[gi][k0 + u] = mfma(kf[u], ubl[gi], m[gi][k0 + u]);
#pragma unroll
            for (int u = 0; u < KB; ++u)
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) m[gi][k0 + u] = mfma(kfl[u], ubh[gi], m[gi][k0 + u]);
            if constexpr (!UNB) {
#pragma unroll
                for (int u = 0; u < KB; ++u) {
                    const f32x4 plv = *reinterpret_cast<const f32x4 *>(plp + (k0 + u) * 16);
                    const f32x4 prv = *reinterpret_cast<const f32x4 *>(prp + (k0 + u) * 16);
#pragma unroll
                    for (int gi = 0; gi < NG; ++gi) {
                        m[gi][k0 + u] *= plv;
                        if (!last) m[gi][k0 + u] *= prv;
                    }
                }
            }
        }
    };
    // N of the first chunk: S0 scaled by its 2^{G_r}
    auto carryScaleState = [&]() {
        if constexpr (UNB) return;   // the carry holds M itself
        const int lane = opaque_tid() & 63, lg = (lane >> 4) & 3;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            const f32x4 prv = *reinterpret_cast<const f32x4 *>(sPr + kt * 16 + lg * 4);
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) m[gi][kt] *= prv;
        }
    };

    // rowscale(kt) (.) M -> dst[K][V], the columns of this wave (the carry's
    // own layout).  A buffer resource and an opaque lane index keep the
    // addresses from being hoisted into registers that live across the whole
    // chunk loop.
    auto carryStoreScaled = [&](float *dst, auto rowscale) {
        const int lane = opaque_tid() & 63, lr = lane & 15, lg = lane >> 4;
        int row_bytes = V * 4;
        asm volatile("" : "+s"(row_bytes));
        const auto rs = make_rsrc(dst, static_cast<uint32_t>(K) * V * 4);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            const f32x4 sc = rowscale(kt, lg);
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const int vo = lg * 4 * row_bytes + (v0 + 16 * (wave * NG + gi) + lr) * 4;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // the element is copied out first: __builtin_bit_cast applied to a
                    // vector element directly compiles to element 0 for every r
                    const float x = m[gi][kt][r] * sc[r];
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rs, vo,
                                                          (kt * 16 + r) * row_bytes, 0);
                }
            }
        }
    };
    auto carryStore = [&](float *dst) {
        carryStoreScaled(dst, [](int, int) { return f32x4{1.f, 1.f, 1.f, 1.f}; });
    };
    // Prefix snapshots (SNAP only): the state after chunks snap_chunks,
    // 2 snap_chunks, ..., NS snap_chunks; snap_ptr is the next one's [K][V]
    // slice, null when none is left.
    float *snap_ptr = SNAP && a.snap ? a.snap + ((static_cast<size_t>(b) * a.NS) * HV + hv) * K * V : nullptr;
    int snap_at = a.snap_chunks;
    // Snapshot after chunk snap_at - 1.  exact: m holds M (after the last
    // chunk).  Otherwise m holds the next chunk's N (end of P2, off the carry's
    // critical block) and M = N / 2^{G_r}, the reciprocal exact to 1 ulp.
    auto carrySnapshot = [&](bool exact) {
        if (exact) {
            carryStore(snap_ptr);
        } else {
            carryStoreScaled(snap_ptr, [&](int kt, int lg) {
                const f32x4 prv = *reinterpret_cast<const f32x4 *>(sPr + kt * 16 + lg * 4);
                f32x4 inv;
#pragma unroll
                for (int r = 0; r < 4; ++r) inv[r] = __builtin_amdgcn_rcpf(prv[r]);
                return inv;
            });
        }
        snap_at += a.snap_chunks;
        snap_ptr = snap_at <= a.NS * a.snap_chunks ? snap_ptr + static_cast<size_t>(HV) * K * V : nullptr;
    };

    // ---------------------------------------------------------------- prologue: chunk 0
    if (carry) {
        const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
        if (a.S0) {
            const size_t s0b = a.s0_bstride ? static_cast<size_t>(a.s0_bstride) : static_cast<size_t>(HV) * K * V;
            const float *S0 = a.S0 + b * s0b + static_cast<size_t>(hv) * K * V;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const int vcol = v0 + 16 * (wave * NG + gi) + lr;
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        m[gi][kt][r] = S0[static_cast<size_t>(kt * 16 + lg * 4 + r) * V + vcol];
            }
        } else {
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) m[gi][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (!UNB && wave == 0) {
            // rows 0-15 x columns 16-31 of A_qk lie above the diagonal: zero for every chunk
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = lg * 4 + r, j = perm(16 + lr);
                sAqk[i * LDC + j] = bf(0.f);
                sAqk[kC * LDC + i * LDC + j] = bf(0.f);
            }
        }
    }
    if (wave >= 4 && wave != 6) {
        loadV(0);
        writeV();
        loadV(1);
        loadOG(0);
    }
    if (UNB && wave >= 4) {
        loadImg(0);
        writeImg();
        loadImg(1);
    }
    if (opw) {
        load_prep(0);
        op1a(0, 0);
        load_prep(1);
        op1b(0, 0);
        op2(0);
    }
    lds_barrier();
    if (!UNB && wave >= 4) phaseAT(0);
    if (carry) {
        carryScaleState();
        carryPX();
    }
    lds_barrier();

    // ---------------------------------------------------------------- main loop
    for (int n = 0; n + 1 < NC; ++n) {
        const int nb = (n + 1) & 1;
        // P1 (carry waves get their carry work and their share of the operand
        // pass in one block, so the scheduler can fill MFMA latency with VALU)
        if (carry) {
            if (opw) {
                op1a(nb, n + 1);
                load_prep(n + 2);
                op1b(nb, n + 1);
            }
            carryMain(n);
            if (opw) op2(nb);
        } else if (opw) {
            op1a(nb, n + 1);
            load_prep(n + 2);
            op1b(nb, n + 1);
            op2(nb);
        }
        lds_barrier();
        // P2
        if (wave >= 4) {
            if constexpr (UNB) {
                writeImg();      // the in-chunk matrices of chunk n+1
                loadImg(n + 2);
            } else {
                phaseAT(nb);
            }
            if (wave != 6) {
                storeO(n);
                writeV();        // v of chunk n+1 for the next phase's carry
                loadV(n + 2);
                loadOG(n + 1);
            }
        }
        if (carry) {
            carryUpdate(n, false);
            carryPX();
            if constexpr (SNAP)
                if (snap_ptr && n + 1 == snap_at) carrySnapshot(false);
        }
        lds_barrier();
    }
    if (carry) {
        carryMain(NC - 1);
        carryUpdate(NC - 1, true);
        if constexpr (SNAP)
            if (snap_ptr && NC == snap_at) carrySnapshot(true);
    }
    lds_barrier();
    if (wave >= 4 && wave != 6) storeO(NC - 1);

    if (a.ST && carry) carryStore(a.ST + (static_cast<size_t>(b) * HV + hv) * K * V);
}

template <int K, int VT, bool SNAP, bool GATED, bool OG, bool BWD = false, bool UNB = false>
hipError_t launch_kvt_s(const PrefillArgs &a, hipStream_t stream) {
    using L = Plan<K>;
    auto kern = prefill_bf16_kernel<K, VT, SNAP, GATED, OG, BWD, UNB>;
    constexpr int lds = L::bytes + L::stage_bytes(VT);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    const unsigned grid = static_cast<unsigned>(a.B) * a.HV * (a.V / VT);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kNT), lds, stream, a);
    return hipGetLastError();
}

template <int K, int VT>
hipError_t launch_kvt(const PrefillArgs &a, hipStream_t stream) {
    if (a.bwd) return launch_kvt_s<K, VT, true, false, false, true>(a, stream);
    if (a.unb) return launch_kvt_s<K, VT, false, false, false, false, true>(a, stream);
    if (a.snap) return launch_kvt_s<K, VT, true, false, false>(a, stream);
    if (!a.A_log) return launch_kvt_s<K, VT, false, false, false>(a, stream);
    // the fused gate; the output gate in the o stores when the workgroup
    // holds whole rows of V, else as its own pass over out afterwards
    if (a.ogate && VT == a.V) return launch_kvt_s<K, VT, false, true, true>(a, stream);
    hipError_t e = launch_kvt_s<K, VT, false, true, false>(a, stream);
    if (e != hipSuccess || !a.ogate) return e;
    OutputGateArgs og{};
    og.o = a.out; og.gate = a.ogate; og.y = a.out;
    og.rows = static_cast<long>(a.B) * a.T * a.HV; og.D = a.V; og.eps = a.og_eps; og.bf16 = true;
    return launch_output_gate(og, stream);
}

template <int K>
hipError_t launch_k(const PrefillArgs &a, hipStream_t stream) {
    // Split V across two workgroups when the halves of every (b, hv) chain all
    // fit on the GPU at once (one workgroup per CU): a chunk takes less time
    // with half of V.  With more chains the split would queue a second round
    // of workgroups behind the first, so each chain is then one workgroup.
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const long chains = static_cast<long>(a.B) * a.HV;
    const bool split = a.V >= 64 && 2 * chains <= cus;
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
