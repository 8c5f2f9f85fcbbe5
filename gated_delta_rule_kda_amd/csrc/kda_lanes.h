// Lane-level helpers shared by the token-recurrent kernels (forward and
// backward): buffer-resource loads, bf16 widening, DPP sums, sums across the
// DPP rows of a wave, the hardware exponential.
#pragma once
#include "kda_internal.h"

namespace kda {
namespace lanes {

constexpr float kLog2e = 1.4426950408889634f;

// 2^x by the hardware exponential alone, without the library's rescaling for
// results below the normal range (1 ulp; such a result may come out as 0, an
// absolute change of less than 2^-126 in a decay factor)
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// x of another lane (DPP); the 0 that stands for lanes without a source lets the
// compiler fold the move into the add that consumes it
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Sum over aligned groups of N consecutive lanes (N = 8: half a DPP row, 16: a
// DPP row), the result in every lane of the group.
template <int N>
__device__ __forceinline__ float group_sum(float s) {
    static_assert(N == 8 || N == 16, "half or whole DPP rows");
    s += dpp<0xb1>(s);    // quad_perm [1,0,3,2]
    s += dpp<0x4e>(s);    // quad_perm [2,3,0,1]
    s += dpp<0x141>(s);   // row_half_mirror
    if constexpr (N == 16) s += dpp<0x140>(s);   // row_mirror
    return s;
}
// Sums over the four DPP rows of a wave (lane positions l % 16 equal) of N
// values per lane, N in {2, 4, 8}, spread over the result so that every lane
// keeps some: swapping two different values at each step needs no copies and
// halves the instructions of summing each value by itself.  After the call,
// lane l (DPP row j = l / 16) holds in out[i] the sum of value
// across_index<N>(i, j) -- see below -- over the four rows.
//   Step 1 (lane swap of the wave's halves) on pairs (x[2m], x[2m+1]):
//     rows 0,1 keep x[2m] (rows 0+2, 1+3 summed), rows 2,3 x[2m+1].
//   Step 2 (swap of neighbouring rows) on pairs of those: the four rows of
//     out[i] end up with values 4i, 4i+2, 4i+1, 4i+3 (N = 2: 0, 0, 1, 1).
template <int N>
__device__ __forceinline__ void across_rows_sums(const float (&x)[N], float (&out)[N < 4 ? 1 : N / 4]) {
    static_assert(N == 2 || N == 4 || N == 8, "2, 4 or 8 values");
    float h[N / 2];
#pragma unroll
    for (int m = 0; m < N / 2; ++m) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[2 * m]), __float_as_uint(x[2 * m + 1]),
                                                         false, false);
        h[m] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if constexpr (N == 2) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(h[0]), __float_as_uint(h[0]), false, false);
        out[0] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    } else {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(h[2 * i]), __float_as_uint(h[2 * i + 1]),
                                                             false, false);
            out[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
    }
}
// which of the N values out[i] of DPP row j holds the sum of
template <int N>
__device__ __forceinline__ int across_index(int i, int j) {
    if constexpr (N == 2) return j >> 1;
    else return 4 * i + ((j & 1) << 1) + (j >> 1);
}

// 4 consecutive elements as loaded (bf16: two packed words; fp32: a float4)
template <bool BF16> struct Raw4;
template <> struct Raw4<true> { uint2 u; };
template <> struct Raw4<false> { float4 f; };
// Raw buffer resource over `bytes` bytes from `p`: out-of-range loads read 0
// and out-of-range stores are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, static_cast<int>(bytes), 0x00020000);
}
template <bool BF16>
__device__ __forceinline__ Raw4<BF16> load_raw4(__amdgpu_buffer_rsrc_t rs, int byte_off) {
    if constexpr (BF16) {
        const auto u = __builtin_amdgcn_raw_buffer_load_b64(rs, byte_off, 0, 0);
        return Raw4<true>{make_uint2(u[0], u[1])};
    } else {
        const auto u = __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0);
        return Raw4<false>{make_float4(__uint_as_float(u[0]), __uint_as_float(u[1]),
                                       __uint_as_float(u[2]), __uint_as_float(u[3]))};
    }
}
__device__ __forceinline__ float4 load_f4(__amdgpu_buffer_rsrc_t rs, int byte_off) {
    const auto u = __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0);
    return make_float4(__uint_as_float(u[0]), __uint_as_float(u[1]), __uint_as_float(u[2]), __uint_as_float(u[3]));
}
template <bool BF16>
__device__ __forceinline__ float4 widen(const Raw4<BF16> &r) {
    if constexpr (BF16)
        return make_float4(__uint_as_float(r.u.x << 16), __uint_as_float(r.u.x & 0xffff0000u),
                           __uint_as_float(r.u.y << 16), __uint_as_float(r.u.y & 0xffff0000u));
    else
        return r.f;
}
// one element of a dtype array through a buffer resource (bf16 or fp32)
template <bool BF16>
__device__ __forceinline__ float load1(__amdgpu_buffer_rsrc_t rs, int elem) {
    if constexpr (BF16)
        return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(rs, elem * 2, 0, 0)) << 16);
    else
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, elem * 4, 0, 0));
}
template <bool BF16>
__device__ __forceinline__ void store1(void *p, size_t i, float x) {
    if constexpr (BF16)
        static_cast<uint16_t *>(p)[i] = float_to_bf16_bits(x);
    else
        static_cast<float *>(p)[i] = x;
}

}  // namespace lanes
}  // namespace kda
