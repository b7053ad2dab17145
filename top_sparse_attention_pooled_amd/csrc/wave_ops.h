// wave_ops.h -- 64-lane wavefront exchange, reduction and scan primitives
// built on DPP and the gfx950 permlane swaps.
//
// A generic __shfl_xor goes through ds_bpermute: an LDS round trip of about
// a hundred cycles, paid at every step of a dependent chain (a 6-level
// butterfly, a 21-stage sorting network).  Here the partner value of lane
// l ^ m comes from
//   m = 1, 2 : DPP quad_perm
//   m = 4, 8 : DPP row_shl / row_shr by m, each writing only the lanes whose
//              bit m is 0 / 1 (bank_mask: banks are the 4-lane groups of a
//              16-lane row)
//   m = 16   : v_permlane16_swap (exchanges odd and even 16-lane rows)
//   m = 32   : v_permlane32_swap (exchanges the two 32-lane halves)
// all of which stay in the vector ALU.  The inclusive scan is the classic
// row_shr 1/2/4/8 ladder with zero fill, then row_bcast15 and row_bcast31.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// DPP control words (gfx9 encoding)
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowShl = 0x100;   // + n: lane l reads lane l + n of its row
constexpr int kRowShr = 0x110;   // + n: lane l reads lane l - n of its row
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;

// Value of lane (lane ^ M) for M in {1, 2, 4, 8, 16, 32}.
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
    const int x = (int)v;
    if constexpr (M == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, x, kQuadXor1, 0xF, 0xF, false);
    } else if constexpr (M == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, x, kQuadXor2, 0xF, 0xF, false);
    } else if constexpr (M == 4) {
        int r = __builtin_amdgcn_update_dpp(0, x, kRowShl + 4, 0xF, 0x5, false);
        r = __builtin_amdgcn_update_dpp(r, x, kRowShr + 4, 0xF, 0xA, false);
        return (uint32_t)r;
    } else if constexpr (M == 8) {
        int r = __builtin_amdgcn_update_dpp(0, x, kRowShl + 8, 0xF, 0x3, false);
        r = __builtin_amdgcn_update_dpp(r, x, kRowShr + 8, 0xF, 0xC, false);
        return (uint32_t)r;
    } else if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (threadIdx.x & 16) ? r[0] : r[1];
    } else {
        static_assert(M == 32, "xor_lane: M must be 1, 2, 4, 8, 16 or 32");
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (threadIdx.x & 32) ? r[0] : r[1];
    }
}

template <int M>
__device__ __forceinline__ float xor_lane_f(float v) {
    return __uint_as_float(xor_lane<M>(__float_as_uint(v)));
}

template <int M>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v) {
    const uint32_t lo = xor_lane<M>((uint32_t)v);
    const uint32_t hi = xor_lane<M>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Runtime-M dispatch (M a power of two <= 32).
__device__ __forceinline__ uint32_t xor_lane_rt(uint32_t v, int m) {
    switch (m) {
        case 1: return xor_lane<1>(v);
        case 2: return xor_lane<2>(v);
        case 4: return xor_lane<4>(v);
        case 8: return xor_lane<8>(v);
        case 16: return xor_lane<16>(v);
        default: return xor_lane<32>(v);
    }
}

// Butterfly all-reduce over the 64 lanes (every lane gets the result).
template <typename Op>
__device__ __forceinline__ uint32_t wave_allreduce_u32(uint32_t v, Op op) {
    v = op(v, xor_lane<1>(v));
    v = op(v, xor_lane<2>(v));
    v = op(v, xor_lane<4>(v));
    v = op(v, xor_lane<8>(v));
    v = op(v, xor_lane<16>(v));
    v = op(v, xor_lane<32>(v));
    return v;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    return wave_allreduce_u32(v, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    return wave_allreduce_u32(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    return wave_allreduce_u32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ float wave_max_f32(float v) {
    v = fmaxf(v, xor_lane_f<1>(v));
    v = fmaxf(v, xor_lane_f<2>(v));
    v = fmaxf(v, xor_lane_f<4>(v));
    v = fmaxf(v, xor_lane_f<8>(v));
    v = fmaxf(v, xor_lane_f<16>(v));
    v = fmaxf(v, xor_lane_f<32>(v));
    return v;
}

// Every lane gets the same sum: partners add the same two values at each
// level, and addition is commutative.
__device__ __forceinline__ float wave_sum_f32(float v) {
    v += xor_lane_f<1>(v);
    v += xor_lane_f<2>(v);
    v += xor_lane_f<4>(v);
    v += xor_lane_f<8>(v);
    v += xor_lane_f<16>(v);
    v += xor_lane_f<32>(v);
    return v;
}

// Inclusive prefix sum over the 64 lanes in lane order.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 1, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 2, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 4, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 8, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, kRowBcast15, 0xA, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, kRowBcast31, 0xC, 0xF, false);
    return (uint32_t)x;
}

// Value held by lane `src` (uniform src).
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int src) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, src);
}

}  // namespace qsa
