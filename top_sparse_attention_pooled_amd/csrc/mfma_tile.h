// mfma_tile.h -- the bf16 query x block-key contraction on the matrix cores
// (v_mfma_f32_16x16x32_bf16), shared by the prefill scoring kernels.
//
// A wavefront computes a 64-query x 64-block tile as 4 x 4 MFMA tiles of
// 16 x 16 over k = 128 (4 steps of 32).  Operand lanes: lane l supplies row
// l % 16 and k-slice 8*(l / 16) .. +7 of A (queries) and of B (blocks, i.e.
// columns); the result lane l holds rows 4*(l / 16) + jj, jj < 4, of column
// l % 16.  Products of bf16 values are exact in fp32; only the order of the
// fp32 additions differs from the canonical order T.
#pragma once

#include "qsa_internal.h"

namespace qsa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t *p) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(p);
    return __builtin_bit_cast(bf16x8_t, v);
}

// A operands of queries q0 .. q0+63 (rows past n_q are zero).
__device__ __forceinline__ void load_query_tile(const uint16_t *qr_bf16, int q0, int n_q,
                                                bf16x8_t (&A)[4][4]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int mrow = lane & 15, kseg = (lane >> 4) * 8;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        const int qi = q0 + rb * 16 + mrow;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            A[rb][ks] = qi < n_q ? load_bf16x8(qr_bf16 + (int64_t)qi * kDIdx + ks * 32 + kseg)
                                 : bf16x8_t{};
    }
}

// B operands of blocks gb0 .. gb0+63 of one sequence's bf16 keys (zero
// columns past cap_blocks or when !live).
__device__ __forceinline__ void load_key_tile(const uint16_t *keys, int64_t gb0,
                                              int64_t cap_blocks, bool live,
                                              bf16x8_t (&B)[4][4]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int mrow = lane & 15, kseg = (lane >> 4) * 8;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const int64_t nb = gb0 + cb * 16 + mrow;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            B[cb][ks] = (live && nb < cap_blocks)
                            ? load_bf16x8(keys + nb * kDIdx + ks * 32 + kseg)
                            : bf16x8_t{};
    }
}

// acc[rb][cb][jj] = <query row rb*16 + 4*(lane/16) + jj, block col cb*16 +
// lane%16 of the B tile>.
__device__ __forceinline__ void mfma_tile(const bf16x8_t (&A)[4][4], const bf16x8_t (&B)[4][4],
                                          f32x4_t (&acc)[4][4]) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[rb][ks], B[cb][ks], c, 0, 0, 0);
            acc[rb][cb] = c;
        }
}

// Both: the tile of blocks gb0 .. gb0+63.
__device__ __forceinline__ void wave_tile_mfma(const bf16x8_t (&A)[4][4], const uint16_t *keys,
                                               int64_t gb0, int64_t cap_blocks, bool live,
                                               f32x4_t (&acc)[4][4]) {
    bf16x8_t B[4][4];
    load_key_tile(keys, gb0, cap_blocks, live, B);
    mfma_tile(A, B, acc);
}

}  // namespace qsa
