// kv_rows.h -- one lane's slice of a K or V row, raw and dequantised.
//
// q8_0 rows: 8 blocks of (binary16 scale, 32 int8) = 272 bytes.  The slice
// of dims 8j .. 8j+7 lies in block j/4 at byte 34*(j/4) + 2 + 8*(j%4), which
// is 2 mod 4 for even blocks: it is read as aligned dwords and realigned with
// a funnel shift.  f32 rows: 256 floats.  f16 rows: 256 binary16 values, the
// slice one 16-byte load, widened exactly.
#pragma once

#include "qsa_internal.h"

namespace qsa {

// Raw bytes of one lane's slice (dims 8j .. 8j+7) of one K or V row.
template <int KVT>
struct RawRow;
template <>
struct RawRow<QSA_KV_F32> {
    float4 u, v;
};
template <>
struct RawRow<QSA_KV_Q8_0> {
    uint32_t w0, w1, w2, sw;
};
template <>
struct RawRow<QSA_KV_F16> {
    uint4 h;  // 8 binary16 values
};

template <int KVT>
__device__ __forceinline__ RawRow<KVT> load_raw(const void *base, int64_t row, int j) {
    RawRow<KVT> r;
    if constexpr (KVT == QSA_KV_F32) {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) +
                                                           row * kHeadDim + 8 * j);
        r.u = p[0];
        r.v = p[1];
    } else if constexpr (KVT == QSA_KV_F16) {
        r.h = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) +
                                               row * kHeadDim + 8 * j);
    } else {
        const uint8_t *b = static_cast<const uint8_t *>(base) + row * kQ8Row;
        const int blk = j >> 2;
        const int start = blk * kQ8Bytes + 2 + 8 * (j & 3);
        const uint32_t *w = reinterpret_cast<const uint32_t *>(b + (start & ~3));
        r.w0 = w[0];
        r.w1 = w[1];
        r.w2 = (start & 3) ? w[2] : 0u;  // only rows whose int8 start 2 mod 4 need it
        r.sw = *reinterpret_cast<const uint32_t *>(b + ((blk * kQ8Bytes) & ~3));
    }
    return r;
}

// Dequantise: q8_0 value = float(binary16 scale) * int8, exact in fp32.
template <int KVT>
__device__ __forceinline__ void dequant(const RawRow<KVT> &r, int j, float (&x)[8]) {
    if constexpr (KVT == QSA_KV_F32) {
        x[0] = r.u.x; x[1] = r.u.y; x[2] = r.u.z; x[3] = r.u.w;
        x[4] = r.v.x; x[5] = r.v.y; x[6] = r.v.z; x[7] = r.v.w;
    } else if constexpr (KVT == QSA_KV_F16) {
        const uint32_t w[4] = {r.h.x, r.h.y, r.h.z, r.h.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] & 0xffffu));
            x[2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] >> 16));
        }
    } else {
        const int blk = j >> 2;
        const bool odd = blk & 1;  // block start 2 mod 4: int8 aligned, scale in high half
        const uint32_t lo = odd ? r.w0 : __builtin_amdgcn_alignbyte(r.w1, r.w0, 2);
        const uint32_t hi = odd ? r.w1 : __builtin_amdgcn_alignbyte(r.w2, r.w1, 2);
        const uint16_t sbits = (uint16_t)(odd ? (r.sw >> 16) : (r.sw & 0xffffu));
        const float d = (float)__builtin_bit_cast(_Float16, sbits);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = d * (float)((int32_t)(lo << (24 - 8 * e)) >> 24);
            x[e + 4] = d * (float)((int32_t)(hi << (24 - 8 * e)) >> 24);
        }
    }
}

// The 8 int8 of a q8_0 slice (dims 8j .. 8j+7, block j/4), realigned.
__device__ __forceinline__ void q8_ints(const RawRow<QSA_KV_Q8_0> &r, int j, uint32_t &lo,
                                        uint32_t &hi) {
    const bool odd = (j >> 2) & 1;
    lo = odd ? r.w0 : __builtin_amdgcn_alignbyte(r.w1, r.w0, 2);
    hi = odd ? r.w1 : __builtin_amdgcn_alignbyte(r.w2, r.w1, 2);
}

// binary16 bits of the slice's block scale.
__device__ __forceinline__ uint32_t q8_scale_bits(const RawRow<QSA_KV_Q8_0> &r, int j) {
    return ((j >> 2) & 1) ? (r.sw >> 16) : (r.sw & 0xffffu);
}

}  // namespace qsa
