// attn_prefill.hip -- sparse attention for many queries on the matrix cores
// (llama.cpp issue #28734, fix summary, "lever1": attention visits the
// selected cells only; discussion #30071: q8_0 rows are dequantised inside
// the gather).
//
// Workgroup = (query i, KV head g), 4 wavefronts; wavefront w takes the
// 32-cell chunks w, w+4, ... of the query's cell list and keeps its own
// online-softmax state; the four states merge at the end.  Per chunk, with
// the hpk <= 8 query heads of the KV head as the 16 M-rows of the tiles
// (rows past hpk are zero):
//   S  = (scale * Q) K^T  : 2 tiles of 16 cells x 8 k-steps of 32 dims with
//        v_mfma_f32_16x16x32_f16.  For q8_0 a k-step is one block: its int8
//        go into the B operand as exact fp16 integers (byte | 0x6400 is 1024
//        + byte) and the block scale multiplies the k-step's fp32 result;
//   online softmax on S in the accumulator layout (a head row's 16 columns
//        sit in one 16-lane DPP row);
//   O += P V : P goes through LDS to the A layout, V is staged transposed in
//        LDS as fp16 [dim][cell] (q8_0: int8 times its scale, one fp16
//        rounding) so each B operand is one 16-byte read.
// q8_0 rows reach the wavefront as whole 16-byte pieces: the chunk's 64 rows
// (K and V, 272 bytes each) are 17 coalesced loads per lane, prefetched one
// chunk ahead in registers and written to an LDS stage, from which the
// operands are read.  f32 and f16 rows, and q8_0 rows reached through a cell
// table, are gathered per lane straight into the operand layout.
// Operands are rounded to fp16 (Q * scale, P, V; f32 K); sums and the
// softmax state are fp32.
#include <type_traits>

#include "kv_rows.h"
#include "qsa_internal.h"
#include "wave_ops.h"

namespace qsa {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPChunk = 32;  // cells per chunk
constexpr int kPWaves = 4;
constexpr int kStride = kPWaves * kPChunk;
constexpr int kCellCap = 4096;  // per-lane kernel: cell indices held in LDS; the rest read directly
constexpr int kStageWords = kPChunk * kQ8Row / 4;  // raw rows of one chunk (K or V)
constexpr int kPieces = 2 * kPChunk * kQ8Row / 16;     // 16-byte pieces per chunk
static_assert(kPieces == 17 * kWave, "a chunk is 17 loads of 16 bytes per lane");

// Per-wavefront LDS.  The q8_0 kernel transposes V in two halves of 128
// dims so that a wavefront's LDS (the stage plus this tail, about 19 KB)
// lets two workgroups share a CU.
constexpr int kVtPitch = kPChunk + 4;  // fp16 per vt row: 18 dwords, so rows 8 apart differ in bank
template <int VROWS>
struct WaveTailT {
    union {
        _Float16 vt[VROWS][kVtPitch];  // V of the chunk, transposed (cells 0..31 used)
        float o[16][kHeadDim / 4];     // merge: a quarter of the dims at a time
    };
    _Float16 p[16][kPChunk];  // probabilities, [head row][cell]
    float m[16], l[16];
};
using WaveTail = WaveTailT<kHeadDim>;      // f32 and f16 rows: all dims at once
using HalfTail = WaveTailT<kHeadDim / 2>;  // q8_0 rows: V in two halves
static_assert(sizeof(_Float16[kHeadDim / 2][kVtPitch]) >= sizeof(float[16][kHeadDim / 4]),
              "the merge buffer fits the half transpose");
struct RowWave {
    WaveTail t;
};
struct Q8Wave {
    uint32_t stage[kStageWords];  // the chunk's K rows, later its V rows, as loaded
    HalfTail t;
};

__device__ __forceinline__ half8_t to_half8(const float (&x)[8]) {
    half8_t h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (_Float16)x[e];
    return h;
}

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// Bytes 0, 1 (sel kLowPair) or 2, 3 (kHighPair) of x, each as the fp16 1024 + byte.
constexpr uint32_t kLowPair = 0x04010400u, kHighPair = 0x04030402u;
__device__ __forceinline__ half2_t byte_pair_1024(uint32_t x, uint32_t sel) {
    return as_half2(__builtin_amdgcn_perm(0x64646464u, x, sel));
}

// Four int8 of w (two's complement) as exact fp16: (b ^ 0x80) is b + 128 as
// an unsigned byte, so 1024 + (b ^ 0x80) - 1152 = b.
__device__ __forceinline__ void int8x4_to_half(uint32_t w, half2_t &h01, half2_t &h23) {
    const half2_t off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    w ^= 0x80808080u;
    h01 = byte_pair_1024(w, kLowPair) + off;
    h23 = byte_pair_1024(w, kHighPair) + off;
}

// Dims 8j .. 8j+7 of a staged q8_0 row (block j/4 at byte 34*(j/4), its
// int8 from byte 2): the 8 int8, realigned when the block is even (its int8
// then start 2 mod 4).  The alignment depends on j/4 only.
__device__ __forceinline__ void staged_slice(const uint8_t *row, int j, uint32_t &lo,
                                             uint32_t &hi) {
    const int blk = j >> 2, off = blk * kQ8Bytes + 2 + 8 * (j & 3);
    const uint32_t *w = reinterpret_cast<const uint32_t *>(row + (off & ~3));
    if (blk & 1) {
        lo = w[0];
        hi = w[1];
    } else {
        const uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
        lo = __builtin_amdgcn_alignbyte(w1, w0, 2);
        hi = __builtin_amdgcn_alignbyte(w2, w1, 2);
    }
}
// binary16 bits of the scale of block blk of a staged q8_0 row.
__device__ __forceinline__ uint32_t staged_scale(const uint8_t *row, int blk) {
    return *reinterpret_cast<const uint16_t *>(row + blk * kQ8Bytes);
}

// Max / sum over the 16 lanes of a DPP row.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, xor_lane_f<1>(v));
    v = fmaxf(v, xor_lane_f<2>(v));
    v = fmaxf(v, xor_lane_f<4>(v));
    v = fmaxf(v, xor_lane_f<8>(v));
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v += xor_lane_f<1>(v);
    v += xor_lane_f<2>(v);
    v += xor_lane_f<4>(v);
    v += xor_lane_f<8>(v);
    return v;
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Query state common to both kernels.
struct QueryCtx {
    int n;              // cells in the list
    int64_t n_present;  // cells of the sequence
    const int32_t *cells;
    int64_t row0;  // s * cap_cells: position p of the sequence is entry row0 + p
};

__device__ __forceinline__ QueryCtx query_ctx(const AttnArgs &a, int i) {
    QueryCtx c;
    const int s = a.q_seq[i];
    const bool qvalid = s >= 0 && s < a.g.n_seq;
    const int n = qvalid ? a.n_sel[i] : 0;
    c.n = n < 0 ? 0 : (n > a.ld_cells ? a.ld_cells : n);
    const int64_t np = qvalid ? a.g.n_cells[s] : 0;
    c.n_present = np < a.g.cap_cells ? np : a.g.cap_cells;
    c.cells = a.sel_cells + (int64_t)i * a.ld_cells;
    c.row0 = (int64_t)(qvalid ? s : 0) * a.g.cap_cells;
    return c;
}

// A operand of S: row col = head g*hpk + col (zero past hpk), dims 32*kb +
// 8*quad .. +7, scaled, fp16.
__device__ __forceinline__ void load_q_operand(const AttnArgs &a, int i, int g, int hpk, int col,
                                               int quad, half8_t (&qa)[8]) {
    const bool live = col < hpk;
    // every load is issued (a dead row reads head g*hpk), then selected
    const float4 *qp = reinterpret_cast<const float4 *>(
        a.q + ((int64_t)i * a.n_head + g * hpk + (live ? col : 0)) * kHeadDim + 8 * quad);
    float4 raw[16];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        raw[2 * kb] = qp[8 * kb];
        raw[2 * kb + 1] = qp[8 * kb + 1];
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        const float4 u = raw[2 * kb], v = raw[2 * kb + 1];
        const float x[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = live ? x[e] * a.scale : 0.0f;
        qa[kb] = to_half8(y);
    }
}

// Online softmax of a chunk's two S tiles (column col of tile t is chunk
// cell 16t + col; -inf where there is no cell) into the running state, and
// P to LDS.
template <typename Tail>
__device__ __forceinline__ void softmax_chunk(const f32x4 (&sacc)[2], int col, int quad,
                                              float (&m_run)[4], float (&l_run)[4],
                                              f32x4 (&o)[16], Tail &t) {
    float corr[4];
    bool moved = false;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const float mx = row16_max(fmaxf(sacc[0][jj], sacc[1][jj]));
        const float m_new = fmaxf(m_run[jj], mx);
        const float p0 = m_new == -INFINITY ? 0.f : __expf(sacc[0][jj] - m_new);
        const float p1 = m_new == -INFINITY ? 0.f : __expf(sacc[1][jj] - m_new);
        corr[jj] = m_run[jj] == -INFINITY ? 0.f : __expf(m_run[jj] - m_new);
        moved |= m_new != m_run[jj];
        l_run[jj] = l_run[jj] * corr[jj] + row16_sum(p0 + p1);
        m_run[jj] = m_new;
        t.p[4 * quad + jj][col] = (_Float16)p0;
        t.p[4 * quad + jj][16 + col] = (_Float16)p1;
    }
    // a row whose max did not move has corr 1 (or o still 0): the rescale
    // is skipped when no row of the wavefront moved
    if (__ballot(moved)) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) o[tt][jj] *= corr[jj];
    }
}

// O += P V from LDS for the output tiles TT0 .. TT0 + NTT - 1 (dims 16*tt ..),
// whose V rows are vt[16*(tt - TT0) ..]: A = P[row col][cells 8*quad ..],
// B = V[cells 8*quad ..][dim].
template <int TT0, int NTT, typename Tail>
__device__ __forceinline__ void pv_tiles(const Tail &t, int col, int quad, f32x4 (&o)[16]) {
    const half8_t pa = *reinterpret_cast<const half8_t *>(&t.p[col][8 * quad]);
#pragma unroll
    for (int tt = TT0; tt < TT0 + NTT; ++tt) {
        // vt rows are 8-byte aligned: two 8-byte reads
        const uint2 *vp = reinterpret_cast<const uint2 *>(&t.vt[16 * (tt - TT0) + col][8 * quad]);
        const uint2 lo = vp[0], hi = vp[1];
        const half8_t vb = __builtin_bit_cast(half8_t, u32x4{lo.x, lo.y, hi.x, hi.y});
        o[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vb, o[tt], 0, 0, 0);
    }
}

// Merge the four wavefronts' states, a quarter of the dims at a time, and
// write the heads of KV head g.
template <typename W>
__device__ __forceinline__ void merge_store(const AttnArgs &a, int i, int g, int hpk,
                                            W (&sw)[kPWaves], const f32x4 (&o)[16],
                                            const float (&m_run)[4], const float (&l_run)[4]) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int col = lane & 15, quad = lane >> 4;
    auto &t = sw[wave_id()].t;
    if (col == 0) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            t.m[4 * quad + jj] = m_run[jj];
            t.l[4 * quad + jj] = l_run[jj];
        }
    }
#pragma unroll
    for (int part = 0; part < 4; ++part) {
        __syncthreads();
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            const int tt = part * 4 + t4;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) t.o[4 * quad + jj][16 * t4 + col] = o[tt][jj];
        }
        __syncthreads();
        // thread: head row r = tid / 16 (16 rows), dims 4*(tid%16) .. +3 of the quarter
        const int r = tid >> 4, d0 = (tid & 15) * 4;
        if (r < hpk) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kPWaves; ++w) M = fmaxf(M, sw[w].t.m[r]);
            float L = 0.f, wt[kPWaves];
#pragma unroll
            for (int w = 0; w < kPWaves; ++w) {
                wt[w] = sw[w].t.m[r] == -INFINITY ? 0.f : __expf(sw[w].t.m[r] - M);
                L += sw[w].t.l[r] * wt[w];
            }
            float *outp = a.out + ((int64_t)i * a.n_head + g * hpk + r) * kHeadDim + part * 64 + d0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float acc = 0.f;
#pragma unroll
                for (int w = 0; w < kPWaves; ++w) acc += sw[w].t.o[r][d0 + e] * wt[w];
                outp[e] = L > 0.f ? acc / L : 0.f;
            }
        }
    }
}

// ---- q8_0 rows, staged through LDS ----

// Load k (0..16) of a chunk: loads 0..7 are K rows of slots 4k .. 4k+3 (16
// lanes a row, bytes 0..255), loads 8..15 the same for V, load 16 the last
// 16 bytes of the K row (lanes < 32) or V row (lanes >= 32) of slot lane%32.
// K and V pass through the same stage, at byte slot*272 + part*16.
__device__ __forceinline__ int piece_slot(int k, int lane) {
    return k < 16 ? 4 * (k & 7) + (lane >> 4) : (lane & 31);
}
__device__ __forceinline__ int piece_kv(int k, int lane) { return k < 16 ? (k >> 3) : (lane >> 5); }
__device__ __forceinline__ int piece_part(int k, int lane) { return k < 16 ? (lane & 15) : 16; }

// Workgroup id -> (query, KV head): ids are dealt to the 8 XCDs
// round-robin, so the KV heads of one query get ids 8 apart, on one XCD at
// about the same time, where the cache line their adjacent rows share is
// read once.  False for the padding of the grid.
__device__ __forceinline__ bool unit_of(const AttnArgs &a, int &i, int &g) {
    const int id = blockIdx.x, per = 8 * a.n_head_kv;
    const int r = id % per;
    g = r >> 3;
    i = (id / per) * 8 + (r & 7);
    return i < a.n_q;
}

// 1-D grid of ceil(n_q / 8) * 8 * n_head_kv, 256 threads, two workgroups
// per CU (LDS and registers are sized for two wavefronts per SIMD).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_prefill_q8(
    AttnArgs a) {
    __shared__ Q8Wave sw[kPWaves];
    int i, g;
    if (!unit_of(a, i, g)) return;
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & (kWave - 1);
    const int col = lane & 15, quad = lane >> 4;  // MFMA column / k-quarter
    const int hpk = a.n_head / a.n_head_kv;
    Q8Wave &ws = sw[wave];
    const QueryCtx qc = query_ctx(a, i);
    const uint8_t *stage = reinterpret_cast<const uint8_t *>(ws.stage);

    half8_t qa[8];
    load_q_operand(a, i, g, hpk, col, quad, qa);
    f32x4 o[16];  // O[row 4*quad + jj][dim 16*tt + col]
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) o[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[4], l_run[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        m_run[jj] = -INFINITY;
        l_run[jj] = 0.f;
    }

    // Lane l (and l + 32) holds the cell of chunk slot l % 32, -1 past the
    // list; the index is clamped so that every load is issued.
    auto chunk_cell = [&](int c0) {
        const int cc = c0 + (lane & 31);
        const int v = qc.cells[min(cc, a.ld_cells - 1)];
        return cc < qc.n ? v : -1;
    };
    // Row of a cell; a cell that is not present reads the sequence's cell 0.
    auto row_of = [&](int cell) {
        const bool ok = cell >= 0 && cell < qc.n_present;
        // (the row index fits 32 bits: the host rejects caches of 2^31 rows)
        return (uint32_t)((qc.row0 + (ok ? cell : 0)) * a.n_head_kv + g);
    };
    // Loads K0 .. K1-1 of the chunk whose slot rows the lanes hold.
    auto issue = [&](uint32_t row, u32x4(&R)[17], auto k0, auto k1) {
#pragma unroll
        for (int k = decltype(k0)::value; k < decltype(k1)::value; ++k) {
            const uint32_t r = (uint32_t)__shfl((int)row, piece_slot(k, lane));
            const uint8_t *base = static_cast<const uint8_t *>(piece_kv(k, lane) ? a.v : a.k);
            R[k] = *reinterpret_cast<const u32x4 *>(base + (uint64_t)r * kQ8Row +
                                                    piece_part(k, lane) * 16);
        }
    };
    auto put = [&](int k, const u32x4 &v) {
        const int at = piece_slot(k, lane) * kQ8Row + piece_part(k, lane) * 16;
        *reinterpret_cast<u32x4 *>(ws.stage + at / 4) = v;
    };
    using K0 = std::integral_constant<int, 0>;
    using K8 = std::integral_constant<int, 8>;
    using K17 = std::integral_constant<int, 17>;

    u32x4 R[17];
    int c0 = wave * kPChunk;
    int cur = -1, nxt = -1;
    if (c0 < qc.n) {
        cur = chunk_cell(c0);
        nxt = chunk_cell(c0 + kStride);
        issue(row_of(cur), R, K0{}, K17{});
    }
    for (; c0 < qc.n; c0 += kStride) {
        const bool more = c0 + kStride < qc.n;
        // K rows of chunk c0 to the stage (the previous chunk's V reads are
        // done), then the next chunk's K in flight
        wave_sync_lds();
#pragma unroll
        for (int k = 0; k < 8; ++k) put(k, R[k]);
        if (lane < 32) put(16, R[16]);
        const uint64_t okmask =
            __ballot(lane < 32 && cur >= 0 && cur < qc.n_present) & 0xffffffffull;
        if (more) issue(row_of(nxt), R, K0{}, K8{});
        wave_sync_lds();

        // S tiles: column col of tile t is chunk slot 16t + col
        f32x4 sacc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint8_t *krow = stage + (16 * t + col) * kQ8Row;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                uint32_t lo, hi;
                staged_slice(krow, kb * 4 + quad, lo, hi);
                half2_t h[4];
                int8x4_to_half(lo, h[0], h[1]);
                int8x4_to_half(hi, h[2], h[3]);
                const half8_t kop = {h[0][0], h[0][1], h[1][0], h[1][1],
                                     h[2][0], h[2][1], h[3][0], h[3][1]};
                const f32x4 r = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    qa[kb], kop, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                const float d =
                    (float)__builtin_bit_cast(_Float16, (uint16_t)staged_scale(krow, kb));
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) acc[jj] = __builtin_fmaf(d, r[jj], acc[jj]);
            }
            if (!((okmask >> (16 * t + col)) & 1))
                acc = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            sacc[t] = acc;
        }
        softmax_chunk(sacc, col, quad, m_run, l_run, o, ws.t);

        // V rows to the stage (S has read the K rows), then the next chunk's
        // V and both 16-byte tails in flight
        wave_sync_lds();
#pragma unroll
        for (int k = 8; k < 16; ++k) put(k, R[k]);
        if (lane >= 32) put(16, R[16]);
        int nxt2 = -1;
        if (more) {
            issue(row_of(nxt), R, K8{}, K17{});
            nxt2 = chunk_cell(c0 + 2 * kStride);
        }
        wave_sync_lds();

        // V to LDS transposed, 128 dims at a time: vt[dim - 128h][cell], the
        // lane's two cells (2*col, 2*col + 1) as one fp16 pair per dim; a cell
        // that is not present gets scale 0 (its int8 are finite).  The four
        // quarter-waves write rows 8 apart at once, in different banks.
        const uint8_t *v0 = stage + (2 * col) * kQ8Row;
        const uint8_t *v1 = v0 + kQ8Row;
        const bool ok0 = (okmask >> (2 * col)) & 1, ok1 = (okmask >> (2 * col + 1)) & 1;
        auto transpose_half = [&](auto hh) {
            constexpr int h = decltype(hh)::value;
#pragma unroll
            for (int q = 4 * h; q < 4 * h + 4; ++q) {
                const int j = q * 4 + quad;  // dims 8j .. 8j+7, block q
                uint32_t lo0, hi0, lo1, hi1;
                staged_slice(v0, j, lo0, hi0);
                staged_slice(v1, j, lo1, hi1);
                const uint32_t s0 = ok0 ? staged_scale(v0, q) : 0u;
                const uint32_t s1 = ok1 ? staged_scale(v1, q) : 0u;
                const half2_t dd = as_half2(s0 | (s1 << 16));
                // interleave the two cells' bytes: (c0 e, c1 e, c0 e+1, c1 e+1)
                const uint32_t w[4] = {__builtin_amdgcn_perm(lo1, lo0, 0x05010400u),
                                       __builtin_amdgcn_perm(lo1, lo0, 0x07030602u),
                                       __builtin_amdgcn_perm(hi1, hi0, 0x05010400u),
                                       __builtin_amdgcn_perm(hi1, hi0, 0x07030602u)};
                const int row = 8 * j - 128 * h;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    half2_t h0, h1;
                    int8x4_to_half(w[c], h0, h1);
                    *reinterpret_cast<uint32_t *>(&ws.t.vt[row + 2 * c][2 * col]) =
                        as_u32(h0 * dd);
                    *reinterpret_cast<uint32_t *>(&ws.t.vt[row + 2 * c + 1][2 * col]) =
                        as_u32(h1 * dd);
                }
            }
        };
        transpose_half(std::integral_constant<int, 0>{});
        wave_sync_lds();
        pv_tiles<0, 8>(ws.t, col, quad, o);
        wave_sync_lds();
        transpose_half(std::integral_constant<int, 1>{});
        wave_sync_lds();
        pv_tiles<8, 8>(ws.t, col, quad, o);
        cur = nxt;
        nxt = nxt2;
    }
    merge_store(a, i, g, hpk, sw, o, m_run, l_run);
}

// ---- rows gathered per lane: f32 and f16 caches, and q8_0 through a cell table ----

// Same grid as k_attn_prefill_q8.
template <int KVT>
__global__ __launch_bounds__(256) void k_attn_prefill_rows(AttnArgs a) {
    __shared__ RowWave sw[kPWaves];
    __shared__ int32_t s_cells[kCellCap];  // the query's cell list (its first kCellCap)
    int i, g;
    if (!unit_of(a, i, g)) return;
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & (kWave - 1);
    const int col = lane & 15, quad = lane >> 4;
    const int hpk = a.n_head / a.n_head_kv;
    WaveTail &ws = sw[wave].t;
    const QueryCtx qc = query_ctx(a, i);

    half8_t qa[8];
    load_q_operand(a, i, g, hpk, col, quad, qa);
    f32x4 o[16];
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) o[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[4], l_run[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        m_run[jj] = -INFINITY;
        l_run[jj] = 0.f;
    }

    for (int x = tid; x < qc.n && x < kCellCap; x += 256) s_cells[x] = qc.cells[x];
    __syncthreads();
    auto cell_at = [&](int cc) { return cc < kCellCap ? s_cells[cc] : qc.cells[cc]; };
    for (int c0 = wave * kPChunk; c0 < qc.n; c0 += kStride) {
        const int c1 = min(qc.n, c0 + kPChunk);
        // S tiles: column col of tile t is cell c0 + 16t + col
        f32x4 sacc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int cc = c0 + 16 * t + col;
            const int cell = cc < c1 ? cell_at(cc) : -1;
            const bool ok = cell >= 0 && cell < qc.n_present;
            const int64_t row = cell_row_at(a.g, qc.row0 + (ok ? cell : 0)) * a.n_head_kv + g;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                float x[8];
                dequant<KVT>(load_raw<KVT>(a.k, row, kb * 4 + quad), kb * 4 + quad, x);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kb], to_half8(x), acc, 0, 0, 0);
            }
            if (!ok) acc = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            sacc[t] = acc;
        }
        softmax_chunk(sacc, col, quad, m_run, l_run, o, ws);
        // V to LDS, transposed; zeros for cells that are not present
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int cc = c0 + 2 * col + u;
            const int cell = cc < c1 ? cell_at(cc) : -1;
            const bool ok = cell >= 0 && cell < qc.n_present;
            const int64_t row = cell_row_at(a.g, qc.row0 + (ok ? cell : 0)) * a.n_head_kv + g;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int j = q * 4 + quad;
                float x[8];
                dequant<KVT>(load_raw<KVT>(a.v, row, j), j, x);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    ws.vt[8 * j + e][2 * col + u] = ok ? (_Float16)x[e] : (_Float16)0.f;
            }
        }
        wave_sync_lds();
        pv_tiles<0, 16>(ws, col, quad, o);
        wave_sync_lds();
    }
    merge_store(a, i, g, hpk, sw, o, m_run, l_run);
}

}  // namespace

size_t attn_prefill_ws_bytes(int, int, int) { return 0; }

hipError_t launch_attn_prefill(const AttnArgs &a, hipStream_t st) {
    if (a.n_q <= 0) return hipSuccess;
    const dim3 grid((a.n_q + 7) / 8 * 8 * a.n_head_kv);
    if (a.kv_type == QSA_KV_F32)
        hipLaunchKernelGGL(k_attn_prefill_rows<QSA_KV_F32>, grid, dim3(256), 0, st, a);
    else if (a.kv_type == QSA_KV_F16)
        hipLaunchKernelGGL(k_attn_prefill_rows<QSA_KV_F16>, grid, dim3(256), 0, st, a);
    else if (a.g.rows)  // a cell table: rows gathered per lane through it
        hipLaunchKernelGGL(k_attn_prefill_rows<QSA_KV_Q8_0>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(k_attn_prefill_q8, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace qsa
