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

// Lane l (and l + 32) holds the cell of chunk slot l % 32, -1 past the
// list; the index is clamped so that every load is issued.
__device__ __forceinline__ int chunk_cell_of(const AttnArgs &a, const QueryCtx &qc, int lane,
                                             int c0) {
    const int cc = c0 + (lane & 31);
    const int v = qc.cells[min(cc, a.ld_cells - 1)];
    return cc < qc.n ? v : -1;
}
// Row of a cell; a cell that is not present reads the sequence's cell 0.
// (The row index fits 32 bits: the host rejects caches of 2^31 rows.)
__device__ __forceinline__ uint32_t row_of_cell(const AttnArgs &a, const QueryCtx &qc, int g,
                                                int cell) {
    const bool ok = cell >= 0 && cell < qc.n_present;
    return (uint32_t)((qc.row0 + (ok ? cell : 0)) * a.n_head_kv + g);
}
// Loads K0 .. K1-1 of the chunk whose slot rows the lanes hold.
template <typename K0, typename K1>
__device__ __forceinline__ void issue_pieces(const AttnArgs &a, uint32_t row, int lane,
                                             u32x4 (&R)[17], K0, K1) {
#pragma unroll
    for (int k = K0::value; k < K1::value; ++k) {
        const uint32_t r = (uint32_t)__shfl((int)row, piece_slot(k, lane));
        const uint8_t *base = static_cast<const uint8_t *>(piece_kv(k, lane) ? a.v : a.k);
        R[k] = *reinterpret_cast<const u32x4 *>(base + (uint64_t)r * kQ8Row +
                                                piece_part(k, lane) * 16);
    }
}

// One wavefront's walk over chunks c0 = first, first + step, ... < end of a
// cell source, with its 16 A rows qa, into the online-softmax state (m_run,
// l_run, o).  Src supplies, for lane l: at(c0), the handle of chunk slot
// l % 32 (prefetched two chunks ahead); row(h), its K/V row; ok(h), whether
// it is a cell to attend; and visible(cur, okmask, col, quad, c0), bit t set
// when the lane's S rows may see slot 16t + col (okmask: the chunk's ok slots).
template <class Src>
__device__ __forceinline__ void q8_walk(const AttnArgs &a, Q8Wave &ws, const half8_t (&qa)[8],
                                        int c0, int step, int end, const Src &src,
                                        f32x4 (&o)[16], float (&m_run)[4], float (&l_run)[4]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int col = lane & 15, quad = lane >> 4;  // MFMA column / k-quarter
    const uint8_t *stage = reinterpret_cast<const uint8_t *>(ws.stage);
    auto issue = [&](uint32_t row, u32x4(&R)[17], auto k0, auto k1) {
        issue_pieces(a, row, lane, R, k0, k1);
    };
    auto put = [&](int k, const u32x4 &v) {
        const int at = piece_slot(k, lane) * kQ8Row + piece_part(k, lane) * 16;
        *reinterpret_cast<u32x4 *>(ws.stage + at / 4) = v;
    };
    using K0 = std::integral_constant<int, 0>;
    using K8 = std::integral_constant<int, 8>;
    using K17 = std::integral_constant<int, 17>;

    u32x4 R[17];
    typename Src::Handle cur = src.none(), nxt = src.none();
    if (c0 < end) {
        cur = src.at(c0);
        nxt = src.at(c0 + step);
        issue(src.row(cur), R, K0{}, K17{});
    }
    for (; c0 < end; c0 += step) {
        const bool more = c0 + step < end;
        // K rows of chunk c0 to the stage (the previous chunk's V reads are
        // done), then the next chunk's K in flight
        wave_sync_lds();
#pragma unroll
        for (int k = 0; k < 8; ++k) put(k, R[k]);
        if (lane < 32) put(16, R[16]);
        const uint64_t okmask = __ballot(lane < 32 && src.ok(cur)) & 0xffffffffull;
        const uint32_t vis = src.visible(cur, okmask, col, quad, c0);
        if (more) issue(src.row(nxt), R, K0{}, K8{});
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
            if (!((vis >> t) & 1)) acc = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            sacc[t] = acc;
        }
        softmax_chunk(sacc, col, quad, m_run, l_run, o, ws.t);

        // V rows to the stage (S has read the K rows), then the next chunk's
        // V and both 16-byte tails in flight
        wave_sync_lds();
#pragma unroll
        for (int k = 8; k < 16; ++k) put(k, R[k]);
        if (lane >= 32) put(16, R[16]);
        typename Src::Handle nxt2 = src.none();
        if (more) {
            issue(src.row(nxt), R, K8{}, K17{});
            nxt2 = src.at(c0 + 2 * step);
        }
        wave_sync_lds();

        // V to LDS transposed, 128 dims at a time: vt[dim - 128h][cell], the
        // lane's two cells (2*col, 2*col + 1) as one fp16 pair per dim; a cell
        // that is not attended gets scale 0 (its int8 are finite).  The four
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
}

// A query's own cell list: handles are cells (-1 past the list).
struct ListSrc {
    typedef int Handle;
    const AttnArgs &a;
    const QueryCtx &qc;
    int g, lane;
    __device__ Handle none() const { return -1; }
    __device__ Handle at(int c0) const { return chunk_cell_of(a, qc, lane, c0); }
    __device__ uint32_t row(Handle h) const { return row_of_cell(a, qc, g, h); }
    __device__ bool ok(Handle h) const { return h >= 0 && h < qc.n_present; }
    __device__ uint32_t visible(Handle, uint64_t okm, int col, int, int) const {
        return (uint32_t)((okm >> col) & 1) | (uint32_t)(((okm >> (16 + col)) & 1) << 1);
    }
};

__device__ __forceinline__ void init_state(f32x4 (&o)[16], float (&m_run)[4], float (&l_run)[4]) {
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) o[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        m_run[jj] = -INFINITY;
        l_run[jj] = 0.f;
    }
}

// 1-D grid of ceil(n_q / 8) * 8 * n_head_kv, 256 threads, two workgroups
// per CU (LDS and registers are sized for two wavefronts per SIMD).  The
// four wavefronts take the chunks of the query's list in turn.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_prefill_q8(
    AttnArgs a) {
    __shared__ Q8Wave sw[kPWaves];
    int i, g;
    if (!unit_of(a, i, g)) return;
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
    const int col = lane & 15, quad = lane >> 4;
    const int hpk = a.n_head / a.n_head_kv;
    const QueryCtx qc = query_ctx(a, i);
    half8_t qa[8];
    load_q_operand(a, i, g, hpk, col, quad, qa);
    f32x4 o[16];  // O[row 4*quad + jj][dim 16*tt + col]
    float m_run[4], l_run[4];
    init_state(o, m_run, l_run);
    const ListSrc src{a, qc, g, lane};
    q8_walk(a, sw[wave], qa, wave * kPChunk, kStride, qc.n, src, o, m_run, l_run);
    merge_store(a, i, g, hpk, sw, o, m_run, l_run);
}

// ---- several decode tokens of a sequence over the union of their lists ----
//
// Tokens are taken t_group at a time (the last group may be shorter).  Per
// group, k_union_build lists every K/V row any token of the group attends
// (ascending) with a bit per token that holds it; k_attn_union_q8 walks that
// union in runs of kURun rows, each workgroup staging a run's rows once for
// all tokens of the group: wavefront w takes the query heads of KV head g of
// 16 / hpk tokens as its 16 A rows (8 heads of 2 tokens for 16 heads over 2
// KV heads), scores every staged row, and a row a token does not hold gets
// -inf before that token's softmax.  Each (token, head) keeps its own online
// softmax; its per-run partial states are merged by k_union_combine.

constexpr int kUnionNT = 1024;
constexpr int kUnionMaxT = 8;
constexpr int kUnionCap = kUnionMaxEntries;  // union entries per group: t_group * ld_cells at most
constexpr int kURun = 2 * kPChunk;  // union rows per attention workgroup

// Exclusive prefix sum over the workgroup (kUnionNT threads) and the total.
__device__ __forceinline__ uint32_t union_scan(uint32_t v, uint32_t *s_w, uint32_t &total) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const uint32_t inc = wave_incl_scan_u32(v);
    if (lane == kWave - 1) s_w[wave] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kUnionNT / kWave; ++w) {
        const uint32_t x = s_w[w];
        before += w < wave ? x : 0u;
        all += x;
    }
    __syncthreads();  // s_w may be reused
    total = all;
    return before + inc - v;
}

// grid (n_groups), kUnionNT threads.  Token t's valid cells (in 0 ..
// n_present-1 of its sequence, the first n_sel entries of its list) are
// keyed (cell << 3) | t.  If every valid token of the group is in one
// sequence and every list strictly ascends, the lists are merged (pairs of
// adjacent runs by merge path, log2 t_group rounds) and equal cells fold into
// one entry with the OR of their token bits; otherwise the lists are
// concatenated, one entry and one bit per (token, cell), which attends
// exactly the same cells.
__global__ __launch_bounds__(kUnionNT) void k_union_build(AttnArgs a, UnionArgs u) {
    __shared__ uint32_t s_buf[2][kUnionCap];
    __shared__ int s_off[kUnionMaxT + 1];  // start of token t's entries; s_off[T] = total
    __shared__ int s_seq[kUnionMaxT];      // token t's sequence (-1: none, or no valid cell)
    __shared__ int s_n[kUnionMaxT];
    __shared__ int s_np[kUnionMaxT];
    __shared__ uint32_t s_w[kUnionNT / kWave];
    __shared__ int s_bad;
    QSA_STAMP(0);
    const int gi = blockIdx.x, tid = threadIdx.x;
    const int q0 = gi * u.t_group;
    const int T = min(u.t_group, a.n_q - q0);
    const int ld = a.ld_cells;
    // 1. the group's lists as one flat range of T*ld entries (token-major),
    // staged in LDS with coalesced loads while threads 0 .. T-1 fetch their
    // token's sequence and sizes; thread tid then takes the kUPer
    // consecutive entries from tid*kUPer (an odd stride: no bank conflicts)
    constexpr int kUPer = kUnionCap / kUnionNT + 1;
    const int flat = T * ld;
    for (int e = tid; e < flat; e += kUnionNT)
        s_buf[1][e] = (uint32_t)a.sel_cells[(int64_t)q0 * ld + e];
    if (tid < T) {
        const int s = a.q_seq[q0 + tid];
        const bool qvalid = s >= 0 && s < a.g.n_seq;
        const int n_raw = qvalid ? a.n_sel[q0 + tid] : 0;
        int64_t np = qvalid ? a.g.n_cells[s] : 0;
        np = np < a.g.cap_cells ? np : a.g.cap_cells;
        s_seq[tid] = qvalid ? s : -1;
        s_n[tid] = n_raw < 0 ? 0 : (n_raw > ld ? ld : n_raw);
        s_np[tid] = (int)np;
    }
    if (tid == 0) s_bad = 0;
    __syncthreads();
    QSA_STAMP(1);  // lists staged
    const int e_first = tid * kUPer;
    int t_first = e_first / ld;  // token of the first entry; 17 < ld, so one step at most
    const int j_first = e_first - t_first * ld;
    uint32_t valid = 0, cnt = 0;  // bit k: entry tid*kUPer + k is a valid cell
#pragma unroll
    for (int k = 0; k < kUPer; ++k) {
        const int e = e_first + k;
        const bool wrap = j_first + k >= ld;
        const int t = t_first + (wrap ? 1 : 0), j = j_first + k - (wrap ? ld : 0);
        if (e < flat) {
            const int cell = (int)s_buf[1][e];
            if (j < s_n[t] && cell >= 0 && cell < s_np[t]) {
                valid |= 1u << k;
                ++cnt;
            }
        }
    }
    uint32_t total;
    uint32_t at = union_scan(cnt, s_w, total);
    // token t's entries start at the compacted index of flat position t*ld:
    // the thread whose range holds that position records it
    for (int t = 1; t < T; ++t) {
        const int d = t * ld - tid * kUPer;
        if (d >= 0 && d < kUPer) s_off[t] = (int)(at + __popc(valid & ((1u << d) - 1u)));
    }
    if (tid == 0) {
        s_off[0] = 0;
        s_off[T] = (int)total;
    }
    __syncthreads();
    if (tid < T && s_off[tid + 1] == s_off[tid]) s_seq[tid] = -1;  // no valid cell
#pragma unroll
    for (int k = 0; k < kUPer; ++k) {
        if (!((valid >> k) & 1u)) continue;
        const int t = t_first + (j_first + k >= ld ? 1 : 0);
        s_buf[0][at++] = (s_buf[1][e_first + k] << 3) | (uint32_t)t;
    }
    __syncthreads();
    QSA_STAMP(2);  // compacted
    const int E = s_off[T];
    int32_t *urow = u.urow + (int64_t)gi * u.cap;
    uint8_t *umask = u.umask + (int64_t)gi * u.cap;
    // 2. merge only lists of one sequence that strictly ascend
    int s0 = -1;
    for (int t = 0; t < T; ++t) {
        const int st = s_seq[t];
        if (st >= 0) {
            if (s0 < 0) s0 = st;
            else if (st != s0) s_bad = 1;  // (benign race: every writer writes 1)
        }
    }
    for (int e = tid; e < E; e += kUnionNT) {
        const uint32_t k = s_buf[0][e];
        const int t = (int)(k & 7u);
        if (e > s_off[t] && (s_buf[0][e - 1] >> 3) >= (k >> 3)) s_bad = 1;
    }
    __syncthreads();
    if (s_bad) {
        for (int e = tid; e < E; e += kUnionNT) {
            const uint32_t k = s_buf[0][e];
            const int t = (int)(k & 7u);
            urow[e] = (int32_t)((int64_t)s_seq[t] * a.g.cap_cells + (k >> 3));
            umask[e] = (uint8_t)(1u << t);
        }
        if (tid == 0) u.n_union[gi] = E;
        return;
    }
    QSA_STAMP(3);  // checked
    // 3. merge path: runs [s_off[t], s_off[t+1]) merged two by two; a merged
    // pair keeps the place of the pair, so the run bounds just halve
    int src = 0;
    for (int width = 1; width < T; width *= 2) {
        const int per = (E + kUnionNT - 1) / kUnionNT;
        for (int p = tid * per; p < min(E, tid * per + per);) {
            // the pair holding output position p: runs r0 = 2*width*k .. +width, then the next width
            int r0 = 0;
            while (r0 + 2 * width <= T && s_off[min(r0 + 2 * width, T)] <= p) r0 += 2 * width;
            const int a0 = s_off[r0], a1 = s_off[min(r0 + width, T)], b1 = s_off[min(r0 + 2 * width, T)];
            const uint32_t *A = s_buf[src] + a0, *B = s_buf[src] + a1;
            const int na = a1 - a0, nb = b1 - a1;
            const int d = p - a0;
            int lo = max(0, d - nb), hi = min(d, na);
            while (lo < hi) {  // A elements among the first d outputs (keys are distinct)
                const int mid = (lo + hi) >> 1;
                if (A[mid] < B[d - mid - 1]) lo = mid + 1;
                else hi = mid;
            }
            int i = lo, j = d - lo;
            const int stop = min(min(E, tid * per + per), b1);
            for (; p < stop; ++p) {
                const bool take_a = i < na && (j >= nb || A[i] < B[j]);
                s_buf[src ^ 1][p] = take_a ? A[i++] : B[j++];
            }
        }
        __syncthreads();
        src ^= 1;
    }
    QSA_STAMP(4);  // merged
    // 4. fold equal cells: a first occurrence gathers the bits of its run
    const uint32_t *M = s_buf[src];
    const int per = (E + kUnionNT - 1) / kUnionNT;
    const int e0 = min(E, tid * per), e1 = min(E, tid * per + per);
    uint32_t n_first = 0;
    for (int e = e0; e < e1; ++e) n_first += (e == 0 || (M[e] >> 3) != (M[e - 1] >> 3)) ? 1u : 0u;
    uint32_t n_union;
    uint32_t ui = union_scan(n_first, s_w, n_union);
    for (int e = e0; e < e1; ++e) {
        const uint32_t cell = M[e] >> 3;
        if (e > 0 && (M[e - 1] >> 3) == cell) continue;
        uint32_t bits = 0;
        for (int f = e; f < E && (M[f] >> 3) == cell; ++f) bits |= 1u << (M[f] & 7u);
        urow[ui] = (int32_t)((int64_t)s0 * a.g.cap_cells + cell);
        umask[ui] = (uint8_t)bits;
        ++ui;
    }
    if (tid == 0) u.n_union[gi] = (int32_t)n_union;
    QSA_STAMP(5);
}

// The union's rows as a cell source: handles are rows (-1 past the run); the
// token bits of the run's rows sit in LDS (bits[e - c_begin]).
struct UnionSrc {
    typedef int Handle;
    const int32_t *urow;
    const uint8_t *bits;
    int c_begin, end, g, n_head_kv, tok0, hpk;  // (all wavefront-uniform)
    __device__ Handle none() const { return -1; }
    __device__ Handle at(int c0) const {
        // (a clamped, unconditional load; end >= 1 whenever a chunk is walked)
        const int e = c0 + (int)(threadIdx.x & 31);
        const int r = urow[min(e, max(end - 1, 0))];
        return e < end ? r : -1;
    }
    __device__ uint32_t row(Handle h) const {
        return (uint32_t)(h < 0 ? 0 : h) * (uint32_t)n_head_kv + (uint32_t)g;
    }
    __device__ bool ok(Handle h) const { return h >= 0; }
    __device__ uint32_t visible(Handle, uint64_t okm, int col, int quad, int c0) const {
        // the lane's S rows 4*quad .. +3 belong to one token (hpk >= 4)
        const int tok = tok0 + 4 * quad / hpk;
        const int e0 = c0 - c_begin + col;  // (slots past the run are not ok)
        const uint32_t b0 = (uint32_t)(okm >> col) & ((uint32_t)bits[e0] >> tok) & 1u;
        const uint32_t b1 =
            (uint32_t)(okm >> (16 + col)) & ((uint32_t)bits[e0 + 16] >> tok) & 1u;
        return b0 | (b1 << 1);
    }
};

// grid (n_groups * n_head_kv * n_runs * n_slices), 256 threads: workgroup
// (group gi, KV head g, run, token slice); wavefront w of slice sl takes
// tokens (4*sl + w) * tpw .. + tpw - 1 (tpw = 16 / hpk), its row col being
// head col % hpk of token col / hpk.  Each wavefront walks every chunk of the
// run and writes its rows' partial states (o[256], m, l) for the combine.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_union_q8(
    AttnArgs a, UnionArgs u) {
    __shared__ Q8Wave sw[kPWaves];
    __shared__ uint8_t s_bits[kURun + kPChunk];  // token bits of the run's rows (zero past it)
    const int hpk = a.n_head / a.n_head_kv, tpw = 16 / hpk;
    const int n_slices = (u.t_group + kPWaves * tpw - 1) / (kPWaves * tpw);
    int id = blockIdx.x;
    const int sl = id % n_slices;
    id /= n_slices;
    const int run = id % u.n_runs;
    id /= u.n_runs;
    const int g = id % a.n_head_kv, gi = id / a.n_head_kv;
    const int n = u.n_union[gi];
    const int c_begin = run * kURun, c_end = min(n, c_begin + kURun);
    if (c_begin >= c_end) return;
    const int wave = wave_id();
    int col = threadIdx.x & 15, quad = (threadIdx.x >> 4) & 3;
    const int q0 = gi * u.t_group;
    const int T = min(u.t_group, a.n_q - q0);
    const int tok0 = (sl * kPWaves + wave) * tpw;
    const uint8_t *umask = u.umask + (int64_t)gi * u.cap;
    if (threadIdx.x < kURun + kPChunk) {
        const int e = c_begin + (int)threadIdx.x;
        s_bits[threadIdx.x] = e < c_end ? umask[e] : (uint8_t)0;
    }
    __syncthreads();
    if (tok0 >= T) return;  // (no workgroup barrier follows)
    // A rows: row col = head g*hpk + col % hpk of token tok0 + col / hpk
    half8_t qa[8];
    {
        const int t = tok0 + col / hpk;
        const bool live = t < T;
        const int qi = q0 + (live ? t : 0);
        const float4 *qp = reinterpret_cast<const float4 *>(
            a.q + ((int64_t)qi * a.n_head + g * hpk + col % hpk) * kHeadDim + 8 * quad);
        float4 raw[16];
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            raw[2 * kb] = qp[8 * kb];
            raw[2 * kb + 1] = qp[8 * kb + 1];
        }
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            const float4 p0 = raw[2 * kb], p1 = raw[2 * kb + 1];
            const float x[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = live ? x[e] * a.scale : 0.0f;
            qa[kb] = to_half8(y);
        }
    }
    f32x4 o[16];
    float m_run[4], l_run[4];
    init_state(o, m_run, l_run);
    const UnionSrc src{u.urow + (int64_t)gi * u.cap, s_bits, c_begin, c_end, g,
                       a.n_head_kv, tok0, hpk};
    q8_walk(a, sw[wave], qa, c_begin, kPChunk, c_end, src, o, m_run, l_run);
    // partial states of the wavefront's rows that are tokens of the group
    // (the lane index is taken afresh: nothing per lane stays live across the walk)
    {
        const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        col = ln & 15;
        quad = ln >> 4;
    }
    const int rows = u.t_group * hpk;
    float *base = u.part + (((int64_t)gi * a.n_head_kv + g) * u.n_runs + run) * rows * kUPartStride;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int r = 4 * quad + jj;
        const int t = tok0 + r / hpk;
        if (t >= T) continue;
        float *pr = base + (int64_t)(t * hpk + r % hpk) * kUPartStride;
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) pr[16 * tt + col] = o[tt][jj];
        if (col == 0) {
            pr[kHeadDim] = m_run[jj];
            pr[kHeadDim + 1] = l_run[jj];
        }
    }
}

// grid (n_q * n_head * 4), 256 threads: workgroup (query q, head h, 64-dim
// slice) merges the partial states of q's group's runs (every run below
// ceil(n_union / kURun) was written for every token of the group: o = 0,
// m = -inf, l = 0 where the token saw no row).  Wavefront w sums runs w,
// w + 4, ... with lane = output dim; its first kUPre runs are loaded at once,
// the rest 8 at a time; the wavefronts' sums are added in a fixed order.
constexpr int kUPre = 17;
__global__ __launch_bounds__(256) void k_union_combine(AttnArgs a, UnionArgs u) {
    __shared__ float s_w[(kUnionCap + kURun - 1) / kURun];  // m of run r, then its weight
    __shared__ float s_red[4];
    __shared__ float s_acc[4][kWave];
    const int slice = blockIdx.x & 3, qh = blockIdx.x >> 2;
    const int q = qh / a.n_head, h = qh % a.n_head;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & (kWave - 1);
    const int hpk = a.n_head / a.n_head_kv, g = h / hpk;
    const int gi = q / u.t_group, t = q % u.t_group;
    const int runs = (u.n_union[gi] + kURun - 1) / kURun;
    const int rows = u.t_group * hpk;
    const float *base = u.part + ((int64_t)gi * a.n_head_kv + g) * u.n_runs * rows * kUPartStride +
                        (int64_t)(t * hpk + h % hpk) * kUPartStride;
    const int64_t stride = (int64_t)rows * kUPartStride;
    const int col = slice * kWave + lane;
    if (runs == 0) {  // no row in the group: nothing was written to merge
        if (wave == 0) a.out[((int64_t)q * a.n_head + h) * kHeadDim + col] = 0.f;
        return;
    }
    const int last = runs - 1;
    // (clamped, unconditional loads of written runs: a run past the end weighs 0)
    float pre[kUPre];
#pragma unroll
    for (int k = 0; k < kUPre; ++k) pre[k] = base[min(wave + 4 * k, last) * stride + col];
    float mloc = -INFINITY;
    for (int r = tid; r < runs; r += 256) {
        const float m = base[r * stride + kHeadDim], l = base[r * stride + kHeadDim + 1];
        const float mm = l > 0.f ? m : -INFINITY;
        s_w[r] = mm;
        mloc = fmaxf(mloc, mm);
    }
    mloc = wave_max_f32(mloc);
    if (lane == 0) s_red[wave] = mloc;
    __syncthreads();
    const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    float lw = 0.f;
    for (int r = tid; r < runs; r += 256) {
        const float m = s_w[r];
        const float w = m == -INFINITY ? 0.f : __expf(m - M);
        s_w[r] = w;
        lw += w * base[r * stride + kHeadDim + 1];
    }
    lw = wave_sum_f32(lw);
    __syncthreads();  // every M read before s_red is reused; every weight written
    if (lane == 0) s_red[wave] = lw;
    __syncthreads();
    const float L = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < kUPre; ++k) {
        const int r = wave + 4 * k;
        acc = fmaf(pre[k], r < runs ? s_w[r] : 0.f, acc);
    }
    for (int r0 = wave + 4 * kUPre; r0 < runs; r0 += 32) {
        float v[8], w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int r = r0 + 4 * k;
            v[k] = base[min(r, last) * stride + col];
            w[k] = r < runs ? s_w[r] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) acc = fmaf(v[k], w[k], acc);
    }
    s_acc[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        const float o = (s_acc[0][lane] + s_acc[1][lane]) + (s_acc[2][lane] + s_acc[3][lane]);
        a.out[((int64_t)q * a.n_head + h) * kHeadDim + col] = L > 0.f ? o / L : 0.f;
    }
}

// ---- the gather alone ----

// The row gather of k_attn_prefill_q8 without its arithmetic: the same
// grid, units and chunk walk, the same 17 loads of 16 bytes per lane and
// chunk (padding slots of a last chunk read the sequence's cell 0, as
// there), two chunks in flight.  The loaded words are XOR-folded into
// sink[workgroup % n_sink], so that the loads cannot be dropped; the fold of
// every sink word is the XOR of every 32-bit word the kernel loaded.
__global__ __launch_bounds__(256) void k_probe_gather_q8(AttnArgs a, uint32_t *sink, int n_sink) {
    int i, g;
    if (!unit_of(a, i, g)) return;
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
    const QueryCtx qc = query_ctx(a, i);
    using K0 = std::integral_constant<int, 0>;
    using K17 = std::integral_constant<int, 17>;
    uint32_t acc = 0;
    for (int c0 = wave * kPChunk; c0 < qc.n; c0 += 2 * kStride) {
        u32x4 R[2][17];
        const bool two = c0 + kStride < qc.n;
        issue_pieces(a, row_of_cell(a, qc, g, chunk_cell_of(a, qc, lane, c0)), lane, R[0], K0{},
                     K17{});
        if (two)
            issue_pieces(a, row_of_cell(a, qc, g, chunk_cell_of(a, qc, lane, c0 + kStride)),
                         lane, R[1], K0{}, K17{});
#pragma unroll
        for (int k = 0; k < 17; ++k) {
            // the tail load (k = 16) is the K row's for lanes < 32, V's above;
            // both are loaded, as in the kernel above
            acc ^= R[0][k][0] ^ R[0][k][1] ^ R[0][k][2] ^ R[0][k][3];
            if (two) acc ^= R[1][k][0] ^ R[1][k][1] ^ R[1][k][2] ^ R[1][k][3];
        }
    }
    acc ^= xor_lane<1>(acc);
    acc ^= xor_lane<2>(acc);
    acc ^= xor_lane<4>(acc);
    acc ^= xor_lane<8>(acc);
    acc ^= xor_lane<16>(acc);
    acc ^= xor_lane<32>(acc);
    if (lane == 0) fold_sink(sink, n_sink, acc);
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

QSA_STAMP_READER(attnp)

size_t union_ws_bytes(int n_q, int t_group, int n_head, int n_head_kv, int ld_cells) {
    return union_layout(nullptr, n_q, t_group, n_head, n_head_kv, ld_cells, nullptr);
}

size_t union_layout(char *base, int n_q, int t_group, int n_head, int n_head_kv, int ld_cells,
                    UnionArgs *u) {
    UnionArgs d{};
    d.t_group = t_group;
    d.n_groups = t_group > 0 ? (n_q + t_group - 1) / t_group : 0;
    d.cap = t_group * ld_cells;
    d.n_runs = (d.cap + kURun - 1) / kURun;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) / 256 * 256;
        return base ? base + at : nullptr;
    };
    d.urow = reinterpret_cast<int32_t *>(take((size_t)d.n_groups * d.cap * 4));
    d.umask = reinterpret_cast<uint8_t *>(take((size_t)d.n_groups * d.cap));
    d.n_union = reinterpret_cast<int32_t *>(take((size_t)d.n_groups * 4));
    d.part = reinterpret_cast<float *>(take((size_t)d.n_groups * n_head_kv * d.n_runs *
                                            (t_group * (n_head / n_head_kv)) * kUPartStride * 4));
    if (u) *u = d;
    return n_q > 0 ? off : 0;
}

hipError_t launch_attn_decode_union(const AttnArgs &a, int t_group, hipStream_t st) {
    if (a.n_q <= 0) return hipSuccess;
    UnionArgs u;
    union_layout(reinterpret_cast<char *>(a.ws), a.n_q, t_group, a.n_head, a.n_head_kv,
                 a.ld_cells, &u);
    hipLaunchKernelGGL(k_union_build, dim3(u.n_groups), dim3(kUnionNT), 0, st, a, u);
    const int hpk = a.n_head / a.n_head_kv, tpw = 16 / hpk;
    const int n_slices = (t_group + kPWaves * tpw - 1) / (kPWaves * tpw);
    const int grid = u.n_groups * a.n_head_kv * u.n_runs * n_slices;
    hipLaunchKernelGGL(k_attn_union_q8, dim3(grid), dim3(256), 0, st, a, u);
    hipLaunchKernelGGL(k_union_combine, dim3(a.n_q * a.n_head * 4), dim3(256), 0, st, a, u);
    return hipGetLastError();
}

hipError_t launch_probe_gather_prefill(const AttnArgs &a, uint32_t *sink, int n_sink,
                                       hipStream_t st) {
    if (a.n_q <= 0) return hipSuccess;
    const dim3 grid((a.n_q + 7) / 8 * 8 * a.n_head_kv);
    hipLaunchKernelGGL(k_probe_gather_q8, grid, dim3(256), 0, st, a, sink, n_sink);
    return hipGetLastError();
}

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
