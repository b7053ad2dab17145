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
//        v_mfma_f32_16x16x32_f16; a k-step is one q8_0 block, dequantised to
//        fp16 in registers straight into the B operand (8 dims per lane);
//   online softmax on S in the accumulator layout (a head row's 16 columns
//        sit in one 16-lane DPP row);
//   O += P V : P goes through LDS to the A layout, V is staged transposed in
//        LDS as fp16 [dim][cell] so each B operand is one 16-byte read.
// Operands are rounded to fp16 (Q * scale, K, V, P); sums and the softmax
// state are fp32.
#include "kv_rows.h"
#include "qsa_internal.h"
#include "wave_ops.h"

namespace qsa {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPChunk = 32;  // cells per chunk
constexpr int kPWaves = 4;
constexpr int kCellCap = 4096;  // cell indices held in LDS; the rest are read directly

struct PrefAttnWave {
    union {
        _Float16 vt[kHeadDim][kPChunk];  // V of the chunk, transposed
        float o[16][kHeadDim / 4];       // merge: a quarter of the dims at a time
    };
    _Float16 p[16][kPChunk];  // probabilities, [head row][cell]
    float m[16], l[16];
};

__device__ __forceinline__ half8_t to_half8(const float (&x)[8]) {
    half8_t h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (_Float16)x[e];
    return h;
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

// grid (n_head_kv, n_q), 256 threads.
template <int KVT>
__global__ __launch_bounds__(256) void k_attn_prefill(AttnArgs a) {
    __shared__ PrefAttnWave sw[kPWaves];
    __shared__ int32_t s_cells[kCellCap];  // the query's cell list (its first kCellCap)
    const int g = blockIdx.x, i = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & (kWave - 1);
    const int col = lane & 15, quad = lane >> 4;  // MFMA column / k-quarter
    const int hpk = a.n_head / a.n_head_kv;
    PrefAttnWave &ws = sw[wave];

    const int s = a.q_seq[i];
    const bool qvalid = s >= 0 && s < a.g.n_seq;
    int n = qvalid ? a.n_sel[i] : 0;
    n = n < 0 ? 0 : (n > a.ld_cells ? a.ld_cells : n);
    int64_t n_present = qvalid ? a.g.n_cells[s] : 0;
    n_present = n_present < a.g.cap_cells ? n_present : a.g.cap_cells;
    const int32_t *cells = a.sel_cells + (int64_t)i * a.ld_cells;
    const int64_t row0 = (int64_t)(qvalid ? s : 0) * a.g.cap_cells;

    // A operand of S: row col = head g*hpk + col (zero past hpk), dims
    // 32*kb + 8*quad .. +7, scaled
    half8_t qa[8];
    {
        const bool live = col < hpk;
        const float *qp = a.q + ((int64_t)i * a.n_head + g * hpk + (live ? col : 0)) * kHeadDim;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                x[e] = live ? qp[32 * kb + 8 * quad + e] * a.scale : 0.0f;
            qa[kb] = to_half8(x);
        }
    }

    f32x4 o[16];  // O[row 4*quad + jj][dim 16*tt + col]
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) o[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[4], l_run[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        m_run[jj] = -INFINITY;
        l_run[jj] = 0.f;
    }

    // the query's cell list, once, for every wavefront
    for (int x = tid; x < n && x < kCellCap; x += 256) s_cells[x] = cells[x];
    __syncthreads();
    auto cell_at = [&](int cc) { return cc < kCellCap ? s_cells[cc] : cells[cc]; };
    // cells of this lane for a chunk: the two S-tile columns (16t + col) and
    // the two V-staging cells (2*col, 2*col + 1)
    auto chunk_cells = [&](int c0, int (&kc)[2], int (&vc)[2]) {
        const int c1 = min(n, c0 + kPChunk);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int cc = c0 + 16 * t + col;
            kc[t] = cc < c1 ? cell_at(cc) : -1;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int cc = c0 + 2 * col + u;
            vc[u] = cc < c1 ? cell_at(cc) : -1;
        }
    };
    // raw K and V rows of a chunk (memory safety needs only 0 <= cell < cap)
    auto issue_rows = [&](const int (&kc)[2], const int (&vc)[2], RawRow<KVT> (&rk)[2][8],
                          RawRow<KVT> (&rv)[2][8]) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const bool ok = kc[t] >= 0 && kc[t] < a.g.cap_cells;
            const int64_t row = ((row0 + (ok ? kc[t] : 0)) * a.n_head_kv + g);
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
                if (ok) rk[t][kb] = load_raw<KVT>(a.k, row, kb * 4 + quad);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bool ok = vc[u] >= 0 && vc[u] < a.g.cap_cells;
            const int64_t row = ((row0 + (ok ? vc[u] : 0)) * a.n_head_kv + g);
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (ok) rv[u][q] = load_raw<KVT>(a.v, row, quad * 8 + q);
        }
    };
    auto process = [&](const int (&kc)[2], const int (&vc)[2], const RawRow<KVT> (&rk)[2][8],
                       const RawRow<KVT> (&rv)[2][8]) {
        // S tiles: column col of tile t is cell kc[t]
        f32x4 sacc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const bool ok = kc[t] >= 0 && kc[t] < n_present;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                float x[8];
                if (ok) {
                    dequant<KVT>(rk[t][kb], kb * 4 + quad, x);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = 0.f;
                }
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kb], to_half8(x), acc, 0, 0, 0);
            }
            if (!ok) acc = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            sacc[t] = acc;
        }
        // online softmax over the chunk, per head row 4*quad + jj
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float mx = row16_max(fmaxf(sacc[0][jj], sacc[1][jj]));
            const float m_new = fmaxf(m_run[jj], mx);
            const float p0 = m_new == -INFINITY ? 0.f : __expf(sacc[0][jj] - m_new);
            const float p1 = m_new == -INFINITY ? 0.f : __expf(sacc[1][jj] - m_new);
            const float corr = m_run[jj] == -INFINITY ? 0.f : __expf(m_run[jj] - m_new);
            l_run[jj] = l_run[jj] * corr + row16_sum(p0 + p1);
            m_run[jj] = m_new;
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) o[tt][jj] *= corr;
            ws.p[4 * quad + jj][col] = (_Float16)p0;
            ws.p[4 * quad + jj][16 + col] = (_Float16)p1;
        }
        // V to LDS, transposed: vt[dim][cell]
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            float x0[8], x1[8];
            const bool ok0 = vc[0] >= 0 && vc[0] < n_present;
            const bool ok1 = vc[1] >= 0 && vc[1] < n_present;
            if (ok0) dequant<KVT>(rv[0][q], quad * 8 + q, x0);
            if (ok1) dequant<KVT>(rv[1][q], quad * 8 + q, x1);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int dim = 64 * quad + 8 * q + e;
                ws.vt[dim][2 * col] = ok0 ? (_Float16)x0[e] : (_Float16)0.0f;
                ws.vt[dim][2 * col + 1] = ok1 ? (_Float16)x1[e] : (_Float16)0.0f;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // O += P V: A = P[row col][cells 8*quad ..], B = V[cells 8*quad ..][dim]
        const half8_t pa = *reinterpret_cast<const half8_t *>(&ws.p[col][8 * quad]);
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) {
            const half8_t vb = *reinterpret_cast<const half8_t *>(&ws.vt[16 * tt + col][8 * quad]);
            o[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vb, o[tt], 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    constexpr int kStride = kPWaves * kPChunk;
    if constexpr (KVT == QSA_KV_Q8_0) {
        // two row buffers: the next chunk's rows are in flight while this
        // one is computed
        RawRow<KVT> rkA[2][8], rvA[2][8], rkB[2][8], rvB[2][8];
        int kcA[2], vcA[2], kcB[2], vcB[2];
        int c0 = wave * kPChunk;
        if (c0 < n) {
            chunk_cells(c0, kcA, vcA);
            issue_rows(kcA, vcA, rkA, rvA);
        }
        while (c0 < n) {
            const int c1 = c0 + kStride;
            if (c1 < n) {
                chunk_cells(c1, kcB, vcB);
                issue_rows(kcB, vcB, rkB, rvB);
            }
            process(kcA, vcA, rkA, rvA);
            if (c1 >= n) break;
            const int c2 = c1 + kStride;
            if (c2 < n) {
                chunk_cells(c2, kcA, vcA);
                issue_rows(kcA, vcA, rkA, rvA);
            }
            process(kcB, vcB, rkB, rvB);
            c0 = c2;
        }
    } else {
        // f32 rows are twice the registers: one buffer
        for (int c0 = wave * kPChunk; c0 < n; c0 += kStride) {
            RawRow<KVT> rk[2][8], rv[2][8];
            int kc[2], vc[2];
            chunk_cells(c0, kc, vc);
            issue_rows(kc, vc, rk, rv);
            process(kc, vc, rk, rv);
        }
    }

    // merge the four wavefronts' states, a quarter of the dims at a time
    if (col == 0) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            ws.m[4 * quad + jj] = m_run[jj];
            ws.l[4 * quad + jj] = l_run[jj];
        }
    }
#pragma unroll
    for (int part = 0; part < 4; ++part) {
        __syncthreads();
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            const int tt = part * 4 + t4;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) ws.o[4 * quad + jj][16 * t4 + col] = o[tt][jj];
        }
        __syncthreads();
        // thread: head row r = tid / 16 (16 rows), dims 4*(tid%16) .. +3 of the quarter
        const int r = tid >> 4, d0 = (tid & 15) * 4;
        if (r < hpk) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kPWaves; ++w) M = fmaxf(M, sw[w].m[r]);
            float L = 0.f, wt[kPWaves];
#pragma unroll
            for (int w = 0; w < kPWaves; ++w) {
                wt[w] = sw[w].m[r] == -INFINITY ? 0.f : __expf(sw[w].m[r] - M);
                L += sw[w].l[r] * wt[w];
            }
            float *outp = a.out + ((int64_t)i * a.n_head + g * hpk + r) * kHeadDim + part * 64 + d0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float acc = 0.f;
#pragma unroll
                for (int w = 0; w < kPWaves; ++w) acc += sw[w].o[r][d0 + e] * wt[w];
                outp[e] = L > 0.f ? acc / L : 0.f;
            }
        }
    }
}

}  // namespace

size_t attn_prefill_ws_bytes(int, int, int) { return 0; }

hipError_t launch_attn_prefill(const AttnArgs &a, hipStream_t st) {
    if (a.n_q <= 0) return hipSuccess;
    const dim3 grid(a.n_head_kv, a.n_q);
    if (a.kv_type == QSA_KV_F32)
        hipLaunchKernelGGL(k_attn_prefill<QSA_KV_F32>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(k_attn_prefill<QSA_KV_Q8_0>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace qsa
