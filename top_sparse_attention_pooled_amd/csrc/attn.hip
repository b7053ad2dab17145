// attn.hip -- attention over the selected cells only (llama.cpp issue #28734,
// fix summary, "lever1": the top-k set, not the whole cache, is what attention
// visits), with q8_0 rows dequantised inside the gather (discussion #30071:
// the compact-gather path that keeps a quantised cache on the sparse path,
// where converting the whole cache first would cost O(n_kv)).
//
// Work unit: one workgroup = one (query, KV head, run of cells).  Its 256
// threads are 8 groups of 32; lane j of a group owns dims 8j .. 8j+7 of the
// head and all G query heads that share the KV head, so each K/V row is read
// once from memory and feeds G heads.  Per 64-cell chunk: the groups score
// their cells (G dot products reduced over 32 lanes with a transposing
// butterfly: 9 shuffles for 8 heads), the chunk's softmax statistics come
// from one wavefront per head, and the groups accumulate P*V; across chunks
// the running (max, sum, output) are rescaled once per chunk.  Decode splits a
// query's cells over many workgroups and merges their partial states in a
// second kernel; prefill gives each workgroup all cells of its query.
//
// q8_0 rows: 8 blocks of (binary16 scale, 32 int8) = 272 bytes.  A lane's
// 8 int8 start at byte 34*(j/4) + 2 + 8*(j%4), which is 2 mod 4 for even
// blocks: they are read as aligned dwords and realigned with a funnel shift.
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kChunk = 64;   // cells per chunk (= one wavefront for the softmax)
constexpr int kGroups = 8;   // 32-lane groups per workgroup

// 8 dequantised values (dims 8j .. 8j+7) of one row.
template <int KVT>
__device__ __forceinline__ void load_row8(const void *base, int64_t row, int j, float (&x)[8]) {
    if (KVT == QSA_KV_F32) {
        const float4 *p = reinterpret_cast<const float4 *>(
            static_cast<const float *>(base) + row * kHeadDim + 8 * j);
        const float4 u = p[0], v = p[1];
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
        x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
    } else {
        const uint8_t *r = static_cast<const uint8_t *>(base) + row * kQ8Row;
        const int blk = j >> 2;
        const int start = blk * kQ8Bytes + 2 + 8 * (j & 3);
        const uint32_t *w = reinterpret_cast<const uint32_t *>(r + (start & ~3));
        uint32_t lo, hi;
        if (start & 3) {  // 2 mod 4: three dwords, shift by 2 bytes
            const uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
            lo = __builtin_amdgcn_alignbyte(w1, w0, 2);
            hi = __builtin_amdgcn_alignbyte(w2, w1, 2);
        } else {
            lo = w[0];
            hi = w[1];
        }
        const int sofs = blk * kQ8Bytes;  // scale: low or high half of a dword
        const uint32_t sw = *reinterpret_cast<const uint32_t *>(r + (sofs & ~3));
        const uint16_t sbits = (uint16_t)((sofs & 3) ? (sw >> 16) : (sw & 0xffffu));
        const float d = (float)__builtin_bit_cast(_Float16, sbits);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = d * (float)((int32_t)(lo << (24 - 8 * e)) >> 24);
            x[e + 4] = d * (float)((int32_t)(hi << (24 - 8 * e)) >> 24);
        }
    }
}

// Sum v[0..G) over the 32 lanes of a group.  On return lane j holds the full
// sum for head head_of_lane<G>(j) in v[0].
template <int G>
__device__ __forceinline__ void group_reduce(float (&v)[G]) {
    int n = G;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) {
        if (n > 1) {
            const int half = n >> 1;
            const bool upper = (threadIdx.x & o) != 0;
#pragma unroll
            for (int h = 0; h < G / 2; ++h) {
                if (h < half) {
                    const float keep = upper ? v[h + half] : v[h];
                    const float send = upper ? v[h] : v[h + half];
                    v[h] = keep + __shfl_xor(send, o, kWave);
                }
            }
            n = half;
        } else {
            v[0] = v[0] + __shfl_xor(v[0], o, kWave);
        }
    }
}

template <int G>
__device__ __forceinline__ int head_of_lane(int j) {
    // the halving steps fix head bits from the top: lane bit 4 picks the upper
    // half of the heads first, then bit 3, ...
    int h = 0, n = G;
    for (int o = 16; o >= 1 && n > 1; o >>= 1) {
        n >>= 1;
        if (j & o) h += n;
    }
    return h;
}

template <int G>
__device__ __forceinline__ bool lane_reports(int j) {
    // lanes that agree on the head bits hold equal copies; the lowest reports
    int bits = 0, n = G;
    for (int o = 16; o >= 1 && n > 1; o >>= 1) {
        n >>= 1;
        bits |= o;
    }
    return (j & ~bits & 31) == 0;
}

// grid (n_runs, n_head_kv, n_q).  Workgroup x covers chunks
// [x*chunks_per_run, (x+1)*chunks_per_run) of the query's selected list.
// direct != 0: one run covers all cells, write the normalised output;
// otherwise write the partial state (o[G][256], m[G], l[G]) to ws.
template <int G, int KVT>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a, int chunks_per_run, int n_runs,
                                              int direct) {
    __shared__ float s_p[G][kChunk];
    __shared__ float s_red[kGroups][G * kHeadDim];
    __shared__ float s_stat[G][2];  // chunk max, chunk sum

    const int run = blockIdx.x, g = blockIdx.y, i = blockIdx.z;
    const int tid = threadIdx.x, grp = tid >> 5, j = tid & 31, wave = tid >> 6,
              lane = tid & 63;
    const int s = a.q_seq[i];
    const bool qvalid = s >= 0 && s < a.g.n_seq;
    int n = qvalid ? a.n_sel[i] : 0;
    if (n < 0) n = 0;
    if (n > a.ld_cells) n = a.ld_cells;
    int64_t n_present = qvalid ? a.g.n_cells[s] : 0;
    if (n_present > a.g.cap_cells) n_present = a.g.cap_cells;
    const int c_begin = run * chunks_per_run * kChunk;
    const int c_end = min(n, c_begin + chunks_per_run * kChunk);
    const int h0 = g * G;

    float m_run[G], l_run[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
    }

    if (c_begin < c_end) {
        float qv[G][8];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float4 *qp = reinterpret_cast<const float4 *>(
                a.q + ((int64_t)i * a.n_head + h0 + h) * kHeadDim + 8 * j);
            const float4 u = qp[0], v = qp[1];
            qv[h][0] = u.x; qv[h][1] = u.y; qv[h][2] = u.z; qv[h][3] = u.w;
            qv[h][4] = v.x; qv[h][5] = v.y; qv[h][6] = v.z; qv[h][7] = v.w;
        }
        const int32_t *cells = a.sel_cells + (int64_t)i * a.ld_cells;
        const int64_t row0 = (int64_t)s * a.g.cap_cells;

        for (int c0 = c_begin; c0 < c_end; c0 += kChunk) {
            const int c1 = min(c_end, c0 + kChunk);
            // scores of this group's cells
            for (int cc = c0 + grp; c1 > cc; cc += kGroups) {
                const int cell = cells[cc];
                const bool ok = cell >= 0 && cell < n_present;
                float kf[8];
                if (ok) {
                    load_row8<KVT>(a.k, (row0 + cell) * a.n_head_kv + g, j, kf);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) kf[e] = 0.f;
                }
                float sv[G];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float acc = qv[h][0] * kf[0];
#pragma unroll
                    for (int e = 1; e < 8; ++e) acc = fmaf(qv[h][e], kf[e], acc);
                    sv[h] = acc;
                }
                group_reduce<G>(sv);
                if (lane_reports<G>(j))
                    s_p[head_of_lane<G>(j)][cc - c0] = ok ? sv[0] * a.scale : -INFINITY;
            }
            __syncthreads();
            // chunk statistics: one wavefront per head, lane = cell
#pragma unroll
            for (int h = 0; h < G; ++h) {
                if ((h & 3) != wave) continue;
                const bool in = c0 + lane < c1;
                const float x = in ? s_p[h][lane] : -INFINITY;
                float mx = x;
#pragma unroll
                for (int o2 = 32; o2 >= 1; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2, kWave));
                const float m_new = fmaxf(m_run[h], mx);  // m_run identical in all threads
                const float pe = (in && x != -INFINITY) ? __expf(x - m_new) : 0.f;
                float sum = pe;
#pragma unroll
                for (int o2 = 32; o2 >= 1; o2 >>= 1) sum += __shfl_xor(sum, o2, kWave);
                s_p[h][lane] = pe;
                if (lane == 0) {
                    s_stat[h][0] = m_new;
                    s_stat[h][1] = sum;
                }
            }
            __syncthreads();
            // rescale the running state, then accumulate P*V
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float m_new = s_stat[h][0];
                const float corr = m_run[h] == -INFINITY ? 0.f : __expf(m_run[h] - m_new);
                l_run[h] = l_run[h] * corr + s_stat[h][1];
                m_run[h] = m_new;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[h][e] *= corr;
            }
            for (int cc = c0 + grp; c1 > cc; cc += kGroups) {
                const int cell = cells[cc];
                const bool ok = cell >= 0 && cell < n_present;
                if (!ok) continue;
                float vf[8];
                load_row8<KVT>(a.v, (row0 + cell) * a.n_head_kv + g, j, vf);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float pw = s_p[h][cc - c0];
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[h][e] = fmaf(pw, vf[e], o[h][e]);
                }
            }
            __syncthreads();
        }
    }

    // merge the 8 groups (same running max in every group), fixed order
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) s_red[grp][h * kHeadDim + 8 * j + e] = o[h][e];
    __syncthreads();
    float *part = a.ws + (((int64_t)i * a.n_head_kv + g) * n_runs + run) *
                             (G * kHeadDim + 2 * G);
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const int t = h * kHeadDim + tid;  // 256 threads = 256 dims
        float acc = s_red[0][t];
#pragma unroll
        for (int q = 1; q < kGroups; ++q) acc += s_red[q][t];
        if (direct) {
            const float l = l_run[h];
            a.out[((int64_t)i * a.n_head + h0 + h) * kHeadDim + tid] = l > 0.f ? acc / l : 0.f;
        } else {
            part[t] = acc;
            if (tid == 0) {
                part[G * kHeadDim + h] = m_run[h];
                part[G * kHeadDim + G + h] = l_run[h];
            }
        }
    }
}

// grid (n_head, n_q), 256 threads = dims.  Merges the runs' partial states.
template <int G>
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a, int n_runs) {
    const int h = blockIdx.x, i = blockIdx.y, t = threadIdx.x;
    const int g = h / G, hh = h % G;
    const float *base = a.ws + ((int64_t)i * a.n_head_kv + g) * n_runs * (G * kHeadDim + 2 * G);
    float M = -INFINITY;
    for (int r = 0; r < n_runs; ++r) {
        const float *part = base + (int64_t)r * (G * kHeadDim + 2 * G);
        if (part[G * kHeadDim + G + hh] > 0.f) M = fmaxf(M, part[G * kHeadDim + hh]);
    }
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
        for (int r = 0; r < n_runs; ++r) {
            const float *part = base + (int64_t)r * (G * kHeadDim + 2 * G);
            const float l = part[G * kHeadDim + G + hh];
            if (!(l > 0.f)) continue;
            const float w = __expf(part[G * kHeadDim + hh] - M);
            L = fmaf(l, w, L);
            O = fmaf(part[hh * kHeadDim + t], w, O);
        }
    }
    a.out[((int64_t)i * a.n_head + h) * kHeadDim + t] = L > 0.f ? O / L : 0.f;
}

template <int G, int KVT>
hipError_t launch_g(const AttnArgs &a, int chunks_per_run, int n_runs, bool direct,
                    hipStream_t st) {
    dim3 grid(n_runs, a.n_head_kv, a.n_q);
    hipLaunchKernelGGL((k_attn<G, KVT>), grid, dim3(256), 0, st, a, chunks_per_run, n_runs,
                       direct ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || direct) return e;
    hipLaunchKernelGGL((k_attn_combine<G>), dim3(a.n_head, a.n_q), dim3(256), 0, st, a, n_runs);
    return hipGetLastError();
}

template <int KVT>
hipError_t launch_kvt(const AttnArgs &a, int chunks_per_run, int n_runs, bool direct,
                      hipStream_t st) {
    switch (a.n_head / a.n_head_kv) {
        case 1: return launch_g<1, KVT>(a, chunks_per_run, n_runs, direct, st);
        case 2: return launch_g<2, KVT>(a, chunks_per_run, n_runs, direct, st);
        case 4: return launch_g<4, KVT>(a, chunks_per_run, n_runs, direct, st);
        case 8: return launch_g<8, KVT>(a, chunks_per_run, n_runs, direct, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch(const AttnArgs &a, int chunks_per_run, int n_runs, bool direct,
                  hipStream_t st) {
    if (a.n_q <= 0) return hipSuccess;
    return a.kv_type == QSA_KV_F32 ? launch_kvt<QSA_KV_F32>(a, chunks_per_run, n_runs, direct, st)
                                   : launch_kvt<QSA_KV_Q8_0>(a, chunks_per_run, n_runs, direct, st);
}

int decode_runs(int ld_cells) { return (ld_cells + kChunk - 1) / kChunk; }

}  // namespace

size_t attn_decode_ws_bytes(int n_q, int n_head, int ld_cells) {
    // per (query, KV head, run): G*256 + 2G floats; summed over KV heads this
    // is n_head*(256 + 2) floats per run
    return (size_t)n_q * decode_runs(ld_cells) * n_head * (kHeadDim + 2) * sizeof(float);
}

hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t st) {
    return launch(a, 1, decode_runs(a.ld_cells), false, st);
}

size_t attn_prefill_ws_bytes(int, int, int) { return 0; }

hipError_t launch_attn_prefill(const AttnArgs &a, hipStream_t st) {
    const int chunks = decode_runs(a.ld_cells);
    return launch(a, chunks, 1, true, st);
}

}  // namespace qsa
