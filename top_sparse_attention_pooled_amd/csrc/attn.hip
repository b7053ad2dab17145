// attn.hip -- attention over the selected cells only (llama.cpp issue #28734,
// fix summary, "lever1": the top-k set, not the whole cache, is what attention
// visits), with q8_0 rows dequantised inside the gather (discussion #30071:
// the compact-gather path that keeps a quantised cache on the sparse path,
// where converting the whole cache first would cost O(n_kv)).
//
// Work unit: one workgroup = one (query, KV head, run of cells).  Its 256
// threads are 8 groups of 32; lane j of a group owns dims 8j .. 8j+7 of the
// head and all G query heads that share the KV head, so each K/V row is read
// once from memory and feeds G heads.  A decode workgroup takes one 32-cell
// chunk (130 workgroups for a 2051-cell set over 2 KV heads) and issues every
// index, K and V load before it uses any.  Per chunk: the groups score
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

constexpr int kChunk = 32;   // cells per chunk; a decode workgroup takes one chunk
constexpr int kGroups = 8;   // 32-lane groups per workgroup
constexpr int kCPG = kChunk / kGroups;  // cells per group per chunk

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

template <int KVT>
__device__ __forceinline__ RawRow<KVT> load_raw(const void *base, int64_t row, int j) {
    RawRow<KVT> r;
    if constexpr (KVT == QSA_KV_F32) {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) +
                                                           row * kHeadDim + 8 * j);
        r.u = p[0];
        r.v = p[1];
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

// Sum v[0..G) over the 32 lanes of a group.  On return lane j holds the full
// sum for head head_of_lane<G>(j) in v[0]: each halving step exchanges half
// of the remaining values, so 8 heads cost 4+2+1+1+1 shuffles, not 8*5.
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
    const int h0 = g * G;
    const int c_begin = run * chunks_per_run * kChunk;
    const int32_t *cells = a.sel_cells + (int64_t)i * a.ld_cells;

    // first round trip: nothing here depends on another load
    const int s = a.q_seq[i];
    const int n_raw = a.n_sel[i];
    int cell[kCPG];
#pragma unroll
    for (int u = 0; u < kCPG; ++u) {
        const int cc = c_begin + grp * kCPG + u;
        cell[u] = cc < a.ld_cells ? cells[cc] : -1;
    }
    float qv[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float4 *qp = reinterpret_cast<const float4 *>(
            a.q + ((int64_t)i * a.n_head + h0 + h) * kHeadDim + 8 * j);
        const float4 u = qp[0], v = qp[1];
        qv[h][0] = u.x; qv[h][1] = u.y; qv[h][2] = u.z; qv[h][3] = u.w;
        qv[h][4] = v.x; qv[h][5] = v.y; qv[h][6] = v.z; qv[h][7] = v.w;
    }
    const bool qvalid = s >= 0 && s < a.g.n_seq;
    const int n = qvalid ? (n_raw < 0 ? 0 : (n_raw > a.ld_cells ? a.ld_cells : n_raw)) : 0;
    const int c_end = min(n, c_begin + chunks_per_run * kChunk);

    float m_run[G], l_run[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
    }

    if (c_begin < c_end) {
        const int64_t row0 = (int64_t)s * a.g.cap_cells;
        for (int c0 = c_begin; c0 < c_end; c0 += kChunk) {
            const int c1 = min(c_end, c0 + kChunk);
            if (c0 != c_begin) {
#pragma unroll
                for (int u = 0; u < kCPG; ++u) {
                    const int cc = c0 + grp * kCPG + u;
                    cell[u] = cc < a.ld_cells ? cells[cc] : -1;
                }
            }
            // second round trip: K/V rows (memory safety needs only
            // 0 <= cell < cap_cells) and the present-cell count
            RawRow<KVT> rk[kCPG], rv[kCPG];
#pragma unroll
            for (int u = 0; u < kCPG; ++u) {
                if (cell[u] >= 0 && cell[u] < a.g.cap_cells) {
                    const int64_t row = (row0 + cell[u]) * a.n_head_kv + g;
                    rk[u] = load_raw<KVT>(a.k, row, j);
                    rv[u] = load_raw<KVT>(a.v, row, j);
                }
            }
            int64_t n_present = a.g.n_cells[s];
            n_present = n_present < a.g.cap_cells ? n_present : a.g.cap_cells;
            // scores of this group's cells
#pragma unroll
            for (int u = 0; u < kCPG; ++u) {
                const int cc = c0 + grp * kCPG + u;
                const bool ok = cc < c1 && cell[u] >= 0 && cell[u] < n_present;
                float kf[8];
                if (ok) {
                    dequant<KVT>(rk[u], j, kf);
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
                if (cc < c1 && lane_reports<G>(j))
                    s_p[head_of_lane<G>(j)][cc - c0] = ok ? sv[0] * a.scale : -INFINITY;
            }
            __syncthreads();
            // chunk statistics: 32 lanes per head, two heads per wavefront
#pragma unroll
            for (int h = 0; h < G; ++h) {
                if (((h >> 1) & 3) != wave || ((h & 1) != (lane >> 5))) continue;
                const int c = lane & 31;
                const bool in = c0 + c < c1;
                const float x = in ? s_p[h][c] : -INFINITY;
                float mx = x;
#pragma unroll
                for (int o2 = 16; o2 >= 1; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2, kWave));
                const float m_new = fmaxf(m_run[h], mx);  // m_run equal in every thread
                const float pe = (in && x != -INFINITY) ? __expf(x - m_new) : 0.f;
                float sum = pe;
#pragma unroll
                for (int o2 = 16; o2 >= 1; o2 >>= 1) sum += __shfl_xor(sum, o2, kWave);
                s_p[h][c] = pe;
                if (c == 0) {
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
#pragma unroll
            for (int u = 0; u < kCPG; ++u) {
                const int cc = c0 + grp * kCPG + u;
                const bool ok = cc < c1 && cell[u] >= 0 && cell[u] < n_present;
                if (!ok) continue;
                float vf[8];
                dequant<KVT>(rv[u], j, vf);
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

constexpr int kCombNT = 1024;
constexpr int kCombGroups = kCombNT / 128;  // run groups x 128 dim pairs

// grid (n_head, n_q).  Merges the runs' partial states of one head: thread
// (rg, dp) sums runs rg, rg+8, ... for dims 2dp, 2dp+1; the 8 partial sums
// are then added in a fixed order.
template <int G>
__global__ __launch_bounds__(kCombNT) void k_attn_combine(AttnArgs a, int n_runs) {
    __shared__ float s_w[1024];
    __shared__ float s_red[32];
    __shared__ float2 s_acc[kCombGroups][128];
    const int h = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
    const int g = h / G, hh = h % G;
    const int stride = G * kHeadDim + 2 * G;
    const float *base = a.ws + ((int64_t)i * a.n_head_kv + g) * n_runs * stride;
    // per-run weights exp(m_r - M), M = max over runs that saw any cell
    float m = -INFINITY, l = 0.f;
    if (tid < n_runs) {
        m = base[(int64_t)tid * stride + G * kHeadDim + hh];
        l = base[(int64_t)tid * stride + G * kHeadDim + G + hh];
        if (!(l > 0.f)) m = -INFINITY;
    }
    float mx = m;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
    if ((tid & 63) == 0) s_red[tid >> 6] = mx;
    __syncthreads();
    float M = s_red[0];
#pragma unroll
    for (int w = 1; w < kCombNT / 64; ++w) M = fmaxf(M, s_red[w]);
    __syncthreads();
    const float wgt = (m != -INFINITY) ? __expf(m - M) : 0.f;
    if (tid < n_runs) s_w[tid] = wgt;
    float lw = l > 0.f ? l * wgt : 0.f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lw += __shfl_xor(lw, o, kWave);
    if ((tid & 63) == 0) s_red[tid >> 6] = lw;
    __syncthreads();
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kCombNT / 64; ++w) L += s_red[w];

    const int rg = tid >> 7, dp = tid & 127;
    float2 acc = make_float2(0.f, 0.f);
    constexpr int U = 8;
    for (int r0 = rg; r0 < n_runs; r0 += kCombGroups * U) {
        float2 v[U];
        float w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = r0 + u * kCombGroups;
            w[u] = r < n_runs ? s_w[r] : 0.f;
            v[u] = (r < n_runs && w[u] != 0.f)
                       ? *reinterpret_cast<const float2 *>(base + (int64_t)r * stride +
                                                           hh * kHeadDim + 2 * dp)
                       : make_float2(0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            acc.x = fmaf(v[u].x, w[u], acc.x);
            acc.y = fmaf(v[u].y, w[u], acc.y);
        }
    }
    s_acc[rg][dp] = acc;
    __syncthreads();
    if (rg == 0) {
        float2 t = s_acc[0][dp];
#pragma unroll
        for (int q = 1; q < kCombGroups; ++q) {
            t.x += s_acc[q][dp].x;
            t.y += s_acc[q][dp].y;
        }
        float2 r = make_float2(L > 0.f ? t.x / L : 0.f, L > 0.f ? t.y / L : 0.f);
        *reinterpret_cast<float2 *>(a.out + ((int64_t)i * a.n_head + h) * kHeadDim + 2 * dp) = r;
    }
}

template <int G, int KVT>
hipError_t launch_g(const AttnArgs &a, int chunks_per_run, int n_runs, bool direct,
                    hipStream_t st) {
    dim3 grid(n_runs, a.n_head_kv, a.n_q);
    hipLaunchKernelGGL((k_attn<G, KVT>), grid, dim3(256), 0, st, a, chunks_per_run, n_runs,
                       direct ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || direct) return e;
    hipLaunchKernelGGL((k_attn_combine<G>), dim3(a.n_head, a.n_q), dim3(kCombNT), 0, st, a,
                       n_runs);
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
