// probe.hip -- memory-traffic floors for the benchmark: kernels that only
// move bytes, so that a kernel of the step can be set against what its
// access pattern alone costs on this device.  Not part of the method.
//
// k_probe_read streams a buffer once with 16-byte loads, XOR-folding the
// words into one word per workgroup (the loads cannot be dropped): over a
// buffer far larger than the last-level cache it gives the sustained HBM
// read rate, over one that fits, re-read, the cache's.  The gather of the
// prefill attention kernel has its own probe beside that kernel.
#include "qsa_internal.h"
#include "wave_ops.h"

namespace qsa {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeNT = 256;

template <bool NT>
__device__ __forceinline__ u32x4 probe_load(const u32x4 *p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

// Grid-stride over n16 16-byte words, four loads in flight per lane.
template <bool NT>
__global__ __launch_bounds__(kProbeNT) void k_probe_read(const u32x4 *src, uint64_t n16,
                                                         uint32_t *sink, int n_sink) {
    const uint64_t stride = (uint64_t)gridDim.x * kProbeNT;
    uint64_t i = (uint64_t)blockIdx.x * kProbeNT + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = probe_load<NT>(src + i), b = probe_load<NT>(src + i + stride);
        const u32x4 c = probe_load<NT>(src + i + 2 * stride);
        const u32x4 d = probe_load<NT>(src + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= probe_load<NT>(src + i);
    uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    v ^= xor_lane<1>(v);
    v ^= xor_lane<2>(v);
    v ^= xor_lane<4>(v);
    v ^= xor_lane<8>(v);
    v ^= xor_lane<16>(v);
    v ^= xor_lane<32>(v);
    if ((threadIdx.x & (kWave - 1)) == 0) fold_sink(sink, n_sink, v);
}

}  // namespace

hipError_t launch_probe_read(const void *src, size_t n_bytes, bool nontemporal, uint32_t *sink,
                             int n_sink, hipStream_t st) {
    const uint64_t n16 = n_bytes / 16;
    // 8 workgroups per CU, fewer when the buffer is small
    const uint64_t want = (n16 + kProbeNT * 4 - 1) / (kProbeNT * 4);
    const int grid = (int)(want < 2048 ? (want > 0 ? want : 1) : 2048);
    const u32x4 *p = static_cast<const u32x4 *>(src);
    if (nontemporal)
        hipLaunchKernelGGL(k_probe_read<true>, dim3(grid), dim3(kProbeNT), 0, st, p, n16, sink,
                           n_sink);
    else
        hipLaunchKernelGGL(k_probe_read<false>, dim3(grid), dim3(kProbeNT), 0, st, p, n16, sink,
                           n_sink);
    return hipGetLastError();
}

}  // namespace qsa
