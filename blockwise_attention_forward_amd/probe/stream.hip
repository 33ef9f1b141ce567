// HBM streaming probe for gfx950: the bandwidth the device sustains for a
// given mix of reads and writes, with no arithmetic to speak of.  `ratio`
// source streams of n 16-byte chunks each are read once (non-temporal
// loads); chunk j of the destination is written with a function of chunk j
// of every source stream (ratio reads per write: the merge of two fp32
// partials into one bf16 output reads four bytes per byte written).  With no
// destination the sources are only read and each work-item writes one float.

#include <hip/hip_runtime.h>

#include "bwa_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kUnroll = 8;  // chunks in flight per stream and work-item

__global__ __launch_bounds__(256) void stream_probe(const u32x4* src, int64_t n, int ratio, u32x4* dst,
                                                    float* sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t j0 = (int64_t)blockIdx.x * 256 + threadIdx.x; j0 < n; j0 += stride * kUnroll) {
        u32x4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) x[u] = u32x4{0u, 0u, 0u, 0u};
        for (int r = 0; r < ratio; ++r) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t j = j0 + u * stride;
                if (j < n) x[u] ^= __builtin_nontemporal_load(src + r * n + j);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = j0 + u * stride;
            if (dst && j < n) dst[j] = x[u];
            acc ^= x[u];
        }
    }
    if (!dst) sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = (float)(acc.x ^ acc.y ^ acc.z ^ acc.w);
}

}  // namespace

extern "C" int32_t bwa_probe_stream(const void* src, int64_t chunks, int32_t ratio, void* dst, int32_t blocks,
                                    float* sink, void* stream) {
    if (!src || chunks < 1 || ratio < 1 || blocks < 1 || (!dst && !sink)) return 1;
    if (((uintptr_t)src | (uintptr_t)dst) % 16) return 1;
    hipLaunchKernelGGL(stream_probe, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src,
                       chunks, ratio, (u32x4*)dst, sink);
    return hipGetLastError() == hipSuccess ? 0 : 8;
}
