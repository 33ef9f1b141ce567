// Matrix-core throughput probe for gfx950: independent 32x32x16 bf16
// accumulation chains on register operands, so that the loop is bound by
// the matrix cores alone.  Four chains per wavefront keep each matrix core
// fed while a chain's previous result is still in flight.

#include <hip/hip_runtime.h>

#include "bwa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;

__global__ __launch_bounds__(256) void mfma_probe(int iters, float* sink, uint64_t* clocks) {
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(1e-3f * (float)(threadIdx.x + i));
        b[i] = (__bf16)(2e-3f * (float)i);
    }
    const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[c][i];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (clocks && blockIdx.x == 0 && threadIdx.x == 0) {
        clocks[0] = t1 - t0;
        clocks[1] = r1 - r0;
    }
}

}  // namespace

extern "C" int32_t bwa_probe_mfma_bf16(int32_t iters, int32_t blocks, float* sink, uint64_t* clocks, void* stream) {
    if (iters < 1 || blocks < 1 || !sink) return 1;
    hipLaunchKernelGGL(mfma_probe, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, iters, sink, clocks);
    return hipGetLastError() == hipSuccess ? 0 : 8;
}
