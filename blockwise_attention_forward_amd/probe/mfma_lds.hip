// Matrix-core throughput with one operand read from LDS for every product,
// as in the attention kernel: each 32x32x16 bf16 product takes a fresh 1 KB
// fragment (one 16-byte read per lane) from LDS, the other operand from
// registers.  Eight wavefronts per workgroup and one workgroup per compute
// unit (the LDS array is sized so that only one fits), two accumulation
// chains per wavefront.  This is the ceiling of the attention kernel's inner
// loop without its softmax, copies and barriers.

#include <hip/hip_runtime.h>

#include "bwa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLdsBytes = 96 * 1024;  // more than half of the 160 KB: one workgroup per compute unit
constexpr int kWindow = 64 * 1024;    // fragments cycle through this much of it

__global__ __launch_bounds__(512, 1) void mfma_lds_probe(int iters, float* sink) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kLdsBytes];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid * 16; i < kLdsBytes; i += 512 * 16) *(uint4*)(lds + i) = uint4{0x3f803f80u, 0x3f803f80u, 0u, 0u};
    __syncthreads();
    f32x16 acc0 = f32x16{}, acc1 = f32x16{};
    bf16x8 b;
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = (__bf16)(1e-3f * (float)(lane + i));
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int base = ((it * 8 + u + wave * 5) & (kWindow / 1024 - 1)) * 1024;  // < kWindow
            const uint4 a = *(const uint4*)(lds + base + lane * 16);
            if (u & 1) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), b, acc1, 0, 0, 0);
            else acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), b, acc0, 0, 0, 0);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc0[i] + acc1[i];
    sink[(size_t)blockIdx.x * 512 + tid] = s;
}

}  // namespace

extern "C" int32_t bwa_probe_mfma_lds_bf16(int32_t iters, int32_t blocks, float* sink, void* stream) {
    if (iters < 1 || blocks < 1 || !sink) return 1;
    hipLaunchKernelGGL(mfma_lds_probe, dim3((unsigned)blocks), dim3(512), 0, (hipStream_t)stream, iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : 8;
}
