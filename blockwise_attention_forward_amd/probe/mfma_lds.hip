// Matrix-core throughput with one operand read from LDS for every product,
// as in the attention kernel: each 32x32x16 bf16 product takes a fresh 1 KB
// fragment (one 16-byte read per lane) from LDS, the other operand from
// registers.  Eight wavefronts per workgroup and one workgroup per compute
// unit (the LDS array is sized so that only one fits), two accumulation
// chains per wavefront.  This is the ceiling of the attention kernel's inner
// loop without its softmax, copies and barriers.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bwa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

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

// The same with a chosen mix of LDS operand reads per pair of products: NB
// 16-byte reads per lane (1 KB each) and NT pairs of transposing 8-byte reads
// (ds_read_b64_tr_b16, 512 B each, so 1 KB per pair), all combined into the
// A operand of both products of the pair.  The attention forward reads (1, 1)
// per pair, the dK/dV kernel (2, 1).
template <int NB, int NT>
__global__ __launch_bounds__(512, 1) void mfma_lds_mix_probe(int iters, float* sink) {
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
        for (int u = 0; u < 4; ++u) {
            uint4 a = uint4{0, 0, 0, 0};
#pragma unroll
            for (int r = 0; r < NB + NT; ++r) {
                // 1 KB run r of this pair, cycling through kWindow
                const int base = (((it * 4 + u) * (NB + NT) + r + wave * 5) & (kWindow / 1024 - 1)) * 1024;
                if (r < NB) {
                    const uint4 x = *(const uint4*)(lds + base + lane * 16);
                    a.x ^= x.x; a.y ^= x.y; a.z ^= x.z; a.w ^= x.w;
                } else {
                    const uint2 x0 = __builtin_bit_cast(
                        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(lds + base + lane * 8)));
                    const uint2 x1 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                                   (lds_s16x4*)(uintptr_t)(lds + base + 512 + lane * 8)));
                    a.x ^= x0.x; a.y ^= x0.y; a.z ^= x1.x; a.w ^= x1.y;
                }
            }
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), b, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), b, acc1, 0, 0, 0);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc0[i] + acc1[i];
    sink[(size_t)blockIdx.x * 512 + tid] = s;
}

}  // namespace

extern "C" int32_t bwa_probe_mfma_lds_mix(int32_t n_b128, int32_t n_tr, int32_t iters, int32_t blocks, float* sink,
                                          void* stream) {
    if (iters < 1 || blocks < 1 || !sink) return 1;
    const dim3 g((unsigned)blocks), t(512);
    hipStream_t s = (hipStream_t)stream;
    if (n_b128 == 2 && n_tr == 0) hipLaunchKernelGGL((mfma_lds_mix_probe<2, 0>), g, t, 0, s, iters, sink);
    else if (n_b128 == 0 && n_tr == 2) hipLaunchKernelGGL((mfma_lds_mix_probe<0, 2>), g, t, 0, s, iters, sink);
    else if (n_b128 == 1 && n_tr == 1) hipLaunchKernelGGL((mfma_lds_mix_probe<1, 1>), g, t, 0, s, iters, sink);
    else if (n_b128 == 2 && n_tr == 1) hipLaunchKernelGGL((mfma_lds_mix_probe<2, 1>), g, t, 0, s, iters, sink);
    else if (n_b128 == 4 && n_tr == 0) hipLaunchKernelGGL((mfma_lds_mix_probe<4, 0>), g, t, 0, s, iters, sink);
    else if (n_b128 == 3 && n_tr == 1) hipLaunchKernelGGL((mfma_lds_mix_probe<3, 1>), g, t, 0, s, iters, sink);
    else if (n_b128 == 6 && n_tr == 0) hipLaunchKernelGGL((mfma_lds_mix_probe<6, 0>), g, t, 0, s, iters, sink);
    else return 1;
    return hipGetLastError() == hipSuccess ? 0 : 8;
}

extern "C" int32_t bwa_probe_mfma_lds_bf16(int32_t iters, int32_t blocks, float* sink, void* stream) {
    if (iters < 1 || blocks < 1 || !sink) return 1;
    hipLaunchKernelGGL(mfma_lds_probe, dim3((unsigned)blocks), dim3(512), 0, (hipStream_t)stream, iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : 8;
}
