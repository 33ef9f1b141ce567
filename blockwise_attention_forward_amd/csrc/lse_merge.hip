// Log-sum-exp merge of attention partials over disjoint key chunks (gfx950).
//
// "Fixed-m softmax for 2D-ring x Ulysses attention (WAN 2.2)", Notes: when a
// head cannot keep a pinned m on every hop, its hop partials combine in LSE
// space, which does not care how far each partial's reference point was
// from its true max.  For each row: lse = ln sum_t exp(lse_t) and
// O = sum_t exp(lse_t - lse) O_t; a row no chunk saw stays O = 0, lse = -inf.
//
// Pure streaming (no reuse): D/4 lanes cover one row with 16-byte loads of
// every partial, so a wavefront reads whole contiguous rows and the work is
// bound by HBM bandwidth.  The per-row weights are computed redundantly by
// the row's lanes from a broadcast load of the partial LSEs.

#include "internal.h"

namespace bwa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <int D, int OUT>
__global__ __launch_bounds__(256) void merge_kernel(const MergeLaunch a) {
    constexpr int TPR = D / 4;        // lanes per row
    constexpr int RPB = 256 / TPR;    // rows per workgroup
    const i64 rows = (i64)a.B * a.L * a.H;
    const i64 r = (i64)blockIdx.x * RPB + threadIdx.x / TPR;
    if (r >= rows) return;
    const int c = (threadIdx.x % TPR) * 4;
    const i64 h = r % a.H;
    const i64 l = (r / a.H) % a.L;
    const i64 b = r / ((i64)a.H * a.L);
    const i64 li = (b * a.H + h) * a.L + l;

    float lse_t[kMaxParts];
    float mx = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < kMaxParts; ++t) {
        if (t < a.n_parts) { lse_t[t] = a.lse[t][li]; mx = fmaxf(mx, lse_t[t]); }
    }
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float lse = -__builtin_inff();
    if (mx != -__builtin_inff()) {
        float tot = 0.0f;
#pragma unroll
        for (int t = 0; t < kMaxParts; ++t) {
            if (t < a.n_parts) {
                const float w = __expf(lse_t[t] - mx);
                tot += w;
                const f32x4 o = *(const f32x4*)(a.o[t] + b * a.sB[t] + l * a.sL[t] + h * a.sH[t] + c);
                acc += w * o;
            }
        }
        acc *= 1.0f / tot;
        lse = mx + __logf(tot);
    }
    const i64 ob = b * a.out_sB + l * a.out_sL + h * a.out_sH + c;
    if (OUT == BWA_F32) {
        *(f32x4*)((float*)a.out + ob) = acc;
    } else {
        *(bf16x4*)((__bf16*)a.out + ob) = __builtin_convertvector(acc, bf16x4);
    }
    if (a.lse_out && c == 0) a.lse_out[li] = lse;
}

template <int D>
hipError_t launch_d(const MergeLaunch& a, hipStream_t stream) {
    constexpr int RPB = 256 / (D / 4);
    const i64 rows = (i64)a.B * a.L * a.H;
    if (rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
    if (a.out_dtype == BWA_F32) hipLaunchKernelGGL((merge_kernel<D, BWA_F32>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((merge_kernel<D, BWA_BF16>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(const MergeLaunch& a, hipStream_t stream) {
    return a.D == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace bwa
