// Log-sum-exp merge of attention partials over disjoint key chunks (gfx950).
//
// "Fixed-m softmax for 2D-ring x Ulysses attention (WAN 2.2)", Notes: when a
// head cannot keep a pinned m on every hop, its hop partials combine in LSE
// space, which does not care how far each partial's reference point was
// from its true max.  For each row: lse = ln sum_t exp(lse_t) and
// O = sum_t exp(lse_t - lse) O_t; a row no chunk saw stays O = 0, lse = -inf.
//
// Pure streaming (no reuse), bound by HBM bandwidth.  A workgroup takes 64
// consecutive tokens of one (b, h): their LSEs are contiguous, so the weight
// pass reads and writes whole lines and leaves the weights in LDS; then D/4
// lanes cover one output row with 16-byte loads, eight rows per thread in
// flight, every partial read once with non-temporal loads.

#include "internal.h"

namespace bwa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kTok = 64;  // tokens of one (b, h) per workgroup

template <int D, int OUT>
__global__ __launch_bounds__(256) void merge_kernel(const MergeLaunch a, const i64 n_lblk) {
    constexpr int TPR = D / 4;       // lanes per row (16-byte loads)
    constexpr int RPP = 256 / TPR;   // rows per pass of the workgroup
    constexpr int R = kTok / RPP;    // rows per thread
    __shared__ float wts[kMaxParts][kTok];
    const i64 bh = blockIdx.x / n_lblk;
    const i64 l0 = (blockIdx.x % n_lblk) * kTok;
    const i64 b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x;
    const int n = a.n_parts;

    // Per-row weights w_t = exp(lse_t - lse), computed once per row; the LSE
    // of a (b, h) is contiguous over tokens, so these loads coalesce.
    if (tid < kTok) {
        const i64 l = l0 + tid;
        if (l < a.L) {
            const i64 li = bh * a.L + l;
            float lt[kMaxParts];
            float mx = -__builtin_inff();
#pragma unroll
            for (int t = 0; t < kMaxParts; ++t)
                if (t < n) { lt[t] = a.lse[t][li]; mx = fmaxf(mx, lt[t]); }
            float tot = 0.0f;
#pragma unroll
            for (int t = 0; t < kMaxParts; ++t)
                if (t < n) { lt[t] = mx == -__builtin_inff() ? 0.0f : __expf(lt[t] - mx); tot += lt[t]; }
            const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
#pragma unroll
            for (int t = 0; t < kMaxParts; ++t)
                if (t < n) wts[t][tid] = lt[t] * inv;
            if (a.lse_out) a.lse_out[li] = tot > 0.0f ? mx + __logf(tot) : -__builtin_inff();
        }
    }
    __syncthreads();

    const int c = (tid % TPR) * 4, rr = tid / TPR;
    f32x4 acc[R];
#pragma unroll
    for (int u = 0; u < R; ++u) acc[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 2
    for (int t = 0; t < n; ++t) {
        const float* base = a.o[t] + b * a.sB[t] + h * a.sH[t] + c;
        const i64 sL = a.sL[t];
        f32x4 o[R];
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const i64 l = l0 + rr + u * RPP;
            o[u] = l < a.L ? __builtin_nontemporal_load((const f32x4*)(base + l * sL)) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const float w = wts[t][rr + u * RPP];
            // A part with weight 0 (its LSE is -inf) adds nothing, whatever its O holds.
            acc[u] += w * (w != 0.0f ? o[u] : f32x4{0.0f, 0.0f, 0.0f, 0.0f});
        }
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const i64 l = l0 + rr + u * RPP;
        if (l >= a.L) continue;
        const i64 ob = b * a.out_sB + l * a.out_sL + h * a.out_sH + c;
        if (OUT == BWA_F32) __builtin_nontemporal_store(acc[u], (f32x4*)((float*)a.out + ob));
        else __builtin_nontemporal_store(__builtin_convertvector(acc[u], bf16x4), (bf16x4*)((__bf16*)a.out + ob));
    }
}

template <int D>
hipError_t launch_d(const MergeLaunch& a, hipStream_t stream) {
    if ((i64)a.B * a.H * a.L == 0) return hipSuccess;
    const i64 n_lblk = (a.L + kTok - 1) / kTok;
    const dim3 grid((unsigned)(n_lblk * a.B * a.H));
    if (a.out_dtype == BWA_F32) hipLaunchKernelGGL((merge_kernel<D, BWA_F32>), grid, dim3(256), 0, stream, a, n_lblk);
    else hipLaunchKernelGGL((merge_kernel<D, BWA_BF16>), grid, dim3(256), 0, stream, a, n_lblk);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(const MergeLaunch& a, hipStream_t stream) {
    return a.D == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace bwa
