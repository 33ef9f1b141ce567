// Fixed-m bound and per-head gate (gfx950).
//
// "Fixed-m softmax for 2D-ring x Ulysses attention (WAN 2.2)": the running
// max of online softmax is replaced by a per-query Cauchy-Schwarz bound known
// before streaming, m_i = scale * ||q_i|| * max_j ||k_j||, with the key max
// taken over every K shard (Notes: global over all shards, so a head's m is
// the same on every hop; Tests: a caller's per-shard max||k|| is promoted to
// the global bound).  A head passes the gate iff max_i m_i <= tau (Notes:
// the two-sided halved bound 106.5).
//
// The work is one streaming pass over Q and every K chunk (HBM-bound, no
// reuse): each row's 2-norm is an fp32 sum of squares (bf16 products are
// exact in fp32) reduced across the lanes that hold the row.  Per-head
// maxima of non-negative norms are combined with integer atomic max on their
// IEEE bits, which orders non-negative floats exactly (order-independent,
// so the result is deterministic).  Three launches: init, norms, finalize.

#include <algorithm>

#include "internal.h"

namespace bwa {
namespace {

constexpr int kRowsPerTask = 256;

struct NormTasks {
    BoundLaunch a;
    i64 task_off[kMaxChunks + 2];  // prefix of task counts: [0]=Q, [1..n]=chunks
};

__global__ __launch_bounds__(256) void init_kernel(const BoundLaunch a) {
    const int bh = blockIdx.x * 256 + threadIdx.x;
    if (bh >= a.B * a.H) return;
    float km = 0.0f;
    if (a.kmax_in)
        for (int c = 0; c < a.n_kmax_in; ++c) km = fmaxf(km, a.kmax_in[(i64)c * a.B * a.H + bh]);
    a.kmax_out[bh] = km;
    a.mmax_out[bh] = 0.0f;  // holds max ||q_i|| until finalize
}

template <int D, int DT>
__global__ __launch_bounds__(256) void norms_kernel(const NormTasks nt) {
    constexpr int EPL = DT == BWA_BF16 ? 8 : 4;  // elements per 16-byte load
    constexpr int TPR = D / EPL;                 // threads per row
    constexpr int RPP = 256 / TPR;               // rows per pass
    __shared__ float red[4];
    const BoundLaunch& a = nt.a;
    const i64 task = blockIdx.x;
    int t = 0;
    while (t <= a.n_chunks && task >= nt.task_off[t + 1]) ++t;
    const BoundTensor& T = (t == 0) ? a.q : a.k[t - 1];
    const i64 local = task - nt.task_off[t];
    const i64 nrb = (T.L + kRowsPerTask - 1) / kRowsPerTask;
    const i64 bh = local / nrb, rb = local % nrb;
    const i64 b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x, sub = tid % TPR;
    float mx = 0.0f;
    for (int pass = 0; pass < kRowsPerTask / RPP; ++pass) {
        const i64 r = rb * kRowsPerTask + pass * RPP + tid / TPR;
        float ss = 0.0f;
        if (r < T.L) {
            const uint8_t* rowp = (const uint8_t*)T.ptr +
                                  (b * T.sB + r * T.sL + h * T.sH) * (DT == BWA_BF16 ? 2 : 4);
            const uint4 w = *(const uint4*)(rowp + sub * 16);
            if (DT == BWA_BF16) {
                const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x0 = __uint_as_float(ws[i] << 16);
                    const float x1 = __uint_as_float(ws[i] & 0xffff0000u);
                    ss = __builtin_fmaf(x0, x0, ss);
                    ss = __builtin_fmaf(x1, x1, ss);
                }
            } else {
                const float xs[4] = {__uint_as_float(w.x), __uint_as_float(w.y),
                                     __uint_as_float(w.z), __uint_as_float(w.w)};
#pragma unroll
                for (int i = 0; i < 4; ++i) ss = __builtin_fmaf(xs[i], xs[i], ss);
            }
        }
#pragma unroll
        for (int o = TPR / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
        const float nrm = __builtin_sqrtf(ss);
        if (r < T.L && sub == 0) {
            if (t == 0) a.m_out[bh * T.L + r] = nrm;
            if (r < T.valid) mx = fmaxf(mx, nrm);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    if (tid == 0) {
        mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        float* dst = (t == 0) ? &a.mmax_out[bh] : &a.kmax_out[bh];
        atomicMax((unsigned int*)dst, __float_as_uint(mx));
    }
}

__global__ __launch_bounds__(256) void finalize_kernel(const BoundLaunch a) {
    const i64 bh = blockIdx.y;
    const float kmax = a.kmax_out[bh];
    const i64 Lq = a.q.L;
    const i64 i0 = (i64)blockIdx.x * 1024 + threadIdx.x;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const i64 i = i0 + u * 256;
        if (i < Lq) a.m_out[bh * Lq + i] = (a.scale * a.m_out[bh * Lq + i]) * kmax;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        const float mm = (a.scale * a.mmax_out[bh]) * kmax;
        a.mmax_out[bh] = mm;
        a.gate_out[bh] = (mm <= a.tau) ? 1 : 0;
    }
}

template <int D, int DT>
void launch_norms(const NormTasks& nt, i64 tasks, hipStream_t stream) {
    hipLaunchKernelGGL((norms_kernel<D, DT>), dim3((unsigned)tasks), dim3(256), 0, stream, nt);
}

}  // namespace

hipError_t launch_fixed_m_bound(const BoundLaunch& a, hipStream_t stream) {
    const int BH = a.B * a.H;
    if (BH == 0) return hipSuccess;
    hipLaunchKernelGGL(init_kernel, dim3((BH + 255) / 256), dim3(256), 0, stream, a);
    NormTasks nt;
    nt.a = a;
    nt.task_off[0] = 0;
    nt.task_off[1] = (i64)BH * ((a.q.L + kRowsPerTask - 1) / kRowsPerTask);
    for (int c = 0; c < a.n_chunks; ++c)
        nt.task_off[c + 2] = nt.task_off[c + 1] + (i64)BH * ((a.k[c].L + kRowsPerTask - 1) / kRowsPerTask);
    for (int c = a.n_chunks + 2; c < kMaxChunks + 2; ++c) nt.task_off[c] = nt.task_off[a.n_chunks + 1];
    const i64 tasks = nt.task_off[a.n_chunks + 1];
    if (tasks > 0) {
        if (a.D == 64) {
            if (a.dtype == BWA_BF16) launch_norms<64, BWA_BF16>(nt, tasks, stream);
            else launch_norms<64, BWA_F32>(nt, tasks, stream);
        } else {
            if (a.dtype == BWA_BF16) launch_norms<128, BWA_BF16>(nt, tasks, stream);
            else launch_norms<128, BWA_F32>(nt, tasks, stream);
        }
    }
    const unsigned fin_x = (unsigned)std::max<i64>(1, (a.q.L + 1023) / 1024);  // >= 1: the gate is always written
    hipLaunchKernelGGL(finalize_kernel, dim3(fin_x, BH), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace bwa
