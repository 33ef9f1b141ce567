// Fixed-m bound and per-head gate (gfx950).
//
// "Fixed-m softmax for 2D-ring x Ulysses attention (WAN 2.2)": the running
// max of online softmax is replaced by a per-query Cauchy-Schwarz bound known
// before streaming, m_i = scale * ||q_i|| * max_j ||k_j||, with the key max
// taken over every K shard (Notes: global over all shards, so a head's m is
// the same on every hop; Tests: a caller's per-shard max||k|| is promoted to
// the global bound).  A head passes the gate iff max_i m_i <= tau (Notes:
// the two-sided halved bound 106.5) and the bound is one that the fixed-m
// body can prove safe in its own arithmetic (description: heads whose bound
// cannot be proven safe keep online softmax).  That body takes exponents
// against m_i less 32 ln 2, so with |s| <= m_i a row's exponents lie in
// [32 - 2 m_i log2 e, 32] (base 2).  Keeping the row's largest term at or
// above 2^-84 (its keys flushed below the fp32/bf16 normal range 2^-126 then
// weigh at most 2^30 * 2^-126 / 2^-84 = 2^-12 of it, for any row of up to
// 2^30 keys) needs 2 m_i log2 e <= 116, i.e. m_i <= 58 ln 2 = 40.2.
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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kFixedSafeMax = 40.2025375f;  // 58 ln 2: the largest bound the fixed-m body proves safe
constexpr int kRowsPerTask = 1024;  // rows of the flattened [B, L, H] order per workgroup
constexpr int kMaxHeadsLds = 256;   // per-head maxima kept in LDS up to this many heads

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

// Rows are taken in memory order (token-major: all heads of a token are
// adjacent), so each workgroup streams one contiguous stretch of the tensor.
// Per-head maxima collect in LDS with integer max on the IEEE bits of the
// non-negative norms, then one global atomic max per head and workgroup (a
// workgroup whose rows straddle two batch elements goes straight to global).
template <int D, int DT>
__global__ __launch_bounds__(256) void norms_kernel(const NormTasks nt) {
    constexpr int EPL = DT == BWA_BF16 ? 8 : 4;  // elements per 16-byte load
    constexpr int TPR = D / EPL;                 // threads per row
    constexpr int RPP = 256 / TPR;               // rows per pass
    constexpr int UNROLL = 8;                    // passes in flight per thread
    __shared__ unsigned hmax[kMaxHeadsLds];
    const BoundLaunch& a = nt.a;
    const i64 task = blockIdx.x;
    int t = 0;
    while (t <= a.n_chunks && task >= nt.task_off[t + 1]) ++t;
    const BoundTensor& T = (t == 0) ? a.q : a.k[t - 1];
    const int TH = (t == 0) ? a.H : a.Hk;  // heads of this tensor
    const int g = a.H / a.Hk;              // query heads per key head
    const i64 rows = (i64)a.B * T.L * TH;
    const i64 r_begin = (task - nt.task_off[t]) * kRowsPerTask;
    const int n_rows = (int)min<i64>(kRowsPerTask, rows - r_begin);
    // Start of the stretch in (b, l, h); rows inside it are offsets of at most
    // kRowsPerTask from here, so 32-bit division finds each row's indices.
    const unsigned H = (unsigned)TH, L = (unsigned)T.L;
    const i64 tok0 = r_begin / H;
    const unsigned h0 = (unsigned)(r_begin - tok0 * H);
    const i64 b0 = tok0 / L;
    const unsigned l0 = (unsigned)(tok0 - b0 * L);
    const bool one_batch = (i64)l0 + (h0 + (unsigned)n_rows - 1) / H < (i64)L;
    const bool in_lds = TH <= kMaxHeadsLds && one_batch;
    const int tid = threadIdx.x, sub = tid % TPR;
    for (int i = tid; i < kMaxHeadsLds; i += 256) hmax[i] = 0u;
    __syncthreads();
    const int es = DT == BWA_BF16 ? 2 : 4;
    for (int j0 = 0; j0 < n_rows; j0 += RPP * UNROLL) {
        u32x4 w[UNROLL];
        unsigned hh[UNROLL], ll[UNROLL], bb[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int j = j0 + u * RPP + tid / TPR;
            const unsigned x = h0 + (unsigned)j, y = l0 + x / H;
            hh[u] = x % H;
            ll[u] = y % L;
            bb[u] = y / L;
            w[u] = u32x4{0, 0, 0, 0};
            if (j < n_rows) {
                const i64 b = b0 + bb[u];
                const uint8_t* rowp = (const uint8_t*)T.ptr + (b * T.sB + (i64)ll[u] * T.sL + (i64)hh[u] * T.sH) * es;
                w[u] = __builtin_nontemporal_load((const u32x4*)(rowp + sub * 16));
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            float ss = 0.0f;
            if (DT == BWA_BF16) {
                const uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x0 = __uint_as_float(ws[i] << 16);
                    const float x1 = __uint_as_float(ws[i] & 0xffff0000u);
                    ss = __builtin_fmaf(x0, x0, ss);
                    ss = __builtin_fmaf(x1, x1, ss);
                }
            } else {
                const float xs[4] = {__uint_as_float(w[u].x), __uint_as_float(w[u].y),
                                     __uint_as_float(w[u].z), __uint_as_float(w[u].w)};
#pragma unroll
                for (int i = 0; i < 4; ++i) ss = __builtin_fmaf(xs[i], xs[i], ss);
            }
#pragma unroll
            for (int o = TPR / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
            const int j = j0 + u * RPP + tid / TPR;
            if (j < n_rows && sub == 0) {
                const i64 b = b0 + bb[u], h = hh[u], l = ll[u];
                const float nrm = __builtin_sqrtf(ss);
                if (t == 0) a.m_out[(b * a.H + h) * T.L + l] = nrm;
                if (l < T.valid) {
                    if (in_lds) {
                        atomicMax(&hmax[h], __float_as_uint(nrm));
                    } else if (t == 0) {
                        atomicMax((unsigned int*)&a.mmax_out[b * a.H + h], __float_as_uint(nrm));
                    } else {  // every query head of key head h
                        for (int r = 0; r < g; ++r)
                            atomicMax((unsigned int*)&a.kmax_out[b * a.H + h * g + r], __float_as_uint(nrm));
                    }
                }
            }
        }
    }
    __syncthreads();
    if (in_lds) {
        for (int h = tid; h < TH; h += 256) {
            const unsigned v = hmax[h];
            if (v == 0u) continue;
            if (t == 0) {
                atomicMax((unsigned int*)&a.mmax_out[b0 * a.H + h], v);
            } else {  // every query head of key head h
                for (int r = 0; r < g; ++r) atomicMax((unsigned int*)&a.kmax_out[b0 * a.H + h * g + r], v);
            }
        }
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
        a.gate_out[bh] = (mm <= a.tau && mm <= kFixedSafeMax) ? 1 : 0;
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
    const i64 BHk = (i64)a.B * a.Hk;
    hipLaunchKernelGGL(init_kernel, dim3((BH + 255) / 256), dim3(256), 0, stream, a);
    NormTasks nt;
    nt.a = a;
    nt.task_off[0] = 0;
    nt.task_off[1] = ((i64)BH * a.q.L + kRowsPerTask - 1) / kRowsPerTask;
    for (int c = 0; c < a.n_chunks; ++c)
        nt.task_off[c + 2] = nt.task_off[c + 1] + (BHk * a.k[c].L + kRowsPerTask - 1) / kRowsPerTask;
    for (int c = a.n_chunks + 2; c < kMaxChunks + 2; ++c) nt.task_off[c] = nt.task_off[a.n_chunks + 1];
    const i64 tasks = nt.task_off[a.n_chunks + 1];
    if (tasks >= ((i64)1 << 24)) return hipErrorInvalidConfiguration;  // 256 work-items each, < 2^32 in all
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
