// Tile run lists for blockwise attention (gfx950).
//
// "Add more optimal dk order optional arg" (flash-attention pull request
// 2512), "Sliding window perf issue": a block-sparse kernel walks partial
// tiles (element mask needed) and full tiles (no mask) and skips the rest;
// "A simplish fix" merges both kinds into one ordered list.  Here every
// query block gets its visited key blocks in ascending order as maximal runs
// of one kind, stored CSR-style in HBM.  The metadata is O(query blocks x
// runs) plus one key interval per row; nothing per token or per tile pair is
// held on chip, which is what capped the segmented splash kernel ("Let
// splash attention exceed 524,288 tokens when packing is off", Effect).
//
// Four launches: row intervals; run count per query block; exclusive scan
// of the counts into row_ptr; run fill.  Integer-only, deterministic.

#include "internal.h"

namespace bwa {
namespace {

__global__ __launch_bounds__(256) void rows_kernel(const BlocksLaunch a) {
    const i64 idx = (i64)blockIdx.x * 256 + threadIdx.x;
    const i64 lq = a.mask.lq;
    if (idx >= a.copies * lq) return;
    const i64 copy = idx / lq, i = idx % lq;
    int lo, hi;
    row_interval(a.mask, copy, i, lo, hi);
    a.row_lo[idx] = lo;
    a.row_hi[idx] = hi;
}

// One wavefront per (copy, query block); each lane keeps bq/64 rows'
// intervals in registers.  A key block is FULL iff every row of the block
// covers it, i.e. j0 >= max lo and min(j0 + bkv, lk) <= min hi over the
// block's rows (all non-empty), so the FULL blocks form one range computed
// directly.  Only the blocks outside it are tested one by one (a block is
// visited iff some row's interval meets it), with wave ballots.
constexpr int kMaxRowsPerLane = 8;  // bq <= 512

template <bool FILL>
__global__ __launch_bounds__(256) void runs_kernel(const BlocksLaunch a) {
    const i64 wg = (i64)blockIdx.x * 4 + (threadIdx.x >> 6);
    const i64 nqb = a.n_qblocks;
    if (wg >= a.copies * nqb) return;
    const int lane = threadIdx.x & 63;
    const i64 copy = wg / nqb, qb = wg % nqb;
    const i64 lq = a.mask.lq, lk = a.mask.lk;
    const int per_lane = a.bq / 64;
    int rlo[kMaxRowsPerLane], rhi[kMaxRowsPerLane];
    bool rex[kMaxRowsPerLane];
    int mn_lo = 0x7fffffff, mx_hi = 0, mx_lo = 0, mn_hi = 0x7fffffff;
#pragma unroll
    for (int t = 0; t < kMaxRowsPerLane; ++t) {
        const i64 r = qb * a.bq + lane + 64 * t;
        rex[t] = t < per_lane && r < lq;
        rlo[t] = rex[t] ? a.row_lo[copy * lq + r] : 0;
        rhi[t] = rex[t] ? a.row_hi[copy * lq + r] : 0;
        if (rex[t]) {
            const bool ne = rlo[t] < rhi[t];
            if (ne) { mn_lo = min(mn_lo, rlo[t]); mx_hi = max(mx_hi, rhi[t]); }
            mx_lo = max(mx_lo, ne ? rlo[t] : 0x7fffffff);  // an empty row rules out FULL
            mn_hi = min(mn_hi, ne ? rhi[t] : -1);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mn_lo = min(mn_lo, __shfl_xor(mn_lo, o));
        mx_hi = max(mx_hi, __shfl_xor(mx_hi, o));
        mx_lo = max(mx_lo, __shfl_xor(mx_lo, o));
        mn_hi = min(mn_hi, __shfl_xor(mn_hi, o));
    }
    i64* rp = a.row_ptr + copy * (nqb + 1);
    const i64 out = FILL ? rp[qb] : 0;
    i64 n = 0;
    int cur_kind = 0, cur_b = 0, cur_e = 0;
    auto emit = [&]() {
        if (FILL && lane == 0) {
            const i64 slot = out + n;
            if (slot < a.capacity) {
                a.run_begin[copy * a.capacity + slot] = cur_b;
                a.run_end[copy * a.capacity + slot] = cur_e;
                a.run_kind[copy * a.capacity + slot] = (uint8_t)cur_kind;
            }
        }
        ++n;
    };
    auto push = [&](int kb, int kind) {
        if (kind == BWA_TILE_SKIP) {
            if (cur_kind) { emit(); cur_kind = 0; }
        } else if (cur_kind == kind && cur_e == kb) {
            cur_e = kb + 1;
        } else {
            if (cur_kind) emit();
            cur_kind = kind; cur_b = kb; cur_e = kb + 1;
        }
    };
    auto partial_range = [&](int k0, int k1) {  // blocks known not to be FULL
        for (int kb = k0; kb < k1; ++kb) {
            const i64 j0 = (i64)kb * a.bkv, j1 = min(j0 + a.bkv, lk);
            bool meets = false;
#pragma unroll
            for (int t = 0; t < kMaxRowsPerLane; ++t)
                meets |= rex[t] && rlo[t] < rhi[t] && rlo[t] < j1 && rhi[t] > j0;
            push(kb, __ballot(meets) != 0 ? BWA_TILE_PARTIAL : BWA_TILE_SKIP);
        }
    };
    if (mx_hi > 0) {
        const int nkb = (int)((lk + a.bkv - 1) / a.bkv);
        const int kb_lo = mn_lo / a.bkv;
        const int kb_hi = (int)((mx_hi + (i64)a.bkv - 1) / a.bkv);
        int f0 = 0, f1 = 0;
        if (mx_lo != 0x7fffffff && mn_hi >= 0) {
            f0 = (mx_lo + a.bkv - 1) / a.bkv;
            f1 = (mn_hi >= lk) ? nkb : mn_hi / a.bkv;
        }
        if (f0 < f1) {
            partial_range(kb_lo, f0);
            if (cur_kind == BWA_TILE_FULL && cur_e == f0) {  // cannot happen after a PARTIAL block; kept exact
                cur_e = f1;
            } else {
                if (cur_kind) emit();
                cur_kind = BWA_TILE_FULL; cur_b = f0; cur_e = f1;
            }
            partial_range(f1, kb_hi);
        } else {
            partial_range(kb_lo, kb_hi);
        }
        if (cur_kind) emit();
    }
    if (!FILL && lane == 0) rp[qb + 1] = n;
}

// Masks whose visible keys are not one interval per row (dilated bands,
// document ids in any order): every key block that meets the union of the
// block's row intervals is classified from the element rule, so the lists
// stay exact.  A row sees a key of the block iff one of its interval's keys
// there passes the dilation test (j = row position mod g) and has the row's
// document id; the block is FULL iff every row of the block sees every key
// of it.  One wavefront per (copy, query block) as above.
constexpr int kMaxIds = 8;  // distinct document ids per key block on the fast test

template <bool FILL>
__global__ __launch_bounds__(256) void runs_exact_kernel(const BlocksLaunch a) {
    const i64 wg = (i64)blockIdx.x * 4 + (threadIdx.x >> 6);
    const i64 nqb = a.n_qblocks;
    if (wg >= a.copies * nqb) return;
    const int lane = threadIdx.x & 63;
    const i64 copy = wg / nqb, qb = wg % nqb;
    const MaskDev& m = a.mask;
    const i64 lq = m.lq, lk = m.lk;
    const int g = m.dilation;
    const bool docs = m.seg_mode == 3;
    const int* kid = docs ? m.ids_kv + copy * lk : nullptr;
    const int per_lane = a.bq / 64;
    int rlo[kMaxRowsPerLane], rhi[kMaxRowsPerLane], rres[kMaxRowsPerLane], rdoc[kMaxRowsPerLane];
    bool rex[kMaxRowsPerLane];
    int mn_lo = 0x7fffffff, mx_hi = 0;
#pragma unroll
    for (int t = 0; t < kMaxRowsPerLane; ++t) {
        const i64 r = qb * a.bq + lane + 64 * t;
        rex[t] = t < per_lane && r < lq;
        rlo[t] = rex[t] ? a.row_lo[copy * lq + r] : 0;
        rhi[t] = rex[t] ? a.row_hi[copy * lq + r] : 0;
        // the residue mod g of the keys this row can see: (r - kv_offset) mod g
        const i64 pos = r - m.kv_offset;
        rres[t] = (int)(((pos % g) + g) % g);
        rdoc[t] = (rex[t] && docs) ? m.ids_q[copy * lq + r] : 0;
        if (rex[t] && rlo[t] < rhi[t]) { mn_lo = min(mn_lo, rlo[t]); mx_hi = max(mx_hi, rhi[t]); }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mn_lo = min(mn_lo, __shfl_xor(mn_lo, o));
        mx_hi = max(mx_hi, __shfl_xor(mx_hi, o));
    }
    i64* rp = a.row_ptr + copy * (nqb + 1);
    const i64 out = FILL ? rp[qb] : 0;
    i64 n = 0;
    int cur_kind = 0, cur_b = 0, cur_e = 0;
    auto emit = [&]() {
        if (FILL && lane == 0) {
            const i64 slot = out + n;
            if (slot < a.capacity) {
                a.run_begin[copy * a.capacity + slot] = cur_b;
                a.run_end[copy * a.capacity + slot] = cur_e;
                a.run_kind[copy * a.capacity + slot] = (uint8_t)cur_kind;
            }
        }
        ++n;
    };
    if (mx_hi > 0) {
        const int kb_lo = mn_lo / a.bkv;
        const int kb_hi = (int)((mx_hi + (i64)a.bkv - 1) / a.bkv);
        for (int kb = kb_lo; kb < kb_hi; ++kb) {
            const int j0 = kb * a.bkv, j1 = (int)min((i64)j0 + a.bkv, lk);
            // document ids of the block's keys: their range, for quick tests
            int dmin = 0x7fffffff, dmax = (int)0x80000000;
            if (docs) {
                for (int j = j0 + lane; j < j1; j += 64) {
                    dmin = min(dmin, kid[j]);
                    dmax = max(dmax, kid[j]);
                }
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) {
                    dmin = min(dmin, __shfl_xor(dmin, o));
                    dmax = max(dmax, __shfl_xor(dmax, o));
                }
            }
            // The block's distinct document ids, up to kMaxIds (ballots over the
            // keys, one id per round): a row whose interval covers the whole
            // block sees it iff its id is among them, with no key scan.
            int dset[kMaxIds];
            int nd = 0;
            bool few = docs && g == 1;
            if (few) {
                for (int u0 = j0; u0 < j1 && few; u0 += 64) {
                    const int j = u0 + lane;
                    const int myid = j < j1 ? kid[j] : 0;
                    unsigned long long left = __ballot(j < j1);
                    while (left) {
                        const int src = __builtin_ctzll(left);
                        const int d = __shfl(myid, src);
                        bool known = false;
                        for (int i = 0; i < nd; ++i) known |= dset[i] == d;
                        if (!known) {
                            if (nd == kMaxIds) { few = false; break; }
                            dset[nd++] = d;
                        }
                        left &= ~__ballot(myid == d);
                    }
                }
            }
            bool sees = false, misses = false;  // some row sees a key / some row misses a key
#pragma unroll
            for (int t = 0; t < kMaxRowsPerLane; ++t) {
                if (!rex[t]) continue;
                const int lo = max(rlo[t], j0), hi = min(rhi[t], j1);
                bool vis = false;
                if (few && lo == j0 && hi == j1) {
                    for (int i = 0; i < nd; ++i) vis |= dset[i] == rdoc[t];
                } else if (lo < hi && (!docs || (rdoc[t] >= dmin && rdoc[t] <= dmax))) {
                    // first key >= lo with the row's residue, then every g-th
                    int j = lo + ((rres[t] - lo % g) % g + g) % g;
                    if (!docs) {
                        vis = j < hi;
                    } else {
                        for (; j < hi && !vis; j += g) vis = kid[j] == rdoc[t];
                    }
                }
                sees |= vis;
                // FULL needs every key of the block: all in the interval, all
                // with the residue (one key when g > 1), all with the row's id
                const bool full = rlo[t] <= j0 && rhi[t] >= j1 && (g == 1 || (j1 - j0 == 1 && j0 % g == rres[t])) &&
                                  (!docs || (dmin == rdoc[t] && dmax == rdoc[t]));
                misses |= !full;
            }
            const int kind = __ballot(sees) == 0 ? BWA_TILE_SKIP
                             : (__ballot(misses) == 0 ? BWA_TILE_FULL : BWA_TILE_PARTIAL);
            if (kind == BWA_TILE_SKIP) {
                if (cur_kind) { emit(); cur_kind = 0; }
            } else if (cur_kind == kind && cur_e == kb) {
                cur_e = kb + 1;
            } else {
                if (cur_kind) emit();
                cur_kind = kind; cur_b = kb; cur_e = kb + 1;
            }
        }
        if (cur_kind) emit();
    }
    if (!FILL && lane == 0) rp[qb + 1] = n;
}

// In-place inclusive scan of row_ptr[1..nqb] (counts) -> CSR offsets;
// row_ptr[0] = 0.  One workgroup per list copy.
__global__ __launch_bounds__(1024) void scan_kernel(const BlocksLaunch a) {
    __shared__ i64 part[1024];
    const i64 nqb = a.n_qblocks;
    i64* v = a.row_ptr + (i64)blockIdx.x * (nqb + 1) + 1;
    const int t = threadIdx.x;
    if (t == 0) v[-1] = 0;
    const i64 chunk = (nqb + 1023) / 1024;
    const i64 s = t * chunk, e = min(nqb, s + chunk);
    i64 sum = 0;
    for (i64 i = s; i < e; ++i) sum += v[i];
    part[t] = sum;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
        const i64 x = (t >= o) ? part[t - o] : 0;
        __syncthreads();
        part[t] += x;
        __syncthreads();
    }
    i64 run = part[t] - sum;  // exclusive prefix of this thread's chunk
    for (i64 i = s; i < e; ++i) { run += v[i]; v[i] = run; }
}

}  // namespace

hipError_t launch_block_mask_build(const BlocksLaunch& a, hipStream_t stream) {
    const i64 nrows = a.copies * a.mask.lq;
    if (nrows > 0)
        hipLaunchKernelGGL(rows_kernel, dim3((unsigned)((nrows + 255) / 256)), dim3(256), 0, stream, a);
    const i64 waves = a.copies * a.n_qblocks;
    const unsigned grid = (unsigned)((waves + 3) / 4);
    const bool exact = a.mask.dilation > 1 || a.mask.seg_mode == 3;
    if (waves > 0) {
        if (exact) hipLaunchKernelGGL(runs_exact_kernel<false>, dim3(grid), dim3(256), 0, stream, a);
        else hipLaunchKernelGGL(runs_kernel<false>, dim3(grid), dim3(256), 0, stream, a);
    }
    if (a.copies > 0)
        hipLaunchKernelGGL(scan_kernel, dim3((unsigned)a.copies), dim3(1024), 0, stream, a);
    if (waves > 0) {
        if (exact) hipLaunchKernelGGL(runs_exact_kernel<true>, dim3(grid), dim3(256), 0, stream, a);
        else hipLaunchKernelGGL(runs_kernel<true>, dim3(grid), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace bwa
