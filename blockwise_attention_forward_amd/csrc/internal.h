// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bwattn.h"

namespace bwa {

typedef int64_t i64;

// Resolved mask passed to kernels by value.  All positions are in the
// problem's own coordinates; q_valid/kv_valid are already clamped to
// [0, lq] / [0, lk].
struct MaskDev {
    i64 lq, lk;
    i64 kv_offset;
    i64 q_valid, kv_valid;
    int causal;
    int window;
    int dilation;  // 1 = none
    i64 prefix;    // 0 = none
    int seg_mode;  // 0 none, 1 cu_seqlens, 2 per-token segment ids (non-decreasing), 3 document ids (any order)
    int num_segments;
    const int* cu_q;
    const int* cu_kv;
    const int* ids_q;   // [B][lq]
    const int* ids_kv;  // [B][lk]
};

// Wait until at most n (0 .. 15, wave-uniform) of this wave's vector-memory
// operations are in flight.  The count is exact: with copies of several tiles
// in flight, waiting for "at most 4" when only 2 may remain would let a wave
// pass the barrier before its part of the current tile has landed.
// s_waitcnt fields (gfx9): vmcnt[3:0] and [15:14], expcnt[6:4],
// lgkmcnt[11:8]; the other counters are left at their maxima.
__device__ inline void wait_vmcnt(int n) {
    switch (n) {
        case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
        case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
        case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
        case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
        case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
        case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
        case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
        case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
        case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
        case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
        case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
        case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
        case 13: __builtin_amdgcn_s_waitcnt(0x0F7D); break;
        case 14: __builtin_amdgcn_s_waitcnt(0x0F7E); break;
        case 15: __builtin_amdgcn_s_waitcnt(0x0F7F); break;
        default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
}

// The LDS address (byte offset) of a copy into LDS (a buffer load with an
// LDS destination) as a value that the compiler cannot trace to an LDS
// object.
// Before an LDS read the compiler waits for every copy it cannot tell apart
// from the read's object; a ring indexed at run time is one such object, so
// the first read of a tile would wait for the copies of the tiles ahead,
// issued just before.  With the address opaque it adds no such wait, and the
// kernel orders each tile's copies before its reads itself: wait_vmcnt for
// the wave's own copies, then the workgroup barrier.  (The empty asm keeps a
// known buffer address from being folded back to its LDS object.)
__device__ inline int lds_opaque(const void* p) {
    int a = __builtin_amdgcn_readfirstlane((int)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p);
    asm volatile("" : "+s"(a));
    return a;
}

// Keys visible to query row i of batch element b lie in one interval
// [lo, hi): every term of the mask bounds them from below or above (padding,
// segment, causal, prefix and window terms of the visibility rule in
// bwattn.h).  Except for dilated bands and document ids, every key of the
// interval is visible.  Rows that see nothing return (0, 0).  Segment
// lookups are binary searches over the cumulative lengths or the
// (non-decreasing) per-token ids; nothing is tabulated per token.  Document
// ids (any order) bound nothing here: their keys are tested one by one.
__device__ inline void row_interval(const MaskDev& m, i64 b, i64 i, int& out_lo, int& out_hi) {
    i64 lo = 0, hi = m.kv_valid;
    bool ok = (i >= 0) && (i < m.q_valid);
    if (ok && m.seg_mode == 1) {
        const int S = m.num_segments;
        if (i < (i64)m.cu_q[0] || i >= (i64)m.cu_q[S]) {
            ok = false;
        } else {
            int a = 0, c = S;  // largest s in [0, S) with cu_q[s] <= i
            while (c - a > 1) {
                int mid = (a + c) >> 1;
                if ((i64)m.cu_q[mid] <= i) a = mid; else c = mid;
            }
            lo = max(lo, (i64)m.cu_kv[a]);
            hi = min(hi, (i64)m.cu_kv[a + 1]);
        }
    } else if (ok && m.seg_mode == 2) {
        const int sid = m.ids_q[b * m.lq + i];
        const int* ids = m.ids_kv + b * m.lk;
        i64 a = 0, c = m.lk;  // first key with id >= sid
        while (a < c) {
            i64 mid = (a + c) >> 1;
            if (ids[mid] < sid) a = mid + 1; else c = mid;
        }
        i64 first = a;
        c = m.lk;  // first key with id > sid
        while (a < c) {
            i64 mid = (a + c) >> 1;
            if (ids[mid] <= sid) a = mid + 1; else c = mid;
        }
        lo = max(lo, first);
        hi = min(hi, a);
    }
    if (m.causal) hi = min(hi, max(i - m.kv_offset + 1, m.prefix - m.kv_offset));
    if (m.window > 0) {
        lo = max(lo, i - m.kv_offset - (i64)m.window + 1);
        if (!m.causal) hi = min(hi, i - m.kv_offset + (i64)m.window);
    }
    lo = max(lo, (i64)0);
    if (!ok || lo >= hi) { lo = 0; hi = 0; }
    out_lo = (int)lo;
    out_hi = (int)hi;
}

// ---- launchers (implemented next to their kernels) ------------------------

struct AttnLaunch {
    const void* q; const void* k; const void* v;
    i64 q_sB, q_sL, q_sH, k_sB, k_sL, k_sH, v_sB, v_sL, v_sH;
    void* o; i64 o_sB, o_sL, o_sH;
    float* lse; i64 lse_sB, lse_sH, lse_sL;  // lse[b * lse_sB + h * lse_sH + row * lse_sL]
    int B, H, D;
    int kv_group;  // query heads per key/value head (h reads key/value head h / kv_group)
    i64 Lq, Lk;
    int in_dtype, out_dtype;
    float scale;
    int mode;
    const float* m;
    const uint8_t* gate;
    // carried partial of earlier key chunks (lse_prev != nullptr): merged in the epilogue
    const float* o_prev; i64 op_sB, op_sL, op_sH;
    const float* lse_prev;
    // balanced launch (split_next != nullptr): split_wg persistent workgroups
    // take whole query blocks and pieces of cut blocks from 8 queues (see
    // SplitShare), counters split_next[0..7]
    unsigned long long* split_next;
    int split_s, split_c, split_wg;
    i64 split_tail;
    float* split_lse;       // [split_tail][split_s][rows per block] piece LSEs
    float* split_o;         // [split_tail][split_s][rows per block][D] piece outputs (normalized)
    // run lists (have_blocks != 0)
    int have_blocks;
    const i64* row_ptr; const int* run_begin; const int* run_end; const uint8_t* run_kind;
    const int* row_lo; const int* row_hi;
    i64 list_batch, capacity, n_qblocks;
    int bkv_list;
    MaskDev mask;
};
hipError_t launch_attn_fwd(const AttnLaunch& a, hipStream_t stream);

// Shares of the balanced launch: `units` query blocks (launch order) dealt to
// the 8 XCDs in contiguous shares, as the plain launch's remap deals them.
// Of XCD x's u blocks, the first d = floor(u / c) * c run whole (c compute
// units per XCD); the t = u - d of the last, partial round are cut into s
// pieces each (none when s == 1).  k0 numbers the cut blocks over all XCDs.
struct SplitShare {
    i64 a, d, t, k0;  // first block, whole blocks, cut blocks, first cut index
};
__host__ __device__ inline SplitShare split_share(i64 units, int c, int s, int x) {
    const i64 q = units >> 3, r = units & 7;
    SplitShare sh{0, 0, 0, 0};
    for (int i = 0; i <= x; ++i) {
        const i64 u = q + (i < r ? 1 : 0);
        const i64 d = s > 1 ? (u / c) * c : u;
        if (i == x) {
            sh.a = i * q + (i < r ? i : r);
            sh.d = d;
            sh.t = u - d;
        } else {
            sh.k0 += u - d;
        }
    }
    return sh;
}
// Plan for `units` blocks on n_cus compute units with keys of length lk:
// workgroups, compute units per XCD, pieces per cut block, cut blocks.
struct SplitPlan {
    int wg, c, s;
    i64 tail;
};
constexpr int kMaxSplit = 16;  // pieces per cut block at most
SplitPlan split_plan(i64 units, int n_cus, i64 lk);
i64 split_workspace_bytes(const SplitPlan& sp, int rows_per_block, int D);
// The allocation-free balanced launch keeps its workspace in a static device
// array of this many bytes; noalloc_scratch returns the array's address on
// the current device (looked up once per device).
constexpr i64 kNoAllocScratchBytes = (i64)64 << 20;
hipError_t noalloc_scratch(void** ptr);
void split_workspace_layout(AttnLaunch& a, void* ws, const SplitPlan& sp, int rows_per_block, int D);
int attn_rows_per_block(int dtype, int D);

struct BlocksLaunch {
    MaskDev mask;
    i64 copies;      // list copies (1 or B)
    int bq, bkv;
    i64 n_qblocks, capacity;
    i64* row_ptr; int* run_begin; int* run_end; uint8_t* run_kind;
    int* row_lo; int* row_hi;
};
hipError_t launch_block_mask_build(const BlocksLaunch& a, hipStream_t stream);

constexpr int kMaxChunks = 16;
struct BoundTensor { const void* ptr; i64 L, sB, sL, sH, valid; };
struct BoundLaunch {
    BoundTensor q;
    BoundTensor k[kMaxChunks];
    int n_chunks;
    int B, H, D, dtype;
    int Hk;  // key heads (H a multiple of Hk: query head h reads key head h / (H / Hk))
    const float* kmax_in;
    int n_kmax_in;
    float scale, tau;
    float* kmax_out; float* mmax_out; float* m_out; uint8_t* gate_out;
};
hipError_t launch_fixed_m_bound(const BoundLaunch& a, hipStream_t stream);

// Backward pass: inputs, outputs and the planning arrays in the caller's
// workspace (per-row delta and key intervals, per 64-row query tile
// summaries, per 128-key block query-tile ranges).
struct BwdLaunch {
    const void* q; const void* k; const void* v; const void* o; const void* dout;
    i64 q_sB, q_sL, q_sH, k_sB, k_sL, k_sH, v_sB, v_sL, v_sH, o_sB, o_sL, o_sH, do_sB, do_sL, do_sH;
    const float* lse;
    void* dq; i64 dq_sB, dq_sL, dq_sH;
    void* dk; i64 dk_sB, dk_sL, dk_sH;
    void* dv; i64 dv_sB, dv_sL, dv_sH;
    int B, H, Hk, D, kv_group;
    i64 Lq, Lk;
    int o_dtype, grad_dtype;
    float scale;
    int order;          // BWA_ORDER_*
    const int* perm;    // BWA_ORDER_CUSTOM: device [nkt]
    float* delta;       // [B][H][Lq]
    int* row_lo; int* row_hi;  // [list_batch][Lq]
    int4* qsum;         // [list_batch][nqt]: envelope lo, hi; common part lo, hi
    // Document ids only: 32-bit filters of the ids of each 64-row query tile's
    // rows that see keys, and of each 64-key tile's keys below kv_valid
    // (bit hash(id) set); a tile pair whose filters share no bit has no
    // (row, key) pair of one document.
    unsigned* qbloom;  // [list_batch][nqt]
    unsigned* kbloom;  // [list_batch][nkt]
    // and {1, id} when every row of the query tile that sees keys (every key
    // of the key tile below kv_valid) has document id `id`, else {0, 0}
    int* qdoc;         // [list_batch][nqt][2]
    int* kdoc;         // [list_batch][nkt][2]
    int* kfirst; int* klast;   // [list_batch][nkb]: query tiles meeting the key block
    i64 list_batch, nqt, nkb, nkt;
    MaskDev mask;
};
hipError_t launch_attn_bwd(const BwdLaunch& a, hipStream_t stream);
// dst[(r * H + h) * (Lq / g) + a] = src[h * Lq + r + g * a]: one batch
// element's LSE [H][Lq] in the row order of its g residue classes.
hipError_t launch_lse_gather(const float* src, float* dst, i64 H, i64 Lq, int g, hipStream_t stream);
i64 bwd_workspace_bytes(i64 B, i64 H, i64 Lq, i64 Lk, i64 list_batch);
void bwd_workspace_layout(BwdLaunch& a, void* ws);

constexpr int kMaxParts = 16;
struct MergeLaunch {
    const float* o[kMaxParts];
    const float* lse[kMaxParts];
    i64 sB[kMaxParts], sL[kMaxParts], sH[kMaxParts];
    int n_parts;
    int B, H, D;
    i64 L;
    void* out; i64 out_sB, out_sL, out_sH; int out_dtype;
    float* lse_out;
};
hipError_t launch_lse_merge(const MergeLaunch& a, hipStream_t stream);

}  // namespace bwa
