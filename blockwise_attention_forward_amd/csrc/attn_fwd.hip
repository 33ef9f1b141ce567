// Blockwise attention forward for gfx950 (MI355X).
//
// A workgroup of NW wavefronts handles NW*32 query rows of one (batch, head);
// each wavefront owns 32 rows.  Keys are walked in tiles of 64 (bf16) or 32
// (fp32) in ascending order over the run list of the query block: FULL tiles
// run an unmasked body, PARTIAL tiles (and a ragged last tile) compare every
// key with the row's visible interval.  This is the forward analogue of the
// partial/full tile lists of "Add more optimal dk order optional arg"
// (flash-attention pull request 2512, "Sliding window perf issue"), walked as
// one ordered list ("A simplish fix").  The walk is wave-uniform (scalar
// registers and branches only).
//
// Scores are computed transposed, S^T = K Q^T, on the 32x32x16 bf16 matrix
// cores so that each lane ends up holding one query row's scores: the row
// max and row sum are in-lane reductions plus one cross-half lane swap.  The
// probabilities then feed O^T = V^T P^T straight from the registers the
// scores came out in.  K and V tiles go from HBM straight into LDS with
// buffer loads that write LDS (no register staging), in an XOR swizzle of
// 16-byte chunks chosen so that the operand reads of a wave hit distinct
// banks; V is read back transposed by the LDS transpose-read instruction.
// Tiles circulate in a ring of three (8-wave blocks) or two buffers: the
// copies of the next tiles are in flight while the current one is computed.
// Inside a wave, the tile is processed in halves of 32 keys so that the
// exponentials of one half overlap the matrix-core work of the other.  K/V
// rows are fetched through buffer resources whose range ends at the last
// valid key, so rows past it read as zero without a branch.  The fp32 path
// (32x32x2 fp32 matrix cores, 32-key tiles) stages through registers.
//
// Softmax bodies ("Fixed-m softmax for 2D-ring x Ulysses attention (WAN 2.2)",
// description):
//   online : running row max m, p = exp(s*scale - m*scale), l and O rescaled
//            by exp((m_old - m_new)*scale) when the max moves;
//   fixed-m: p = 2^32 exp(s*scale - m_i) with the caller's per-row bound
//            m_i; no max, no rescale (the constant factor cancels in O and
//            is taken out of LSE).
// Each body is its own loop (a fixed-m launch compiles a single branch-free
// body; that page's Notes measured a 3x loss when two bodies share the hot
// loop).  The gated mode picks one of the two loops per workgroup from the
// head's gate, so fixed-m heads and fallback heads share one grid.
// Exponentials use the hardware base-2 exponential with log2(e) folded into
// the scale; LSE is returned in natural-log units.

#include <algorithm>
#include <mutex>

#include "internal.h"

namespace bwa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Fixed-m reference: p = 2^(kFixedShift) * exp(s - m_i), i.e. the exponent is
// taken against m_i less kFixedShift*ln 2.  With |s| <= m_i the exponents of
// a row lie in [kFixedShift - 2 m_i log2 e, kFixedShift]: the shift moves the
// worst row (every key anti-aligned, s = -m_i) away from the bottom of the
// fp32/bf16 normal range while p stays at most 2^32, so l and O keep more
// than 2^90 of headroom.  The bound's gate admits a head only when
// 2 m_i log2 e <= 116, so the largest p of every row is at least 2^-84 and
// 2^30 keys flushed below 2^-126 carry at most 2^-12 of its weight.
constexpr float kFixedShift = 32.0f;
constexpr float kNegInf = -__builtin_inff();
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

enum { BODY_ONLINE = 0, BODY_FIXED = 1, MODE_GATED = 2 };

// Waves per workgroup of the bf16 kernel (32 query rows each).
#ifndef BWA_BF16_WAVES
#define BWA_BF16_WAVES 8
#endif
constexpr int kBf16Waves = BWA_BF16_WAVES;
// Plain launches whose rows see fewer keys than this (in the mask's own
// terms) run half blocks.
constexpr i64 kHalfBlockKeys = 4096;

__device__ inline i64 xcd_remap(i64 id, i64 n) {
    // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
    // contiguous range of logical work so that the query blocks of one head
    // share that XCD's L2 while they stream the same K/V tiles.
    const i64 q = n >> 3, r = n & 7, x = id & 7, slot = id >> 3;
    return (x < r) ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Value of x in the lane 32 apart, combined with x by max / add.
__device__ inline float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Scalar load (constant address space, uniform address): the value lands in a
// scalar register and is waited for on the scalar/LDS counter, so reading a
// run-list entry does not wait behind the tile copies in flight on the
// vector-memory counter (which counts in order).
template <class T>
__device__ inline T ld_s(const T* p) {
    return *((const __attribute__((address_space(4))) T*)p);
}

// Byte p through the scalar load of its aligned 4-byte word.
__device__ inline int ld_s_u8(const uint8_t* p) {
    const uintptr_t a = (uintptr_t)p;
    const uint32_t w = ld_s((const uint32_t*)(a & ~(uintptr_t)3));
    return (int)((w >> (8 * (a & 3))) & 0xffu);
}

// ---------------------------------------------------------------------------
// Tile walk over runs [kb, ke) of one kind; every value is wave-uniform.
// ---------------------------------------------------------------------------
struct Walk {
    const int* rb; const int* re; const uint8_t* rk;
    int nruns, bkv, Lk;
    bool list;
    int b0, e0, b1, e1, b2, e2;  // inline runs: partial, full, partial

    __device__ inline void get(int r, int& kb, int& ke, int& kind) const {
        if (list) {
            kb = ld_s(rb + r) * bkv;
            ke = min(ld_s(re + r) * bkv, Lk);
            kind = ld_s_u8(rk + r);
        } else if (r == 0) {
            kb = b0; ke = e0; kind = BWA_TILE_PARTIAL;
        } else if (r == 1) {
            kb = b1; ke = e1; kind = BWA_TILE_FULL;
        } else {
            kb = b2; ke = e2; kind = BWA_TILE_PARTIAL;
        }
    }
};

template <int TILE>
struct Cursor {
    int r = -1, j0 = 0, ke = 0, kind = 0;
    // Advance to the next tile; false when the walk is over.
    template <class W>
    __device__ inline bool next(const W& w) {
        j0 += TILE;
        while (j0 >= ke) {
            if (++r >= w.nruns) return false;
            int kb;
            w.get(r, kb, ke, kind);
            j0 = kb;
        }
        return true;
    }
    __device__ inline bool masked(int Lk) const { return kind != BWA_TILE_FULL || j0 + TILE > Lk; }
};

// Tiles of a walk (the count the kernel's cursor visits).
__device__ inline i64 walk_tiles(const Walk& w, int tile) {
    i64 n = 0;
    for (int r = 0; r < w.nruns; ++r) {
        int kb, ke, kind;
        w.get(r, kb, ke, kind);
        if (ke > kb) n += (ke - kb + tile - 1) / tile;
    }
    return n;
}

// A walk cut down to its tiles [t0, t1): the runs from roff on, each run
// clamped to key positions [cb, ce).  Runs are increasing and disjoint, so
// the clamp only changes the first and the last; tiles keep the positions
// they have in the whole walk.
struct ClipWalk {
    Walk w;
    int nruns, Lk, roff, cb, ce;

    __device__ inline void get(int r, int& kb, int& ke, int& kind) const {
        w.get(r + roff, kb, ke, kind);
        kb = max(kb, cb);
        ke = min(ke, ce);
    }
};

template <int TILE>
__device__ inline ClipWalk clip_walk(const Walk& w, i64 t0, i64 t1) {
    ClipWalk c;
    c.w = w;
    c.Lk = w.Lk;
    c.roff = 0;
    c.cb = -0x7fffffff;
    c.ce = 0x7fffffff;
    c.nruns = 0;
    int first = -1;
    i64 t = 0;
    for (int r = 0; r < w.nruns && t0 < t1; ++r) {
        int kb, ke, kind;
        w.get(r, kb, ke, kind);
        const i64 n = ke > kb ? (ke - kb + TILE - 1) / TILE : 0;
        if (n == 0) continue;
        if (first < 0 && t0 < t + n) {
            first = r;
            c.cb = kb + (int)(t0 - t) * TILE;
        }
        if (first >= 0 && t1 <= t + n) {
            c.ce = kb + (int)(t1 - t) * TILE;
            c.roff = first;
            c.nruns = r - first + 1;
            break;
        }
        t += n;
    }
    return c;
}

template <int NT>
__device__ inline void block_reduce4(int& mn_lo, int& mx_hi, int& mx_lo, int& mn_hi, int* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mn_lo = min(mn_lo, __shfl_xor(mn_lo, o));
        mx_hi = max(mx_hi, __shfl_xor(mx_hi, o));
        mx_lo = max(mx_lo, __shfl_xor(mx_lo, o));
        mn_hi = min(mn_hi, __shfl_xor(mn_hi, o));
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[w * 4 + 0] = mn_lo; red[w * 4 + 1] = mx_hi;
        red[w * 4 + 2] = mx_lo; red[w * 4 + 3] = mn_hi;
    }
    __syncthreads();
    mn_lo = red[0]; mx_hi = red[1]; mx_lo = red[2]; mn_hi = red[3];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) {
        mn_lo = min(mn_lo, red[i * 4 + 0]); mx_hi = max(mx_hi, red[i * 4 + 1]);
        mx_lo = max(mx_lo, red[i * 4 + 2]); mn_hi = min(mn_hi, red[i * 4 + 3]);
    }
    __syncthreads();
    mn_lo = uni(mn_lo); mx_hi = uni(mx_hi); mx_lo = uni(mx_lo); mn_hi = uni(mn_hi);
}

// Walk of query block qb.  The lane-level bounds over the lane's rows:
// mn_lo/mx_hi over rows that see something, mx_lo/mn_hi over existing rows
// (0x7fffffff / -1 when such a row sees nothing, which rules out FULL tiles).
template <int TILE, int NT>
__device__ inline Walk make_walk(const AttnLaunch& p, i64 b, i64 qb, int mn_lo, int mx_hi, int mx_lo, int mn_hi,
                                 int* red) {
    Walk w;
    w.Lk = (int)p.Lk;
    w.list = p.have_blocks != 0;
    w.b0 = w.e0 = w.b1 = w.e1 = w.b2 = w.e2 = 0;
    if (w.list) {
        const i64 lb = p.list_batch == 1 ? 0 : b;
        const i64* rp = p.row_ptr + lb * (p.n_qblocks + 1);
        const i64 r0 = min(rp[qb], p.capacity), r1 = min(rp[qb + 1], p.capacity);
        w.rb = p.run_begin + lb * p.capacity + r0;
        w.re = p.run_end + lb * p.capacity + r0;
        w.rk = p.run_kind + lb * p.capacity + r0;
        w.nruns = uni((int)max(r1 - r0, (i64)0));
        w.bkv = p.bkv_list;
        return w;
    }
    // Inline: the rows' intervals are monotone in the row index for every
    // mask this library describes, so the block's visible keys lie in
    // [min lo, max hi) and the tiles inside [max lo, min hi) are full.
    // Visiting a tile with no visible pair is harmless (it is masked), so
    // the walk is correct for any interval mask.
    block_reduce4<NT>(mn_lo, mx_hi, mx_lo, mn_hi, red);
    w.nruns = 3;
    if (mx_hi == 0) { w.nruns = 0; return w; }  // no row of this block sees anything
    const int t0 = (mn_lo / TILE) * TILE, t1 = mx_hi;
    // Dilated bands and document ids hide keys inside the intervals: no tile
    // is known to be full.
    const bool exact_only = p.mask.dilation > 1 || p.mask.seg_mode == 3;
    const bool all_rows = !exact_only && mx_lo != 0x7fffffff && mn_hi >= 0;
    const int f0 = all_rows ? ((mx_lo + TILE - 1) / TILE) * TILE : 0;
    const int f1 = all_rows ? (mn_hi / TILE) * TILE : 0;
    if (!all_rows || f0 >= f1) {
        w.b0 = t0; w.e0 = t1;
        return w;
    }
    w.b0 = t0; w.e0 = f0; w.b1 = f0; w.e1 = f1; w.b2 = f1; w.e2 = t1;
    return w;
}

// ---------------------------------------------------------------------------
// Softmax pieces on the 32x32 accumulator layout: lane l holds column
// (query) l%32 and rows (keys) 8*(r/4) + (l/32)*4 + r%4, r = 0..15.
// ---------------------------------------------------------------------------
template <int NKB>
__device__ inline void apply_mask(f32x16 (&s)[NKB], int j0, int lo, int hi) {
    const int hb = (threadIdx.x >> 5) & 1;
    const int lo_rel = lo - (j0 + hb * 4);
    const unsigned span = (unsigned)max(hi - lo, 0);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
            s[kb][r] = ((unsigned)(off - lo_rel) < span) ? s[kb][r] : kNegInf;
        }
}

// Dilated bands and document ids: keys inside a row's interval that the
// element rule still hides (only tiles listed or walked as PARTIAL).  A key j
// of the interval is visible iff j = row position (mod g) and, with
// document ids, the key's id equals the row's.
struct XMask {
    int g;           // dilation (1 = none)
    unsigned pat;    // bits 0, g, 2g, ... below 32
    const int* kid;  // document ids of this batch element's keys, or nullptr
    int lk;
};

__device__ inline XMask make_xmask(const AttnLaunch& p, i64 b) {
    XMask x;
    x.g = p.mask.dilation;
    x.pat = 0u;
    for (int o = 0; o < 32; o += x.g) x.pat |= 1u << o;
    x.kid = p.mask.seg_mode == 3 ? p.mask.ids_kv + b * p.mask.lk : nullptr;
    x.lk = (int)p.mask.lk;
    return x;
}

// The row's terms: its position mod g, and its document id.
__device__ inline void xmask_row(const AttnLaunch& p, i64 b, i64 row, bool row_ok, int& xres, int& xdoc) {
    const int g = p.mask.dilation;
    const i64 pos = row - p.mask.kv_offset;
    xres = (int)(((pos % g) + g) % g);
    xdoc = (row_ok && p.mask.seg_mode == 3) ? p.mask.ids_q[b * p.mask.lq + row] : 0;
}

// Hide the keys of one 32-key block (first key jb) in the accumulator layout
// (lane: one query row, keys jb + hb*4 + 8*(r/4) + r%4) that the row cannot see.
__device__ inline void xmask32(f32x16& s, int jb, int xres, int xdoc, const XMask& xm) {
    const int hb = (threadIdx.x >> 5) & 1;
    const int jl = jb + hb * 4;  // the key of r = 0
    unsigned bits = 0xffffffffu;
    if (xm.g > 1) {
        const int m = ((xres - jl % xm.g) % xm.g + xm.g) % xm.g;  // offsets with the row's residue: m, m+g, ...
        bits = m < 32 ? (xm.pat << m) : 0u;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int o = 8 * (r >> 2) + (r & 3);
        bool ok = (bits >> o) & 1u;
        if (xm.kid) {
            const int j = jl + o;
            ok = ok && j < xm.lk && xm.kid[j] == xdoc;
        }
        s[r] = ok ? s[r] : kNegInf;
    }
}

// The same for the bf16 walk, with the tile's key ids staged in LDS next to
// its K and V (kidl: ids of the tile's 64 keys; kb0: 0 or 32, the block's
// first key in the tile).  A lane reads its 16 keys' ids as 4 runs of 4.
__device__ inline void xmask32_lds(f32x16& s, int jb, int kb0, int xres, int xdoc, const XMask& xm,
                                   const int* kidl) {
    const int hb = (threadIdx.x >> 5) & 1;
    const int jl = jb + hb * 4;  // the key of r = 0
    unsigned bits = 0xffffffffu;
    if (xm.g > 1) {
        const int m = ((xres - jl % xm.g) % xm.g + xm.g) % xm.g;
        bits = m < 32 ? (xm.pat << m) : 0u;
    }
    i32x4 idg[4] = {};
    if (xm.kid) {
#pragma unroll
        for (int q = 0; q < 4; ++q) idg[q] = *(const i32x4*)(kidl + kb0 + hb * 4 + 8 * q);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int o = 8 * (r >> 2) + (r & 3);
        bool ok = (bits >> o) & 1u;
        if (xm.kid) ok = ok && jl + o < xm.lk && idg[r >> 2][r & 3] == xdoc;
        s[r] = ok ? s[r] : kNegInf;
    }
}

template <int NKB, int NDB>
__device__ inline void online_update(f32x16 (&s)[NKB], f32x16 (&acc)[NDB], float& m_run, float& l_run,
                                     float scale_l2) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = pair_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float ms = m_use * scale_l2;
    // Subtract in score units first: an unchanged max gives exactly 1 (and a
    // row that has seen nothing gives 0) whatever the contraction of the
    // scale multiply.
    const float alpha = fast_exp2((m_run - m_use) * scale_l2);
    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(__builtin_fmaf(s[kb][r], scale_l2, -ms));
            s[kb][r] = e;
            rs += e;
        }
    l_run = l_run * alpha + rs;
    if (alpha != 1.0f) {
#pragma unroll
        for (int d = 0; d < NDB; ++d) acc[d] *= alpha;
    }
    m_run = m_new;
}

template <int NKB>
__device__ inline void fixed_update(f32x16 (&s)[NKB], float& l_run, float scale_l2, float m_l2) {
    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(__builtin_fmaf(s[kb][r], scale_l2, -m_l2));
            s[kb][r] = e;
            rs += e;
        }
    l_run += rs;
}

// Epilogue of one query row (the lane pair l, l + 32 holds it): this call's
// partial is O = acc / l and LSE = reference + ln l (natural-log units).  With
// a previous partial of other key chunks (prev_o != nullptr) the two merge in
// LSE space ("Fixed-m softmax for 2D-ring x Ulysses attention (WAN 2.2)",
// Notes): lse = ln(e^lse + e^lse_prev), O = e^(lse-lse') O + e^(lse_prev-lse')
// O_prev; a side whose LSE is -inf has weight 0 and its O row is not read.
// o_row points at the row's first element (OUT decides fp32 or bf16); lse_at
// is written by the lane with hb == 0.
template <int D, int OUT, int BODY>
__device__ inline void store_rows(const AttnLaunch& p, f32x16 (&acc)[D / 32], float m_run, float l_run,
                                  float m_fixed, bool row_ok, void* o_row, float* lse_at, const float* prev_o,
                                  const float* prev_lse) {
    const int hb = (threadIdx.x >> 5) & 1;
    const float l = pair_sum(l_run);
    if (!row_ok) return;
    const bool any = l > 0.0f;
    float lse = any ? (BODY == BODY_FIXED ? m_fixed - kFixedShift * kLn2 : m_run * p.scale) + __logf(l) : kNegInf;
    const float w_own = any ? 1.0f / l : 0.0f;  // normalizes this call's partial
    float w_cur = 1.0f, w_prev = 0.0f;
    if (prev_o) {
        const float lp = *prev_lse;
        const float mx = fmaxf(lse, lp);
        if (mx != kNegInf) {  // once per row: the accurate exp and log
            const float ec = any ? expf(lse - mx) : 0.0f;
            const float ep = lp != kNegInf ? expf(lp - mx) : 0.0f;
            const float tot = ec + ep;
            w_cur = ec / tot;
            w_prev = ep / tot;
            lse = mx + logf(tot);
        }
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = db * 32 + 8 * g + hb * 4;
            float o0 = acc[db][4 * g] * w_own, o1 = acc[db][4 * g + 1] * w_own;
            float o2 = acc[db][4 * g + 2] * w_own, o3 = acc[db][4 * g + 3] * w_own;
            if (prev_o) {
                // Normalized sides, each product rounded, one add: the same
                // bits whichever side is this call's (both sides of a split
                // unit store their normalized partial as fl(acc * w_own)).
#pragma clang fp contract(off)
                f32x4 pv = {0.0f, 0.0f, 0.0f, 0.0f};
                if (w_prev != 0.0f) pv = *(const f32x4*)(prev_o + d);
                o0 = o0 * w_cur + w_prev * pv[0];
                o1 = o1 * w_cur + w_prev * pv[1];
                o2 = o2 * w_cur + w_prev * pv[2];
                o3 = o3 * w_cur + w_prev * pv[3];
            }
            if (OUT == BWA_F32) {
                f32x4 v = {o0, o1, o2, o3};
                *(f32x4*)((float*)o_row + d) = v;
            } else {
                uint2 v = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
                *(uint2*)((__bf16*)o_row + d) = v;
            }
        }
    if (hb == 0) *lse_at = lse;
}

// The call's own outputs, merged with the caller's carried partial if any.
template <int D, int OUT, int BODY>
__device__ inline void store_out(const AttnLaunch& p, f32x16 (&acc)[D / 32], float m_run, float l_run,
                                 float m_fixed, i64 b, i64 h, i64 row) {
    const bool row_ok = row < p.Lq;
    const i64 r = row_ok ? row : 0;
    const i64 li = (b * p.H + h) * p.Lq + r;  // the carried LSE: [B][H][Lq]
    void* o_row = OUT == BWA_F32 ? (void*)((float*)p.o + b * p.o_sB + r * p.o_sL + h * p.o_sH)
                                 : (void*)((__bf16*)p.o + b * p.o_sB + r * p.o_sL + h * p.o_sH);
    const float* prev_o = p.lse_prev ? p.o_prev + b * p.op_sB + r * p.op_sL + h * p.op_sH : nullptr;
    store_rows<D, OUT, BODY>(p, acc, m_run, l_run, m_fixed, row_ok, o_row, p.lse + b * p.lse_sB + h * p.lse_sH + r * p.lse_sL,
                             prev_o, p.lse_prev ? p.lse_prev + li : nullptr);
}

// ---------------------------------------------------------------------------
// bf16 kernel: NW waves of 32 query rows (BQ = 32*NW rows per workgroup),
// 64-key tiles, 32x32x16 bf16 MFMA.
//
// K and V tiles go from HBM straight into LDS (buffer loads with an LDS
// destination: lane i of an instruction fills bytes [16i, 16i+16) of a 1 KB
// run, and lanes past the buffer's range write zeros).  Each lane picks the
// global 16-byte chunk that belongs at its LDS slot, so the tiles land
// already swizzled and no register staging, transpose or LDS store remains.
//   K tile: row r (key), D/8 chunks, swizzled by k_swz.  The Q K^T operand
//           read (lane: row kb*32 + l%32, chunk ds*2 + l/32) hits distinct
//           chunks of each 256-byte bank window.
//   V tile: row r (key), D/8 chunks, swizzled by v_swz.
//           The P V operand needs V^T (8 keys of one d per lane); it is read
//           with two transposing 64-bit LDS reads: in each group of 16 lanes,
//           lane i receives element i%4 of the 4-element rows addressed by
//           lanes i/4 + 4s (s = 0..3).  Lane 16g + 4s + u therefore points at
//           V[key0 + s][dbase + 16*(g&1) + 4u], and lane l receives
//           V[key0 + 0..3][dbase + l%32]; the XOR puts the 4 rows each
//           half-wave touches in disjoint banks.
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <int D, int NW>
struct Bf16Cfg {
    static constexpr int TILE = 64;
    static constexpr int NT = NW * 64;
    static constexpr int BQ = NW * 32;
    static constexpr int NCH = D / 8;                 // 16-byte chunks per row
    static constexpr int NDB = D / 32;                // 32-wide d blocks of O^T
    static constexpr int NDS = D / 16;                // 16-deep steps of Q K^T
    static constexpr int TILE_BYTES = TILE * D * 2;   // one K or V tile
    static constexpr int RUNS = TILE_BYTES / 1024;    // 1 KB load runs per tile
    static constexpr int RUNS_PER_WAVE = (RUNS + NW - 1) / NW;
    static constexpr int NBUF = NW == 8 ? 3 : 2;      // K/V tile buffers in the copy ring
};

template <int D, int NW>
struct Bf16State {
    using C = Bf16Cfg<D, NW>;
    uint4 qf[C::NDS];
    // Lane byte offsets of the fragment reads inside a tile (computed once per
    // block, see lds_lane_offsets): K fragment of step ds in key block 0, and
    // the first transposing V^T read of d block db.
    int koff[C::NDS];
    int voff[C::NDB];
    f32x16 acc[C::NDB];
    float m_run, l_run, m_fixed, m_l2, scale_l2;
    int lo, hi;
    int xres, xdoc;  // dilated bands / document ids (the XM kernels only)
    // The wave's rows (wave-uniform): every visible key lies in
    // [w_lo_min, w_hi_max); every key of [w_lo_max, w_hi_min) is inside every
    // row's interval (empty when some row of the wave sees nothing); w_doc is
    // the document id of all the wave's rows that see something when they
    // share one (w_doc_one).
    int w_lo_min, w_hi_max, w_lo_max, w_hi_min;
    int w_doc;
    bool w_doc_one;
};

// The wave-level fields of st from the lane's row (lanes l and l + 32 hold
// the same row).
template <int D, int NW>
__device__ inline void wave_rows(Bf16State<D, NW>& st, bool row_ok, int lo, int hi) {
    const bool ne = row_ok && lo < hi;
    int a = ne ? lo : 0x7fffffff, b = ne ? hi : 0;
    int c = row_ok ? (ne ? lo : 0x7fffffff) : 0, d = row_ok ? (ne ? hi : -1) : 0x7fffffff;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        a = min(a, __shfl_xor(a, o));
        b = max(b, __shfl_xor(b, o));
        c = max(c, __shfl_xor(c, o));
        d = min(d, __shfl_xor(d, o));
    }
    st.w_lo_min = uni(a);
    st.w_hi_max = uni(b);
    st.w_lo_max = uni(c);
    st.w_hi_min = uni(d);
    const unsigned long long seen = __builtin_amdgcn_ballot_w64(ne);
    st.w_doc = seen ? __builtin_amdgcn_readlane(st.xdoc, __builtin_ctzll(seen)) : 0;
    st.w_doc_one = __builtin_amdgcn_ballot_w64(ne && st.xdoc != st.w_doc) == 0;
}

// Swizzles of the 16-byte chunk index c of row r.  A 256-byte bank window
// holds one row of D = 128 or two rows of D = 64; the XOR spreads the rows a
// matrix-core operand read touches over distinct chunks of the window.
template <int D> __device__ inline int k_swz(int r, int c) {
    return D == 128 ? c ^ (r & 15) : c ^ ((r >> 1) & 7);
}
template <int D> __device__ inline int v_swz(int r, int c) {
    return D == 128 ? c ^ ((r & 3) << 2) : c ^ (((r >> 1) & 1) << 2);
}

// The lane's byte offsets of its fragment reads within a tile.  The swizzles
// depend on the row only through bits that the key-block (32 rows) and
// 16-key steps leave alone, so one offset per K step ds and one per V d block
// cover every read of a tile: key block kb adds kb*32 rows, V key step kk adds
// kk*16 rows and the second transposing read 8 rows, all constants.  The
// offsets are hidden from the optimizer (empty asm operand), so each read is
// lane offset + (buffer base + constant), with the sum of constants folded
// into the LDS instruction's immediate offset, instead of the buffer base
// being recombined with the lane bits for every read of every ring slot.
template <int D, int NW>
__device__ inline void lds_lane_offsets(Bf16State<D, NW>& st) {
    using C = Bf16Cfg<D, NW>;
    const int lane = threadIdx.x & 63, l32 = lane & 31, hb = lane >> 5;
    const int g1 = (lane >> 4) & 1, s_row = (lane >> 2) & 3, u = lane & 3;
#pragma unroll
    for (int ds = 0; ds < C::NDS; ++ds) {
        st.koff[ds] = l32 * (D * 2) + k_swz<D>(l32, ds * 2 + hb) * 16;
        asm volatile("" : "+v"(st.koff[ds]));
    }
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
        const int r0 = hb * 4 + s_row, c = db * 4 + g1 * 2 + (u >> 1);  // chunk of d = db*32 + 16*g1 + 4u
        st.voff[db] = r0 * (D * 2) + v_swz<D>(r0, c) * 16 + (u & 1) * 8;
        asm volatile("" : "+v"(st.voff[db]));
    }
}

// Issue the HBM -> LDS copies of one K and one V tile (rows past kv_lim read as zero).
// K and V buffer resources for a whole walk (online-only launches): one range
// per tensor slice, from its first row to the end of row kv_lim - 1, with a
// tile's rows addressed by the lane offset plus j0 rows, so no resource is
// rebuilt per tile.  Rows past kv_lim fall outside the range and read as
// zero, as with one range per tile.  Taken only when every row a tile can
// address keeps its byte offset below 2^31.
struct WalkRsrc {
    __amdgpu_buffer_rsrc_t kr, vr;
    int ksl2, vsl2;  // row strides in bytes
    bool whole;
};

template <int D>
__device__ inline WalkRsrc walk_rsrc(const AttnLaunch& p, const __bf16* kbase, const __bf16* vbase, int kv_lim) {
    WalkRsrc w;
    const i64 kb = kv_lim > 0 ? ((i64)(kv_lim - 1) * p.k_sL + D) * 2 : 0;
    const i64 vb = kv_lim > 0 ? ((i64)(kv_lim - 1) * p.v_sL + D) * 2 : 0;
    w.whole = (p.Lk + 64) * (i64)max(p.k_sL, p.v_sL) * 2 < ((i64)1 << 31);
    w.kr = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, w.whole ? (int)kb : 0, kRsrcFlags);
    w.vr = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, w.whole ? (int)vb : 0, kRsrcFlags);
    w.ksl2 = (int)(p.k_sL * 2);
    w.vsl2 = (int)(p.v_sL * 2);
    return w;
}

template <int D, int NW, bool XM = false, bool WR = false>
__device__ inline void bf16_issue_tile(const AttnLaunch& p, const __bf16* kbase, const __bf16* vbase, int j0,
                                       int kv_lim, uint8_t* kl, uint8_t* vl, int* kidl, const XMask& xm,
                                       const WalkRsrc* wr = nullptr) {
    using C = Bf16Cfg<D, NW>;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (XM && xm.kid) {
        // Document ids of the tile's keys (4 bytes per lane; every wave
        // writes the same bytes, so each wave's copy count stays the same).
        const int n = uni(min(max(xm.lk - j0, 0), C::TILE));
        const __amdgpu_buffer_rsrc_t ir = __builtin_amdgcn_make_buffer_rsrc((void*)(xm.kid + j0), 0, n * 4,
                                                                            kRsrcFlags);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ir, (lds_void*)kidl, 4, (unsigned)(lane * 4), 0, 0, 0);
    }
    if (WR && wr->whole) {
        const int ko = j0 * wr->ksl2, vo = j0 * wr->vsl2;
#pragma unroll
        for (int it = 0; it < C::RUNS_PER_WAVE; ++it) {
            const int run = wave * C::RUNS_PER_WAVE + it;
            if (C::RUNS % NW == 0 || run < C::RUNS) {
                const int slot = run * 64 + lane;
                const int r = slot / C::NCH, pc = slot % C::NCH;
                const int kc = k_swz<D>(r, pc), vc = v_swz<D>(r, pc);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr->kr, (lds_void*)(kl + run * 1024), 16,
                                                         (unsigned)(r * wr->ksl2 + kc * 16 + ko), 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr->vr, (lds_void*)(vl + run * 1024), 16,
                                                         (unsigned)(r * wr->vsl2 + vc * 16 + vo), 0, 0, 0);
            }
        }
        return;
    }
    const int nvalid = uni(min(max(kv_lim - j0, 0), C::TILE));
    // The range ends with the last valid row's D elements: reads of later
    // rows fall outside it and return zero.
    const int kbytes = uni(nvalid > 0 ? (int)(((nvalid - 1) * p.k_sL + D) * 2) : 0);
    const int vbytes = uni(nvalid > 0 ? (int)(((nvalid - 1) * p.v_sL + D) * 2) : 0);
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (i64)j0 * p.k_sL), 0, kbytes, kRsrcFlags);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (i64)j0 * p.v_sL), 0, vbytes, kRsrcFlags);
#pragma unroll
    for (int it = 0; it < C::RUNS_PER_WAVE; ++it) {
        const int run = wave * C::RUNS_PER_WAVE + it;
        if (C::RUNS % NW == 0 || run < C::RUNS) {
            const int slot = run * 64 + lane;  // 16-byte slot in the tile
            const int r = slot / C::NCH, pc = slot % C::NCH;
            const int kc = k_swz<D>(r, pc), vc = v_swz<D>(r, pc);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(kl + run * 1024), 16,
                                                     (unsigned)(r * p.k_sL * 2 + kc * 16), 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vl + run * 1024), 16,
                                                     (unsigned)(r * p.v_sL * 2 + vc * 16), 0, 0, 0);
        }
    }
}

// Fragment reads run kPrefetch matrix-core steps ahead of their use.
constexpr int kPrefetch = 4;
// Online softmax keeps its reference max until a row's max grows by more
// than 2^kLazy (base-2 units); probabilities then stay below 2^kLazy, and the
// rescale of O and l is skipped for most tiles.  The result is the same in
// real arithmetic for any reference point.
constexpr float kLazy = 8.0f;

// Softmax of one 32-key half (16 values per lane) in four slices of four
// values, so that the slices can be interleaved with matrix-core work.
struct Half {
    f32x16 s;   // scores, then probabilities
    float rs;   // running row sum of this half (per lane)
    uint4 pb[2];  // bf16 probabilities: keys 0..15 and 16..31 of the half
};

__device__ inline void half_mask(Half& x, int j0, int kb, int lo, int hi) {
    const int hb = (threadIdx.x >> 5) & 1;
    const int lo_rel = lo - (j0 + kb * 32 + hb * 4);
    const unsigned span = (unsigned)max(hi - lo, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        x.s[r] = ((unsigned)(off - lo_rel) < span) ? x.s[r] : kNegInf;
    }
}

// exp of slice q (values 4q..4q+3) and its packing; ms = reference * scale_l2.
__device__ inline void half_exp_slice(Half& x, int q, float scale_l2, float ms) {
#pragma unroll
    for (int r = 4 * q; r < 4 * q + 4; ++r) {
        const float e = fast_exp2(__builtin_fmaf(x.s[r], scale_l2, -ms));
        x.s[r] = e;
        x.rs += e;
    }
    const uint32_t a = pack_bf16x2(x.s[4 * q], x.s[4 * q + 1]);
    const uint32_t b = pack_bf16x2(x.s[4 * q + 2], x.s[4 * q + 3]);
    uint4& pb = x.pb[q >> 1];
    if (q & 1) { pb.z = a; pb.w = b; } else { pb.x = a; pb.y = b; }
}

// The same slice leaving the scores in x.s, for the speculative online order
// below (the half may be redone against a new reference).
__device__ inline void half_exp_slice_keep(Half& x, int q, float scale_l2, float ms) {
    float e[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        e[r] = fast_exp2(__builtin_fmaf(x.s[4 * q + r], scale_l2, -ms));
        x.rs += e[r];
    }
    const uint32_t a = pack_bf16x2(e[0], e[1]);
    const uint32_t b = pack_bf16x2(e[2], e[3]);
    uint4& pb = x.pb[q >> 1];
    if (q & 1) { pb.z = a; pb.w = b; } else { pb.x = a; pb.y = b; }
}

// Whether some row's max in this half exceeds its reference by more than
// 2^kLazy (base 2); mx: the lane's row max.  Nothing is changed.
__device__ inline bool half_online_need(const Half& x, float m_run, float scale_l2, float& mx) {
    const float a0 = fmaxf(fmaxf(x.s[0], x.s[1]), x.s[2]), a1 = fmaxf(fmaxf(x.s[3], x.s[4]), x.s[5]);
    const float a2 = fmaxf(fmaxf(x.s[6], x.s[7]), x.s[8]), a3 = fmaxf(fmaxf(x.s[9], x.s[10]), x.s[11]);
    const float a4 = fmaxf(fmaxf(x.s[12], x.s[13]), x.s[14]);
    const float b0 = fmaxf(fmaxf(a0, a1), a2), b1 = fmaxf(fmaxf(a3, a4), x.s[15]);
    mx = pair_max(fmaxf(b0, b1));
    const bool need = mx * scale_l2 > (m_run == kNegInf ? kNegInf : m_run * scale_l2 + kLazy);
    return __builtin_amdgcn_ballot_w64(need) != 0;
}

// The rare step: reference max(m_run, mx) for the lane's row; returns the
// factor acc and l are scaled by.
__device__ inline float online_move_ref(float& m_run, float mx, float scale_l2) {
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * scale_l2);
    m_run = m_new;
    return alpha;
}

// Online reference update for one half: returns the factor acc and l must be
// scaled by (1 when the reference stays), or sets rescale = false.
__device__ inline float half_online_ref(const Half& x, float& m_run, float scale_l2, bool& rescale) {
    // Tree of three-way maxima: depth 3 instead of a chain of 8.
    const float a0 = fmaxf(fmaxf(x.s[0], x.s[1]), x.s[2]), a1 = fmaxf(fmaxf(x.s[3], x.s[4]), x.s[5]);
    const float a2 = fmaxf(fmaxf(x.s[6], x.s[7]), x.s[8]), a3 = fmaxf(fmaxf(x.s[9], x.s[10]), x.s[11]);
    const float a4 = fmaxf(fmaxf(x.s[12], x.s[13]), x.s[14]);
    const float b0 = fmaxf(fmaxf(a0, a1), a2), b1 = fmaxf(fmaxf(a3, a4), x.s[15]);
    float mx = pair_max(fmaxf(b0, b1));
    const bool need = mx * scale_l2 > (m_run == kNegInf ? kNegInf : m_run * scale_l2 + kLazy);
    rescale = __builtin_amdgcn_ballot_w64(need) != 0;
    float alpha = 1.0f;
    if (rescale) {
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
        alpha = fast_exp2((m_run - m_use) * scale_l2);
        m_run = m_new;
    }
    return alpha;
}

// SPEC (online body only): a half's exponentials use the reference the rows
// already have, while the check whether some row's max has moved past it by
// more than 2^kLazy runs beside them; in the rare case it has, the half is
// redone against the new reference.  The results are those of the plain
// order (check first, then the exponentials), without the check on the
// exponentials' critical path.
template <int D, int NW, int BODY, bool XM, bool SPEC = false>
__device__ inline void bf16_compute_tile(const uint8_t* kl, const uint8_t* vl, Bf16State<D, NW>& st, int j0,
                                         bool masked, const XMask& xm, const int* kidl) {
    using C = Bf16Cfg<D, NW>;
    constexpr int NDS = C::NDS, NDB = C::NDB;
    // K fragment of step i = kb*NDS + ds: row kb*32 + l32, chunk ds*2 + hb
    // (l32 = lane % 32, hb = lane / 32), at the lane's offset for ds.
    auto kfrag = [&](int i) {
        const int kb = i / NDS, ds = i % NDS;
        return *(const uint4*)(kl + st.koff[ds] + kb * 32 * (D * 2));
    };
    // V^T fragment of step j = kk*NDB + db: keys kk*16 + {hb*4 + 0..3} then
    // kk*16 + 8 + {hb*4 + 0..3}, for d = db*32 + l32.
    auto vfrag = [&](int j) {
        const int kk = j / NDB, db = j % NDB;
        const uint8_t* a = vl + st.voff[db] + kk * 16 * (D * 2);  // rows kk*16 + hb*4 + 0..3
        const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
        const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 8 * (D * 2)));  // rows + 8
        uint4 out;
        out.x = __builtin_bit_cast(uint2, x0).x;
        out.y = __builtin_bit_cast(uint2, x0).y;
        out.z = __builtin_bit_cast(uint2, x1).x;
        out.w = __builtin_bit_cast(uint2, x1).y;
        return out;
    };
    auto qk = [&](Half& x, const uint4& kf, int ds) {
        x.s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf),
                                                      __builtin_bit_cast(bf16x8, st.qf[ds]), x.s, 0, 0, 0);
    };
    auto pv = [&](const uint4& vf, const uint4& pb, int db) {
        st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf),
                                                             __builtin_bit_cast(bf16x8, pb), st.acc[db], 0, 0, 0);
    };
    Half h0, h1;
    h0.s = f32x16{}; h1.s = f32x16{};
    h0.rs = 0.0f; h1.rs = 0.0f;

    // A: S^T of keys 0..31 (half 0).
    uint4 kf[2 * NDS];
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) kf[i] = kfrag(i);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
        kf[ds + kPrefetch] = kfrag(ds + kPrefetch);
        qk(h0, kf[ds], ds);
        __builtin_amdgcn_sched_barrier(0);
    }
    // B: S^T of keys 32..63 (half 1) under the softmax of half 0.  The
    // online reference of half 0 is settled after the first matrix-core
    // step, which does not depend on it, so that its reduction runs under it.
    float ms = st.m_l2;  // fixed-m reference (scaled)
    bool resc = false;
    float alpha = 1.0f, mx0 = 0.0f, mx1 = 0.0f;
    if (SPEC) ms = (st.m_run == kNegInf ? 0.0f : st.m_run) * st.scale_l2;
    if (masked) {
        half_mask(h0, j0, 0, st.lo, st.hi);
        if (XM) xmask32_lds(h0.s, j0, 0, st.xres, st.xdoc, xm, kidl);
    }
    uint4 vf[4 * NDB];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
        const int i = NDS + ds;
        if (i + kPrefetch < 2 * NDS) kf[i + kPrefetch] = kfrag(i + kPrefetch);
        else vf[i + kPrefetch - 2 * NDS] = vfrag(i + kPrefetch - 2 * NDS);
        qk(h1, kf[i], ds);
        if constexpr (SPEC) {
            if (ds < 4) half_exp_slice_keep(h0, ds, st.scale_l2, ms);
            if (ds == (NDS > 4 ? 4 : NDS - 1)) resc = half_online_need(h0, st.m_run, st.scale_l2, mx0);
        } else {
            if (BODY == BODY_ONLINE && ds == 0) {
                alpha = half_online_ref(h0, st.m_run, st.scale_l2, resc);
                ms = (st.m_run == kNegInf ? 0.0f : st.m_run) * st.scale_l2;
            }
            if (BODY == BODY_ONLINE ? (ds >= 1 && ds <= 4) : ds < 4)
                half_exp_slice(h0, BODY == BODY_ONLINE ? ds - 1 : ds, st.scale_l2, ms);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!SPEC) {
        // Slices the loop had no step for (online body, fewer than 5 steps).
#pragma unroll
        for (int q = (BODY == BODY_ONLINE ? NDS - 1 : 4); q < 4; ++q) half_exp_slice(h0, q, st.scale_l2, ms);
    }
    if (BODY == BODY_ONLINE && resc) {  // rare: the row max moved by more than 2^kLazy
        if constexpr (SPEC) {
            alpha = online_move_ref(st.m_run, mx0, st.scale_l2);
            ms = (st.m_run == kNegInf ? 0.0f : st.m_run) * st.scale_l2;
            h0.rs = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) half_exp_slice_keep(h0, q, st.scale_l2, ms);
        }
        st.l_run *= alpha;
#pragma unroll
        for (int d = 0; d < NDB; ++d) st.acc[d] *= alpha;
    }
    // C: O^T += V^T P^T for keys 0..31 under the softmax of half 1 (its
    // online reference settled under the first step, as above).
    if (masked) {
        half_mask(h1, j0, 1, st.lo, st.hi);
        if (XM) xmask32_lds(h1.s, j0 + 32, 32, st.xres, st.xdoc, xm, kidl);
    }
    bool resc1 = false;
    float alpha1 = 1.0f;
#pragma unroll
    for (int j = 0; j < 2 * NDB; ++j) {
        if (j + kPrefetch < 4 * NDB) vf[j + kPrefetch] = vfrag(j + kPrefetch);
        pv(vf[j], h0.pb[j / NDB], j % NDB);
        if constexpr (SPEC) {
            if (j < 4) half_exp_slice_keep(h1, j, st.scale_l2, ms);
            if (j == (2 * NDB > 4 ? 4 : 2 * NDB - 1)) resc1 = half_online_need(h1, st.m_run, st.scale_l2, mx1);
        } else {
            if (BODY == BODY_ONLINE && j == 0) {
                alpha1 = half_online_ref(h1, st.m_run, st.scale_l2, resc1);
                ms = (st.m_run == kNegInf ? 0.0f : st.m_run) * st.scale_l2;
            }
            if (BODY == BODY_ONLINE ? (j >= 1 && j <= 4) : j < 4)
                half_exp_slice(h1, BODY == BODY_ONLINE ? j - 1 : j, st.scale_l2, ms);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!SPEC) {
#pragma unroll
        for (int q = (BODY == BODY_ONLINE ? 2 * NDB - 1 : 4); q < 4; ++q) half_exp_slice(h1, q, st.scale_l2, ms);
    }
    if (BODY == BODY_ONLINE && resc1) {
        if constexpr (SPEC) {
            alpha1 = online_move_ref(st.m_run, mx1, st.scale_l2);
            ms = (st.m_run == kNegInf ? 0.0f : st.m_run) * st.scale_l2;
            h1.rs = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) half_exp_slice_keep(h1, q, st.scale_l2, ms);
        }
        st.l_run = (st.l_run + h0.rs) * alpha1;
        h0.rs = 0.0f;
#pragma unroll
        for (int d = 0; d < NDB; ++d) st.acc[d] *= alpha1;
    }
    // D: O^T += V^T P^T for keys 32..63.
#pragma unroll
    for (int j = 2 * NDB; j < 4 * NDB; ++j) {
        if (j + kPrefetch < 4 * NDB) vf[j + kPrefetch] = vfrag(j + kPrefetch);
        pv(vf[j], h1.pb[(j - 2 * NDB) / NDB], j % NDB);
        __builtin_amdgcn_sched_barrier(0);
    }
    st.l_run += h0.rs + h1.rs;
}

// The copy ring: NBUF K/V tile buffers, each its own LDS object, visited in
// a compile-time unrolled order.  Reads of buffer I can then be told apart
// from the copies still landing in the other buffers, so they do not wait
// for them; the explicit wait before each barrier covers the copies of the
// tile about to be used.
template <int D, int NW>
struct Ring {
    using C = Bf16Cfg<D, NW>;
    uint8_t* k[C::NBUF];
    uint8_t* v[C::NBUF];
    int* kid[C::NBUF];  // document ids of the keys (element-test kernels only)
};

template <int D, int NW, int BODY, bool XM, int I, bool SPEC, class W>
__device__ __attribute__((always_inline)) inline bool bf16_step(const AttnLaunch& p, Bf16State<D, NW>& st,
                                                               const W& walk, const Ring<D, NW>& ring,
                                                               Cursor<64>& cur, Cursor<64>& ahead, bool& more,
                                                               int& n_after, const __bf16* kbase,
                                                               const __bf16* vbase, int kv_lim, const XMask& xm,
                                                               const WalkRsrc& wr) {
    using C = Bf16Cfg<D, NW>;
    constexpr int NB = C::NBUF;
    constexpr int LOADS = 2 * C::RUNS_PER_WAVE;
    const int j0 = cur.j0;
    const bool masked = cur.masked(walk.Lk);
    // This tile's copies are complete in every wave, and every wave is done
    // with the buffer the next copy goes to (the previous tile's).
    // At most NB - 2 (0 or 1) later tiles are in flight: a compile-time count
    // either way, not a branch tree over the run-time product.
    if (NB == 3 && n_after) {
        if (XM && xm.kid) wait_vmcnt(LOADS + 1);  // K, V and the key ids
        else wait_vmcnt(LOADS);
    } else {
        wait_vmcnt(0);
    }
    __syncthreads();
    if (more) more = ahead.next(walk);
    if (more) {
        constexpr int J = (I + NB - 1) % NB;
        bf16_issue_tile<D, NW, XM, SPEC>(p, kbase, vbase, ahead.j0, kv_lim, ring.k[J], ring.v[J], ring.kid[J], xm,
                                         &wr);
        ++n_after;
    }
    // Tiles listed as partial, classified again for the wave's own rows: a
    // tile none of them sees is skipped (its terms would all be zero), a tile
    // all of them see whole runs unmasked.  Both give the bits of the masked
    // computation.  With document ids the tile's key ids (in LDS with its K
    // and V) decide too, when the wave's rows share one document.
    bool skip = false, wmasked = masked;
    if (masked) {
        if (j0 + C::TILE <= st.w_lo_min || j0 >= st.w_hi_max) skip = true;
        else if (!XM && j0 >= st.w_lo_max && j0 + C::TILE <= st.w_hi_min) wmasked = false;
        if (XM && !skip && xm.kid && xm.g == 1 && st.w_doc_one) {
            const int lane = threadIdx.x & 63, key = j0 + lane;
            const bool hit = ring.kid[I][lane] == st.w_doc && key >= st.w_lo_min && key < st.w_hi_max;
            const unsigned long long m = __builtin_amdgcn_ballot_w64(hit);
            if (m == 0ull) skip = true;
            else if (m == ~0ull && j0 >= st.w_lo_max && j0 + C::TILE <= st.w_hi_min) wmasked = false;
        }
    }
    if (!skip) bf16_compute_tile<D, NW, BODY, XM, SPEC>(ring.k[I], ring.v[I], st, j0, wmasked, xm, ring.kid[I]);
    const bool have = cur.next(walk);
    if (have) --n_after;
    return have;
}

// Every tile of the walk, accumulated into st; the caller stores the result.
template <int D, int NW, int BODY, bool XM, bool SPEC = false, class W>
__device__ inline void bf16_walk(const AttnLaunch& p, Bf16State<D, NW>& st, const W& walk,
                                 const Ring<D, NW>& ring, i64 b, i64 h) {
    using C = Bf16Cfg<D, NW>;
    constexpr int NB = C::NBUF;
    static_assert(NB == 2 || NB == 3, "ring of 2 or 3 buffers");
    static_assert((2 * C::RUNS_PER_WAVE + 1) * (NB - 2) <= 15, "wait_vmcnt covers at most 15 outstanding copies");
    const i64 hk = (int)h / p.kv_group;  // key/value head of query head h
    const __bf16* kbase = (const __bf16*)p.k + b * p.k_sB + hk * p.k_sH;
    const __bf16* vbase = (const __bf16*)p.v + b * p.v_sB + hk * p.v_sH;
    const int kv_lim = (int)p.mask.kv_valid;
    XMask xm{1, 0u, nullptr, 0};
    if (XM) xm = make_xmask(p, b);
    WalkRsrc wr;
    wr.whole = false;
    if (SPEC) wr = walk_rsrc<D>(p, kbase, vbase, kv_lim);
    // Copies run NB - 1 tiles ahead of the compute.
    Cursor<C::TILE> cur, ahead;
    bool have = cur.next(walk);
    ahead = cur;
    bool more = have;
    int n_after = 0;  // tiles issued beyond the current one
    if (have)
        bf16_issue_tile<D, NW, XM, SPEC>(p, kbase, vbase, ahead.j0, kv_lim, ring.k[0], ring.v[0], ring.kid[0], xm, &wr);
    if (NB == 3) {
        if (more) more = ahead.next(walk);
        if (more) {
            bf16_issue_tile<D, NW, XM, SPEC>(p, kbase, vbase, ahead.j0, kv_lim, ring.k[1], ring.v[1], ring.kid[1], xm,
                                             &wr);
            ++n_after;
        }
    }
    while (have) {
        have = bf16_step<D, NW, BODY, XM, 0, SPEC>(p, st, walk, ring, cur, ahead, more, n_after, kbase, vbase, kv_lim,
                                             xm, wr);
        if (!have) break;
        have = bf16_step<D, NW, BODY, XM, 1, SPEC>(p, st, walk, ring, cur, ahead, more, n_after, kbase, vbase, kv_lim,
                                             xm, wr);
        if (NB == 3) {
            if (!have) break;
            have = bf16_step<D, NW, BODY, XM, NB - 1, SPEC>(p, st, walk, ring, cur, ahead, more, n_after, kbase, vbase,
                                                      kv_lim, xm, wr);
        }
    }
}

template <int D, int NW, int BODY, int OUT, bool XM, bool SPEC = false, class W>
__device__ inline void bf16_run(const AttnLaunch& p, Bf16State<D, NW>& st, const W& walk,
                                const Ring<D, NW>& ring, i64 b, i64 h, i64 row) {
    bf16_walk<D, NW, BODY, XM, SPEC>(p, st, walk, ring, b, h);
    store_out<D, OUT, BODY>(p, st.acc, st.m_run, st.l_run, st.m_fixed, b, h, row);
}

template <int D, int NW, int MODE, int OUT, bool XM>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void attn_fwd_bf16(const AttnLaunch p) {
    using C = Bf16Cfg<D, NW>;
    __shared__ __attribute__((aligned(1024))) uint8_t k0[C::TILE_BYTES], v0[C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t k1[C::TILE_BYTES], v1[C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t k2[C::NBUF == 3 ? C::TILE_BYTES : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t v2[C::NBUF == 3 ? C::TILE_BYTES : 16];
    __shared__ __attribute__((aligned(256))) int kd0[XM ? 64 : 1], kd1[XM ? 64 : 1], kd2[XM ? 64 : 1];
    Ring<D, NW> ring;
    ring.k[0] = k0; ring.v[0] = v0; ring.k[1] = k1; ring.v[1] = v1;
    if (C::NBUF == 3) { ring.k[C::NBUF - 1] = k2; ring.v[C::NBUF - 1] = v2; }
    if (XM) {
        ring.kid[0] = kd0; ring.kid[1] = kd1;
        if (C::NBUF == 3) ring.kid[C::NBUF - 1] = kd2;
    }
    __shared__ int red[4 * NW];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hb = lane >> 5;
    // A query block of the run lists (32 kBf16Waves rows) is taken by SPLIT
    // workgroups of NW waves, each over its own share of the rows.
    constexpr int SPLIT = kBf16Waves / NW;
    static_assert(SPLIT * NW == kBf16Waves, "a list block splits into whole workgroups");
    const i64 nq = p.n_qblocks * SPLIT;
    const i64 logical = xcd_remap(blockIdx.x, gridDim.x);
    const i64 bh = logical / nq;
    const i64 qi = nq - 1 - (logical % nq);
    const i64 qb = qi / SPLIT;  // the list block
    const i64 b = bh / p.H, h = bh % p.H;
    bool fixed = MODE == BODY_FIXED;
    if (p.gate) {
        const bool g = p.gate[bh] != 0;
        if (MODE == MODE_GATED) fixed = g;
        else if (g != (MODE == BODY_FIXED)) return;
    }

    Bf16State<D, NW> st;
    const i64 row = qi * C::BQ + wave * 32 + l32;
    const bool row_ok = row < p.Lq;
    int lo = 0, hi = 0;
    if (row_ok) {
        if (p.have_blocks) {
            const i64 lb = p.list_batch == 1 ? 0 : b;
            lo = p.row_lo[lb * p.Lq + row];
            hi = p.row_hi[lb * p.Lq + row];
        } else {
            row_interval(p.mask, b, row, lo, hi);
        }
    }
    st.lo = lo;
    st.hi = hi;
    // Q^T operand fragments: lane holds Q[row][ds*16 + hb*8 + 0..7].
    const __bf16* qp = (const __bf16*)p.q + b * p.q_sB + row * p.q_sL + h * p.q_sH;
#pragma unroll
    for (int ds = 0; ds < C::NDS; ++ds)
        st.qf[ds] = row_ok ? *(const uint4*)(qp + ds * 16 + hb * 8) : uint4{0, 0, 0, 0};
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) st.acc[d] = f32x16{};
    st.m_run = kNegInf;
    st.l_run = 0.0f;
    st.m_fixed = 0.0f;
    st.m_l2 = 0.0f;
    if (fixed && row_ok) {
        st.m_fixed = p.m[bh * p.Lq + row];
        st.m_l2 = st.m_fixed * kLog2e - kFixedShift;
    }
    st.scale_l2 = p.scale * kLog2e;
    st.xres = 0;
    st.xdoc = 0;
    if (XM) xmask_row(p, b, row, row_ok, st.xres, st.xdoc);
    wave_rows(st, row_ok, lo, hi);
    lds_lane_offsets(st);

    const bool ne = row_ok && lo < hi;
    const Walk w0 = make_walk<C::TILE, C::NT>(p, b, qb, ne ? lo : 0x7fffffff, ne ? hi : 0,
                                              row_ok ? (ne ? lo : 0x7fffffff) : 0,
                                              row_ok ? (ne ? hi : -1) : 0x7fffffff, red);
    if constexpr (SPLIT == 1) {
        if (MODE == MODE_GATED) {
            if (fixed) bf16_run<D, NW, BODY_FIXED, OUT, XM>(p, st, w0, ring, b, h, row);
            else bf16_run<D, NW, BODY_ONLINE, OUT, XM>(p, st, w0, ring, b, h, row);
        } else {
            bf16_run<D, NW, MODE, OUT, XM, MODE == BODY_ONLINE && !XM>(p, st, w0, ring, b, h, row);
        }
    } else {
        // A half block walks its list block's runs clipped to the keys its
        // own rows see (the clip starts on a tile boundary); the tiles
        // outside are those only the other half needs.  An inline walk is
        // already built from these rows.
        ClipWalk walk;
        walk.w = w0;
        walk.nruns = w0.nruns;
        walk.Lk = w0.Lk;
        walk.roff = 0;
        walk.cb = -0x7fffffff;
        walk.ce = 0x7fffffff;
        if (w0.list) {
            int mn = ne ? lo : 0x7fffffff, mx = ne ? hi : 0, u0 = 0, u1 = 0;
            block_reduce4<C::NT>(mn, mx, u0, u1, red);
            if (mx == 0) walk.nruns = 0;  // no row of this half sees anything
            walk.cb = (mn / C::TILE) * C::TILE;
            walk.ce = mx;
        }
        if (MODE == MODE_GATED) {
            if (fixed) bf16_run<D, NW, BODY_FIXED, OUT, XM>(p, st, walk, ring, b, h, row);
            else bf16_run<D, NW, BODY_ONLINE, OUT, XM>(p, st, walk, ring, b, h, row);
        } else {
            bf16_run<D, NW, MODE, OUT, XM, MODE == BODY_ONLINE && !XM>(p, st, walk, ring, b, h, row);
        }
    }
}

// ---------------------------------------------------------------------------
// Balanced launch.  The plain launch runs one workgroup per query block and
// the device deals workgroups to its 8 XCDs round-robin, so each XCD gets an
// equal, contiguous share of blocks (the remap above) and runs it in rounds
// of one block per compute unit.  XCDs do not run at the same speed, and a
// share that is not a multiple of the XCD's units leaves a last, partial
// round, so units idle at the end.  Here one workgroup per compute unit
// loops over queues, one per XCD, of the same shares (so blocks that share a
// head's keys still run together on one XCD's L2): first the share's whole
// blocks, then the blocks of its last partial round cut along their key
// tiles into s pieces each (piece index first, so the pieces running at one
// time stream the same key range).  A workgroup whose queue is empty takes
// items from the next XCD's queue, so fast XCDs take over the slow ones'
// work.  A piece stores its normalized partial and LSE in the workspace; a
// second kernel merges the s partials of each cut block in LSE space, in
// piece order ("Fixed-m softmax for 2D-ring x Ulysses attention (WAN 2.2)",
// Notes: the combine of partials over disjoint key ranges).  Workgroups
// never wait for each other, and the kernel boundary orders the partials
// before the merge.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void zero_ints_kernel(int* p, i64 n) {
    const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0;
}

// Query block u (launch order) skipped by this call (gate and mode).
__device__ inline bool unit_skipped(const AttnLaunch& p, i64 bh) {
    if (!p.gate || p.mode == BWA_MODE_GATED) return false;
    return (p.gate[bh] != 0) != (p.mode == BWA_MODE_FIXED_M);
}

// One item: query block u whole (piece < 0: final output), or piece 'piece'
// of cut block k (partial into the workspace).
template <int D, int NW, int MODE, int OUT>
__device__ inline void bal_item(const AttnLaunch& p, const Ring<D, NW>& ring, int* red, i64 u, int piece, i64 k) {
    using C = Bf16Cfg<D, NW>;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hb = lane >> 5;
    const i64 bh = u / p.n_qblocks;
    const i64 qb = p.n_qblocks - 1 - (u % p.n_qblocks);
    const i64 b = bh / p.H, h = bh % p.H;
    if (unit_skipped(p, bh)) return;
    const bool fixed = MODE == MODE_GATED ? (p.gate && p.gate[bh] != 0) : MODE == BODY_FIXED;

    Bf16State<D, NW> st;
    const i64 row = qb * C::BQ + wave * 32 + l32;
    const bool row_ok = row < p.Lq;
    int lo = 0, hi = 0;
    if (row_ok) {
        if (p.have_blocks) {
            const i64 lb = p.list_batch == 1 ? 0 : b;
            lo = p.row_lo[lb * p.Lq + row];
            hi = p.row_hi[lb * p.Lq + row];
        } else {
            row_interval(p.mask, b, row, lo, hi);
        }
    }
    st.lo = lo;
    st.hi = hi;
    const __bf16* qp = (const __bf16*)p.q + b * p.q_sB + row * p.q_sL + h * p.q_sH;
#pragma unroll
    for (int ds = 0; ds < C::NDS; ++ds)
        st.qf[ds] = row_ok ? *(const uint4*)(qp + ds * 16 + hb * 8) : uint4{0, 0, 0, 0};
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) st.acc[d] = f32x16{};
    st.m_run = kNegInf;
    st.l_run = 0.0f;
    st.m_fixed = 0.0f;
    st.m_l2 = 0.0f;
    if (fixed && row_ok) {
        st.m_fixed = p.m[bh * p.Lq + row];
        st.m_l2 = st.m_fixed * kLog2e - kFixedShift;
    }
    st.scale_l2 = p.scale * kLog2e;
    st.xres = 0;
    st.xdoc = 0;
    wave_rows(st, row_ok, lo, hi);
    lds_lane_offsets(st);
    const bool ne = row_ok && lo < hi;
    const Walk walk = make_walk<C::TILE, C::NT>(p, b, qb, ne ? lo : 0x7fffffff, ne ? hi : 0,
                                                row_ok ? (ne ? lo : 0x7fffffff) : 0,
                                                row_ok ? (ne ? hi : -1) : 0x7fffffff, red);
    auto finish = [&](auto body_tag) {
        constexpr int BODY = decltype(body_tag)::value;
        const i64 n = walk_tiles(walk, C::TILE);
        const int s = piece < 0 ? 1 : p.split_s;
        const int c = piece < 0 ? 0 : piece;
        bf16_walk<D, NW, BODY, false, MODE == BODY_ONLINE>(p, st, clip_walk<C::TILE>(walk, c * n / s, (c + 1) * n / s),
                                                           ring, b, h);
        if (piece < 0) {
            store_out<D, OUT, BODY>(p, st.acc, st.m_run, st.l_run, st.m_fixed, b, h, row);
        } else {
            const i64 slot = k * s + piece;
            const int rib = wave * 32 + l32;
            store_rows<D, BWA_F32, BODY>(p, st.acc, st.m_run, st.l_run, st.m_fixed, row_ok,
                                         p.split_o + (slot * C::BQ + rib) * D, p.split_lse + slot * C::BQ + rib,
                                         nullptr, nullptr);
        }
    };
    if (MODE == MODE_GATED ? fixed : MODE == BODY_FIXED) finish(std::integral_constant<int, BODY_FIXED>{});
    else finish(std::integral_constant<int, BODY_ONLINE>{});
}

template <int D, int NW, int MODE, int OUT>
__global__ __launch_bounds__(NW * 64, 1) void attn_fwd_bf16_bal(const AttnLaunch p) {
    using C = Bf16Cfg<D, NW>;
    __shared__ __attribute__((aligned(1024))) uint8_t k0[C::TILE_BYTES], v0[C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t k1[C::TILE_BYTES], v1[C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t k2[C::NBUF == 3 ? C::TILE_BYTES : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t v2[C::NBUF == 3 ? C::TILE_BYTES : 16];
    Ring<D, NW> ring;
    ring.k[0] = k0; ring.v[0] = v0; ring.k[1] = k1; ring.v[1] = v1;
    if (C::NBUF == 3) { ring.k[C::NBUF - 1] = k2; ring.v[C::NBUF - 1] = v2; }
    __shared__ int red[4 * NW];
    __shared__ i64 s_unit, s_k;
    __shared__ int s_piece, s_xq;

    if (threadIdx.x == 0) s_xq = blockIdx.x & 7;  // this workgroup's XCD: its own queue first
    for (;;) {
        // Every wave is done with the previous item's tile buffers and flags.
        __syncthreads();
        if (threadIdx.x == 0) {
            const i64 U = (i64)p.B * p.H * p.n_qblocks;
            const int s = p.split_s, c = p.split_c;
            int xq = s_xq;
            i64 unit = -1, k = 0;
            int piece = -1;
            // The next item of queue xq; an empty queue stays empty, so move
            // on to the next one (taking work of another XCD) until all are.
            for (int tries = 0; tries < 8; ++tries, xq = (xq + 1) & 7) {
                const SplitShare sh = split_share(U, c, s, xq);
                const i64 i = (i64)atomicAdd(p.split_next + xq, 1ull);
                if (i < sh.d) {
                    unit = sh.a + i;
                    break;
                }
                if (i < sh.d + sh.t * s) {
                    const i64 pc = i - sh.d, j = pc % sh.t;
                    unit = sh.a + sh.d + j;
                    piece = (int)(pc / sh.t);
                    k = sh.k0 + j;
                    break;
                }
            }
            s_xq = xq;
            s_unit = unit;
            s_piece = piece;
            s_k = k;
        }
        __syncthreads();
        const i64 unit = s_unit;
        if (unit < 0) break;
        bal_item<D, NW, MODE, OUT>(p, ring, red, unit, s_piece, s_k);
    }
}

// Merge of the s piece partials of cut block k (one workgroup each) into the
// output rows, in piece order.  Two threads per row, each over half of D.
template <int D, int NW, int OUT>
__global__ __launch_bounds__(NW * 64) void merge_pieces_kernel(const AttnLaunch p) {
    using C = Bf16Cfg<D, NW>;
    constexpr int TPR = NW * 64 / C::BQ;  // threads per row
    constexpr int NV = D / TPR / 4;       // float4 per thread
    const i64 U = (i64)p.B * p.H * p.n_qblocks;
    const i64 k = blockIdx.x;
    int x = 0;
    SplitShare sh = split_share(U, p.split_c, p.split_s, 0);
    while (k >= sh.k0 + sh.t) sh = split_share(U, p.split_c, p.split_s, ++x);
    const i64 u = sh.a + sh.d + (k - sh.k0);
    const i64 bh = u / p.n_qblocks;
    if (unit_skipped(p, bh)) return;
    const i64 qb = p.n_qblocks - 1 - (u % p.n_qblocks);
    const i64 b = bh / p.H, h = bh % p.H;
    const int s = p.split_s;
    const int tid = threadIdx.x, rib = tid / TPR, part = tid % TPR;
    const i64 row = qb * C::BQ + rib;
    if (row >= p.Lq) return;
    const float* lse_k = p.split_lse + k * s * C::BQ + rib;
    const float* o_k = p.split_o + (k * s * C::BQ + rib) * D + part * (D / TPR);
    // A carried partial of other key chunks (lse_prev != nullptr) is part s.
    // o may be o_prev itself: each thread reads its part of the row before it
    // writes it, and the two threads of a row are adjacent lanes of one wave.
    const i64 li = (b * p.H + h) * p.Lq + row;
    const int n_parts = p.lse_prev ? s + 1 : s;
    auto part_lse = [&](int c) { return c < s ? lse_k[c * C::BQ] : p.lse_prev[li]; };
    auto part_o = [&](int c) {
        return c < s ? (const f32x4*)(o_k + (i64)c * C::BQ * D)
                     : (const f32x4*)(p.o_prev + b * p.op_sB + row * p.op_sL + h * p.op_sH + part * (D / TPR));
    };
    float mx = kNegInf;
    for (int c = 0; c < n_parts; ++c) mx = fmaxf(mx, part_lse(c));
    f32x4 acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float lse = kNegInf;
    if (mx != kNegInf) {
        float tot = 0.0f;
        for (int c = 0; c < n_parts; ++c) {
            const float lc = part_lse(c);
            if (lc != kNegInf) tot += expf(lc - mx);
        }
        for (int c = 0; c < n_parts; ++c) {
            const float lc = part_lse(c);
            if (lc == kNegInf) continue;  // an empty part's O rows are not read
            const float w = expf(lc - mx) / tot;
            const f32x4* oc = part_o(c);
#pragma unroll
            for (int i = 0; i < NV; ++i) acc[i] += w * oc[i];
        }
        lse = mx + logf(tot);
    }
    const i64 off = b * p.o_sB + row * p.o_sL + h * p.o_sH + part * (D / TPR);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        if (OUT == BWA_F32) {
            *(f32x4*)((float*)p.o + off + 4 * i) = acc[i];
        } else {
            uint2 v = {pack_bf16x2(acc[i][0], acc[i][1]), pack_bf16x2(acc[i][2], acc[i][3])};
            *(uint2*)((__bf16*)p.o + off + 4 * i) = v;
        }
    }
    if (part == 0) p.lse[b * p.lse_sB + h * p.lse_sH + row * p.lse_sL] = lse;
}

// ---------------------------------------------------------------------------
// fp32 kernel: 32-key tiles, 32x32x2 fp32 MFMA, no reduced-precision step.
// ---------------------------------------------------------------------------
template <int D, int BODY, int OUT, bool XM>
__device__ inline void f32_run(const AttnLaunch& p, const Walk& walk, float* ks, float* vs, const float (&qf)[D / 2],
                               int lo, int hi, float m_fixed, i64 b, i64 h, i64 row) {
    constexpr int TILE = 32, NDB = D / 32, LD = D + 1;
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hb = lane >> 5;
    const float scale_l2 = p.scale * kLog2e, m_l2 = m_fixed * kLog2e - kFixedShift;
    f32x16 acc[NDB];
#pragma unroll
    for (int d = 0; d < NDB; ++d) acc[d] = f32x16{};
    float m_run = kNegInf, l_run = 0.0f;
    const i64 hk = (int)h / p.kv_group;  // key/value head of query head h
    const float* kbase = (const float*)p.k + b * p.k_sB + hk * p.k_sH;
    const float* vbase = (const float*)p.v + b * p.v_sB + hk * p.v_sH;
    const int kv_lim = (int)p.mask.kv_valid;
    XMask xm{1, 0u, nullptr, 0};
    int xres = 0, xdoc = 0;
    if (XM) {
        xm = make_xmask(p, b);
        xmask_row(p, b, row, row < p.Lq, xres, xdoc);
    }
    Cursor<TILE> cur;
    while (cur.next(walk)) {
        const int j0 = cur.j0;
        __syncthreads();
        for (int idx = tid; idx < TILE * D / 4; idx += 256) {
            const int r = idx / (D / 4), c = idx % (D / 4);
            const int j = j0 + r;
            f32x4 kv4 = {0, 0, 0, 0}, vv4 = {0, 0, 0, 0};
            if (j < kv_lim) {
                kv4 = *(const f32x4*)(kbase + (i64)j * p.k_sL + c * 4);
                vv4 = *(const f32x4*)(vbase + (i64)j * p.v_sL + c * 4);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ks[r * LD + c * 4 + e] = kv4[e];
                vs[r * LD + c * 4 + e] = vv4[e];
            }
        }
        __syncthreads();
        f32x16 s[1] = {f32x16{}};
#pragma unroll
        for (int ds = 0; ds < D / 2; ++ds)
            s[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[l32 * LD + ds * 2 + hb], qf[ds], s[0], 0, 0, 0);
        if (cur.masked(walk.Lk)) {
            apply_mask<1>(s, j0, lo, hi);
            if (XM) xmask32(s[0], j0, xres, xdoc, xm);
        }
        if (BODY == BODY_FIXED) fixed_update<1>(s, l_run, scale_l2, m_l2);
        else online_update<1, NDB>(s, acc, m_run, l_run, scale_l2);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int key = 8 * (t >> 2) + hb * 4 + (t & 3);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * LD + db * 32 + l32], s[0][t], acc[db], 0, 0, 0);
        }
    }
    store_out<D, OUT, BODY>(p, acc, m_run, l_run, m_fixed, b, h, row);
}

template <int D, int MODE, int OUT, bool XM>
__global__ __launch_bounds__(256, 1) void attn_fwd_f32(const AttnLaunch p) {
    constexpr int TILE = 32, LD = D + 1;
    __shared__ float ks[TILE * LD];
    __shared__ float vs[TILE * LD];
    __shared__ int red[16];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hb = lane >> 5;
    const i64 logical = xcd_remap(blockIdx.x, gridDim.x);
    const i64 bh = logical / p.n_qblocks;
    const i64 qb = p.n_qblocks - 1 - (logical % p.n_qblocks);
    const i64 b = bh / p.H, h = bh % p.H;
    bool fixed = MODE == BODY_FIXED;
    if (p.gate) {
        const bool g = p.gate[bh] != 0;
        if (MODE == MODE_GATED) fixed = g;
        else if (g != (MODE == BODY_FIXED)) return;
    }
    const i64 row = qb * 128 + wave * 32 + l32;
    const bool row_ok = row < p.Lq;
    int lo = 0, hi = 0;
    if (row_ok) {
        if (p.have_blocks) {
            const i64 lb = p.list_batch == 1 ? 0 : b;
            lo = p.row_lo[lb * p.Lq + row];
            hi = p.row_hi[lb * p.Lq + row];
        } else {
            row_interval(p.mask, b, row, lo, hi);
        }
    }
    const float* qp = (const float*)p.q + b * p.q_sB + row * p.q_sL + h * p.q_sH;
    float qf[D / 2];
#pragma unroll
    for (int ds = 0; ds < D / 2; ++ds) qf[ds] = row_ok ? qp[ds * 2 + hb] : 0.0f;
    const float m_fixed = (fixed && row_ok) ? p.m[bh * p.Lq + row] : 0.0f;
    const bool ne = row_ok && lo < hi;
    const Walk walk = make_walk<TILE, 256>(p, b, qb, ne ? lo : 0x7fffffff, ne ? hi : 0,
                                           row_ok ? (ne ? lo : 0x7fffffff) : 0,
                                           row_ok ? (ne ? hi : -1) : 0x7fffffff, red);
    if (fixed) f32_run<D, BODY_FIXED, OUT, XM>(p, walk, ks, vs, qf, lo, hi, m_fixed, b, h, row);
    else f32_run<D, BODY_ONLINE, OUT, XM>(p, walk, ks, vs, qf, lo, hi, m_fixed, b, h, row);
}

// Whether a plain bf16 launch runs half blocks: when its rows see few keys
// (a window, or a short key range), or with document ids.  Measured on
// 8192 x 8192 with 16 heads: windows of 512 and 2048 keys 8-17% faster,
// dilated bands and document ids 9-10%; causal and dense rows (4096 and
// 8192 keys on average) 0-6% slower, so they keep whole blocks.
inline bool half_blocks(const AttnLaunch& a) {
    if (a.mask.seg_mode == 3) return true;
    i64 keys = a.mask.kv_valid;
    if (a.mask.window > 0) keys = std::min<i64>(keys, (a.mask.causal ? 1 : 2) * (i64)a.mask.window);
    else if (a.mask.causal) keys = (keys + 1) / 2;
    return keys < kHalfBlockKeys;
}

template <int D, int MODE, int OUT>
hipError_t launch_one(const AttnLaunch& a, hipStream_t stream) {
    const i64 grid = a.n_qblocks * (i64)a.B * a.H;
    if (grid == 0) return hipSuccess;
    if (a.split_next) {
        constexpr int NW = kBf16Waves;
        hipLaunchKernelGGL(zero_ints_kernel, dim3(1), dim3(256), 0, stream, (int*)a.split_next, (i64)16);
        hipLaunchKernelGGL((attn_fwd_bf16_bal<D, NW, MODE, OUT>), dim3((unsigned)a.split_wg), dim3(NW * 64), 0,
                           stream, a);
        if (a.split_tail > 0 && a.split_s > 1)
            hipLaunchKernelGGL((merge_pieces_kernel<D, NW, OUT>), dim3((unsigned)a.split_tail), dim3(NW * 64), 0,
                               stream, a);
        return hipGetLastError();
    }
    // Dilated bands and document ids take the kernels with the element test.
    const bool xm = a.mask.dilation > 1 || a.mask.seg_mode == 3;
    if (a.in_dtype == BWA_BF16) {
        constexpr int NW = kBf16Waves;
        if (half_blocks(a)) {
            // Short rows: half blocks of NW / 2 waves, two workgroups per
            // compute unit, so that one's prologue, epilogue and partial
            // tiles overlap the other's products.
            constexpr int NH = NW / 2;
            if (xm)
                hipLaunchKernelGGL((attn_fwd_bf16<D, NH, MODE, OUT, true>), dim3((unsigned)(2 * grid)), dim3(NH * 64),
                                   0, stream, a);
            else
                hipLaunchKernelGGL((attn_fwd_bf16<D, NH, MODE, OUT, false>), dim3((unsigned)(2 * grid)),
                                   dim3(NH * 64), 0, stream, a);
        } else if (xm)
            hipLaunchKernelGGL((attn_fwd_bf16<D, NW, MODE, OUT, true>), dim3((unsigned)grid), dim3(NW * 64), 0,
                               stream, a);
        else
            hipLaunchKernelGGL((attn_fwd_bf16<D, NW, MODE, OUT, false>), dim3((unsigned)grid), dim3(NW * 64), 0,
                               stream, a);
    } else {
        if (xm) hipLaunchKernelGGL((attn_fwd_f32<D, MODE, OUT, true>), dim3((unsigned)grid), dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((attn_fwd_f32<D, MODE, OUT, false>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

template <int D, int MODE>
hipError_t launch_mode(const AttnLaunch& a, hipStream_t stream) {
    return a.out_dtype == BWA_F32 ? launch_one<D, MODE, BWA_F32>(a, stream)
                                  : launch_one<D, MODE, BWA_BF16>(a, stream);
}

template <int D>
hipError_t launch_d(const AttnLaunch& a, hipStream_t stream) {
    if (a.mode == BWA_MODE_FIXED_M) return launch_mode<D, BODY_FIXED>(a, stream);
    if (a.mode == BWA_MODE_GATED) return launch_mode<D, MODE_GATED>(a, stream);
    return launch_mode<D, BODY_ONLINE>(a, stream);
}

}  // namespace

static i64 pad256(i64 x) { return (x + 255) / 256 * 256; }

SplitPlan split_plan(i64 units, int n_cus, i64 lk) {
    SplitPlan sp;
    sp.wg = n_cus;
    sp.c = std::max(1, n_cus / 8);
    // Pieces of about a quarter of a block, at least 8 tiles each; the cut
    // blocks are each XCD's last, partial round.
    const i64 tiles = std::max<i64>(1, (lk + 63) / 64);
    sp.s = (int)std::max<i64>(1, std::min<i64>(std::min<i64>(kMaxSplit, 4), tiles / 8));
    const SplitShare last = split_share(units, sp.c, sp.s, 7);
    sp.tail = last.k0 + last.t;
    return sp;
}

i64 split_workspace_bytes(const SplitPlan& sp, int rows_per_block, int D) {
    const i64 parts = sp.tail * sp.s * rows_per_block;
    return 256 + pad256(parts * 4) + parts * D * 4;
}

void split_workspace_layout(AttnLaunch& a, void* ws, const SplitPlan& sp, int rows_per_block, int D) {
    uint8_t* base = (uint8_t*)ws;
    const i64 parts = sp.tail * sp.s * rows_per_block;
    a.split_next = (unsigned long long*)base;
    base += 256;
    a.split_lse = (float*)base;
    base += pad256(parts * 4);
    a.split_o = (float*)base;
    a.split_s = sp.s;
    a.split_c = sp.c;
    a.split_tail = sp.tail;
    a.split_wg = sp.wg;
    (void)D;
}

// Workspace of the allocation-free balanced launch: queue counters and the
// cut blocks' partials.  Every device the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: kernels get the address that hipGetSymbolAddress returns
// for the current device.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

int attn_rows_per_block(int dtype, int D) { return dtype == BWA_BF16 ? 32 * kBf16Waves : 128; }

hipError_t launch_attn_fwd(const AttnLaunch& a, hipStream_t stream) {
    if (a.D == 64) return launch_d<64>(a, stream);
    return launch_d<128>(a, stream);
}

}  // namespace bwa
