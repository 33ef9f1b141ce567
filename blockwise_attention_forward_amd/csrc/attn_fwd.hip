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
// scores came out in.  V is staged transposed in LDS (a register transpose
// per thread while storing), K row-major; both use an XOR swizzle of 16-byte
// chunks so that the matrix-core operand reads of a wave hit distinct banks.
// Tiles are double-buffered: the global loads of the next tile are in flight
// while the current tile is computed.  K/V rows are fetched through buffer
// resources whose range ends at the last valid key, so rows past it read as
// zero without a branch.
//
// Softmax bodies ("Fixed-m softmax for 2D-ring x Ulysses attention (WAN 2.2)",
// description):
//   online : running row max m, p = exp(s*scale - m*scale), l and O rescaled
//            by exp((m_old - m_new)*scale) when the max moves;
//   fixed-m: p = exp(s*scale - m_i) with the caller's per-row bound m_i; no
//            max, no rescale.
// Each body is its own loop (a fixed-m launch compiles a single branch-free
// body; that page's Notes measured a 3x loss when two bodies share the hot
// loop).  The gated mode picks one of the two loops per workgroup from the
// head's gate, so fixed-m heads and fallback heads share one grid.
// Exponentials use the hardware base-2 exponential with log2(e) folded into
// the scale; LSE is returned in natural-log units.

#include "internal.h"

namespace bwa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

enum { BODY_ONLINE = 0, BODY_FIXED = 1, MODE_GATED = 2 };

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
            kb = uni(rb[r] * bkv);
            ke = uni(min(re[r] * bkv, Lk));
            kind = uni((int)rk[r]);
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
    __device__ inline bool next(const Walk& w) {
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

// Walk of query block qb (BQ rows).  lo/hi: this lane's row interval.
template <int TILE, int NT>
__device__ inline Walk make_walk(const AttnLaunch& p, i64 b, i64 qb, int lo, int hi, bool row_exists,
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
    const bool ne = row_exists && lo < hi;
    int mn_lo = ne ? lo : 0x7fffffff, mx_hi = ne ? hi : 0;
    int mx_lo = row_exists ? (ne ? lo : 0x7fffffff) : 0;
    int mn_hi = row_exists ? (ne ? hi : -1) : 0x7fffffff;
    block_reduce4<NT>(mn_lo, mx_hi, mx_lo, mn_hi, red);
    w.nruns = 3;
    if (mx_hi == 0) { w.nruns = 0; return w; }  // no row of this block sees anything
    const int t0 = (mn_lo / TILE) * TILE, t1 = mx_hi;
    const bool all_rows = mx_lo != 0x7fffffff && mn_hi >= 0;
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

// Epilogue: O = acc / l, LSE = ln-sum-exp; rows that saw nothing -> 0, -inf.
template <int D, int OUT, int BODY>
__device__ inline void store_out(const AttnLaunch& p, f32x16 (&acc)[D / 32], float m_run, float l_run,
                                 float m_fixed, i64 b, i64 h, i64 row) {
    const int hb = (threadIdx.x >> 5) & 1;
    const float l = pair_sum(l_run);
    if (row >= p.Lq) return;
    const bool any = l > 0.0f;
    const float inv = any ? 1.0f / l : 0.0f;
    const i64 base = b * p.o_sB + row * p.o_sL + h * p.o_sH;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = db * 32 + 8 * g + hb * 4;
            const float o0 = acc[db][4 * g] * inv, o1 = acc[db][4 * g + 1] * inv;
            const float o2 = acc[db][4 * g + 2] * inv, o3 = acc[db][4 * g + 3] * inv;
            if (OUT == BWA_F32) {
                f32x4 v = {o0, o1, o2, o3};
                *(f32x4*)((float*)p.o + base + d) = v;
            } else {
                uint2 v = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
                *(uint2*)((__bf16*)p.o + base + d) = v;
            }
        }
    if (hb == 0) {
        float lse = kNegInf;
        if (any) lse = (BODY == BODY_FIXED ? m_fixed : m_run * p.scale) + __logf(l);
        p.lse[(b * p.H + h) * p.Lq + row] = lse;
    }
}

// ---------------------------------------------------------------------------
// bf16 kernel: NW waves (BQ = 32*NW rows), 64-key tiles, 32x32x16 bf16 MFMA.
// ---------------------------------------------------------------------------
template <int D, int NW>
struct Bf16Cfg {
    static constexpr int TILE = 64;
    static constexpr int NT = NW * 64;
    static constexpr int BQ = NW * 32;
    static constexpr int NCH = D / 8;               // 16-byte chunks per K row
    static constexpr int NDB = D / 32;              // 32-wide d blocks of O^T
    static constexpr int NDS = D / 16;              // 16-deep steps of Q K^T
    static constexpr int KCH = TILE * NCH;          // K chunks per tile
    static constexpr int KL = (KCH + NT - 1) / NT;  // K chunks per thread
    static constexpr int VK = (TILE * NCH) / NT >= 4 ? 4 : 2;  // keys per V task
    static constexpr int VT = (TILE / VK) * NCH;    // V tasks per tile
    static constexpr int VL = (VT + NT - 1) / NT;   // V tasks per thread
    static constexpr int TILE_BYTES = TILE * D * 2;
};

template <int D, int NW>
struct Bf16State {
    using C = Bf16Cfg<D, NW>;
    uint4 qf[C::NDS];
    f32x16 acc[C::NDB];
    float m_run, l_run, m_fixed, m_l2, scale_l2;
    int lo, hi;
    uint4 sk[C::KL];
    uint4 sv[C::VL][C::VK];
};

template <int D, int NW>
__device__ inline void bf16_load_tile(const AttnLaunch& p, Bf16State<D, NW>& st, const __bf16* kbase,
                                      const __bf16* vbase, int j0, int kv_lim) {
    using C = Bf16Cfg<D, NW>;
    const int tid = threadIdx.x;
    // Range of the buffer resources: the tile's rows below kv_lim (wave-uniform).
    const int nvalid = uni(min(max(kv_lim - j0, 0), C::TILE));
    const int kbytes = uni((int)(nvalid * p.k_sL * 2)), vbytes = uni((int)(nvalid * p.v_sL * 2));
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (i64)j0 * p.k_sL), 0, kbytes, kRsrcFlags);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (i64)j0 * p.v_sL), 0, vbytes, kRsrcFlags);
#pragma unroll
    for (int it = 0; it < C::KL; ++it) {
        const int lin = it * C::NT + tid, r = lin / C::NCH, c = lin % C::NCH;
        if (C::KCH % C::NT == 0 || lin < C::KCH)
            st.sk[it] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, (int)(r * p.k_sL * 2 + c * 16), 0, 0));
    }
#pragma unroll
    for (int it = 0; it < C::VL; ++it) {
        const int task = it * C::NT + tid, g = task / C::NCH, cd = task % C::NCH;
        if (C::VT % C::NT == 0 || task < C::VT) {
#pragma unroll
            for (int e = 0; e < C::VK; ++e)
                st.sv[it][e] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(
                               vr, (int)((g * C::VK + e) * p.v_sL * 2 + cd * 16), 0, 0));
        }
    }
}

// V^T tile layout: row d (D rows of TILE keys, 128 bytes), 8 chunks of 16
// bytes.  Chunk kk*2 + hb holds keys kk*16 + {hb*4 + 0..3, 8 + hb*4 + 0..3},
// the 8 keys the matrix-core operand of lane half hb needs for k-step kk;
// the chunk index is XOR-swizzled with (d ^ d>>3) & 7.
__device__ inline int vt_offset(int d, int key) {
    const int kk = key >> 4, kin = key & 15;
    const int hb = (kin >> 2) & 1, half = kin >> 3, pos = kin & 3;
    const int chunk = kk * 2 + hb;
    return d * 128 + ((chunk ^ ((d ^ (d >> 3)) & 7)) * 16) + half * 8 + pos * 2;
}

template <int D, int NW>
__device__ inline void bf16_store_tile(uint8_t* kl, uint8_t* vl, const Bf16State<D, NW>& st) {
    using C = Bf16Cfg<D, NW>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < C::KL; ++it) {
        const int lin = it * C::NT + tid, r = lin / C::NCH, c = lin % C::NCH;
        if (C::KCH % C::NT == 0 || lin < C::KCH)
            *(uint4*)(kl + r * (D * 2) + ((c ^ (r & (C::NCH - 1))) * 16)) = st.sk[it];
    }
#pragma unroll
    for (int it = 0; it < C::VL; ++it) {
        const int task = it * C::NT + tid, g = task / C::NCH, cd = task % C::NCH;
        if (C::VT % C::NT == 0 || task < C::VT) {
            const int key0 = g * C::VK;
#pragma unroll
            for (int wi = 0; wi < 4; ++wi)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int d = cd * 8 + wi * 2 + s;
                    uint32_t w[C::VK];
#pragma unroll
                    for (int e = 0; e < C::VK; ++e) {
                        const uint32_t x = ((const uint32_t*)&st.sv[it][e])[wi];
                        w[e] = s ? (x >> 16) : (x & 0xffffu);
                    }
                    if (C::VK == 4) {
                        uint2 val = {w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
                        *(uint2*)(vl + vt_offset(d, key0)) = val;
                    } else {
                        *(uint32_t*)(vl + vt_offset(d, key0)) = w[0] | (w[1] << 16);
                    }
                }
        }
    }
}

template <int D, int NW, int BODY>
__device__ inline void bf16_compute_tile(const uint8_t* kl, const uint8_t* vl, Bf16State<D, NW>& st,
                                         int j0, bool masked) {
    using C = Bf16Cfg<D, NW>;
    const int lane = threadIdx.x & 63, l32 = lane & 31, hb = lane >> 5;
    f32x16 s[2] = {f32x16{}, f32x16{}};
    // K fragments: row kb*32 + l32, chunk ds*2 + hb (swizzled); prefetched one step ahead.
    const int kr0 = l32, kr1 = 32 + l32;
    auto kfrag = [&](int r, int ds) {
        const int c = ds * 2 + hb;
        return *(const uint4*)(kl + r * (D * 2) + ((c ^ (r & (C::NCH - 1))) * 16));
    };
    uint4 a0 = kfrag(kr0, 0), a1 = kfrag(kr1, 0);
#pragma unroll
    for (int ds = 0; ds < C::NDS; ++ds) {
        uint4 n0 = a0, n1 = a1;
        if (ds + 1 < C::NDS) { n0 = kfrag(kr0, ds + 1); n1 = kfrag(kr1, ds + 1); }
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a0),
                                                       __builtin_bit_cast(bf16x8, st.qf[ds]), s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a1),
                                                       __builtin_bit_cast(bf16x8, st.qf[ds]), s[1], 0, 0, 0);
        a0 = n0; a1 = n1;
    }
    auto vfrag = [&](int db, int kk) {
        const int d = db * 32 + l32, c = kk * 2 + hb;
        return *(const uint4*)(vl + d * (C::TILE * 2) + ((c ^ ((d ^ (d >> 3)) & 7)) * 16));
    };
    uint4 vf = vfrag(0, 0);
    if (masked) apply_mask<2>(s, j0, st.lo, st.hi);
    if (BODY == BODY_FIXED) fixed_update<2>(s, st.l_run, st.scale_l2, st.m_l2);
    else online_update<2, C::NDB>(s, st.acc, st.m_run, st.l_run, st.scale_l2);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int kb = kk >> 1, r0 = 8 * (kk & 1);
        uint4 pb;
        pb.x = pack_bf16x2(s[kb][r0 + 0], s[kb][r0 + 1]);
        pb.y = pack_bf16x2(s[kb][r0 + 2], s[kb][r0 + 3]);
        pb.z = pack_bf16x2(s[kb][r0 + 4], s[kb][r0 + 5]);
        pb.w = pack_bf16x2(s[kb][r0 + 6], s[kb][r0 + 7]);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            uint4 nv = vf;
            const int step = kk * C::NDB + db + 1;
            if (step < 4 * C::NDB) nv = vfrag(step % C::NDB, step / C::NDB);
            st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, vf), __builtin_bit_cast(bf16x8, pb), st.acc[db], 0, 0, 0);
            vf = nv;
        }
    }
}

template <int D, int NW, int BODY, int OUT>
__device__ inline void bf16_run(const AttnLaunch& p, Bf16State<D, NW>& st, const Walk& walk, uint8_t* lds,
                                i64 b, i64 h, i64 row) {
    using C = Bf16Cfg<D, NW>;
    const __bf16* kbase = (const __bf16*)p.k + b * p.k_sB + h * p.k_sH;
    const __bf16* vbase = (const __bf16*)p.v + b * p.v_sB + h * p.v_sH;
    const int kv_lim = (int)p.mask.kv_valid;
    Cursor<C::TILE> cur;
    bool have = cur.next(walk);
    int buf = 0;
    if (have) {
        bf16_load_tile<D, NW>(p, st, kbase, vbase, cur.j0, kv_lim);
        bf16_store_tile<D, NW>(lds, lds + C::TILE_BYTES, st);
        __syncthreads();
    }
    while (have) {
        const int j0 = cur.j0;
        const bool masked = cur.masked(walk.Lk);
        have = cur.next(walk);
        if (have) bf16_load_tile<D, NW>(p, st, kbase, vbase, cur.j0, kv_lim);
        const uint8_t* kl = lds + buf * 2 * C::TILE_BYTES;
        bf16_compute_tile<D, NW, BODY>(kl, kl + C::TILE_BYTES, st, j0, masked);
        if (have) {
            uint8_t* nl = lds + (buf ^ 1) * 2 * C::TILE_BYTES;
            bf16_store_tile<D, NW>(nl, nl + C::TILE_BYTES, st);
            __syncthreads();
            buf ^= 1;
        }
    }
    store_out<D, OUT, BODY>(p, st.acc, st.m_run, st.l_run, st.m_fixed, b, h, row);
}

template <int D, int NW, int MODE, int OUT>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void attn_fwd_bf16(const AttnLaunch p) {
    using C = Bf16Cfg<D, NW>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * C::TILE_BYTES];
    __shared__ int red[4 * NW];

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

    Bf16State<D, NW> st;
    const i64 row = qb * C::BQ + wave * 32 + l32;
    const bool row_ok = row < p.Lq;
    st.lo = 0; st.hi = 0;
    if (row_ok) {
        if (p.have_blocks) {
            const i64 lb = p.list_batch == 1 ? 0 : b;
            st.lo = p.row_lo[lb * p.Lq + row];
            st.hi = p.row_hi[lb * p.Lq + row];
        } else {
            row_interval(p.mask, b, row, st.lo, st.hi);
        }
    }
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
        st.m_l2 = st.m_fixed * kLog2e;
    }
    st.scale_l2 = p.scale * kLog2e;

    const Walk walk = make_walk<C::TILE, C::NT>(p, b, qb, st.lo, st.hi, row_ok, red);
    if (MODE == MODE_GATED) {
        if (fixed) bf16_run<D, NW, BODY_FIXED, OUT>(p, st, walk, lds, b, h, row);
        else bf16_run<D, NW, BODY_ONLINE, OUT>(p, st, walk, lds, b, h, row);
    } else {
        bf16_run<D, NW, MODE, OUT>(p, st, walk, lds, b, h, row);
    }
}

// ---------------------------------------------------------------------------
// fp32 kernel: 32-key tiles, 32x32x2 fp32 MFMA, no reduced-precision step.
// ---------------------------------------------------------------------------
template <int D, int BODY, int OUT>
__device__ inline void f32_run(const AttnLaunch& p, const Walk& walk, float* ks, float* vs, const float (&qf)[D / 2],
                               int lo, int hi, float m_fixed, i64 b, i64 h, i64 row) {
    constexpr int TILE = 32, NDB = D / 32, LD = D + 1;
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hb = lane >> 5;
    const float scale_l2 = p.scale * kLog2e, m_l2 = m_fixed * kLog2e;
    f32x16 acc[NDB];
#pragma unroll
    for (int d = 0; d < NDB; ++d) acc[d] = f32x16{};
    float m_run = kNegInf, l_run = 0.0f;
    const float* kbase = (const float*)p.k + b * p.k_sB + h * p.k_sH;
    const float* vbase = (const float*)p.v + b * p.v_sB + h * p.v_sH;
    const int kv_lim = (int)p.mask.kv_valid;
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
        if (cur.masked(walk.Lk)) apply_mask<1>(s, j0, lo, hi);
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

template <int D, int MODE, int OUT>
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
    const Walk walk = make_walk<TILE, 256>(p, b, qb, lo, hi, row_ok, red);
    if (fixed) f32_run<D, BODY_FIXED, OUT>(p, walk, ks, vs, qf, lo, hi, m_fixed, b, h, row);
    else f32_run<D, BODY_ONLINE, OUT>(p, walk, ks, vs, qf, lo, hi, m_fixed, b, h, row);
}

template <int D, int MODE, int OUT>
hipError_t launch_one(const AttnLaunch& a, hipStream_t stream) {
    const i64 grid = a.n_qblocks * (i64)a.B * a.H;
    if (grid == 0) return hipSuccess;
    if (a.in_dtype == BWA_BF16) {
        constexpr int NW = D == 128 ? 8 : 4;
        hipLaunchKernelGGL((attn_fwd_bf16<D, NW, MODE, OUT>), dim3((unsigned)grid), dim3(NW * 64), 0, stream, a);
    } else {
        hipLaunchKernelGGL((attn_fwd_f32<D, MODE, OUT>), dim3((unsigned)grid), dim3(256), 0, stream, a);
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

int attn_rows_per_block(int dtype, int D) { return (dtype == BWA_BF16 && D == 128) ? 256 : 128; }

hipError_t launch_attn_fwd(const AttnLaunch& a, hipStream_t stream) {
    if (a.D == 64) return launch_d<64>(a, stream);
    return launch_d<128>(a, stream);
}

}  // namespace bwa
