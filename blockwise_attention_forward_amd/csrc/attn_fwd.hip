// Blockwise attention forward for gfx950 (MI355X).
//
// One workgroup of 4 wavefronts handles 128 query rows of one (batch, head);
// each wavefront owns 32 rows.  Keys are walked in tiles of 64 (bf16) or 32
// (fp32) in ascending order, tile by tile over the run list of the query
// block: FULL tiles run an unmasked body, PARTIAL tiles (and the ragged last
// tile) compare every key with the row's visible interval.  This is the
// forward analogue of the partial/full tile lists of "Add more optimal dk
// order optional arg" (flash-attention pull request 2512, "Sliding window
// perf issue"), walked as one ordered list ("A simplish fix").
//
// Scores are computed transposed, S^T = K Q^T, on the 32x32x16 bf16 matrix
// cores so that each lane ends up holding one query row's scores: the row
// max and row sum are in-lane reductions plus one exchange with the lane
// 32 apart.  The probabilities then feed O^T = V^T P^T straight from the
// registers the scores came out in.  V is staged transposed in LDS (a 4x8
// register transpose per thread while storing), K row-major; both use an XOR
// swizzle of 16-byte chunks so that the matrix-core operand reads of a wave
// hit distinct banks.  Tiles are double-buffered: the global loads of the
// next tile are in flight while the current tile is computed.
//
// Softmax bodies ("Fixed-m softmax for 2D-ring x Ulysses attention (WAN 2.2)",
// description):
//   online : running row max m, p = exp(s*scale - m*scale), l and O rescaled
//            by exp((m_old - m_new)*scale) whenever the max moves;
//   fixed-m: p = exp(s*scale - m_i) with the caller's per-row bound m_i; no
//            max, no rescale.  Each is its own specialisation (one branch-free
//            body per launch; the Notes of that page measured a 3x loss when
//            two bodies share a kernel's hot loop).
// Exponentials use the hardware base-2 exponential with log2(e) folded into
// the scale; LSE is returned in natural-log units.

#include "internal.h"

namespace bwa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBQ = 128;  // query rows per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

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

// ---------------------------------------------------------------------------
// Tile walk: runs of key ranges [kb, ke) of one kind, visited tile by tile.
// ---------------------------------------------------------------------------
struct RunWalk {
    // list mode
    const int* rb; const int* re; const uint8_t* rk;
    i64 r0, nruns;
    int bkv_list;
    // inline mode (3 runs: partial, full, partial)
    int ib[3], ie[3], ik[3];
    bool inline_mode;
    int Lk;

    __device__ inline void get(i64 r, int& kb, int& ke, int& kind) const {
        if (inline_mode) {
            kb = ib[r]; ke = ie[r]; kind = ik[r];
        } else {
            const i64 i = r0 + r;
            kb = rb[i] * bkv_list;
            ke = min(re[i] * bkv_list, Lk);
            kind = rk[i];
        }
    }
};

template <int TILE>
struct Cursor {
    i64 r;
    int j0, ke, kind;
    bool valid;

    __device__ inline void seek(const RunWalk& w, i64 start) {
        for (r = start; r < w.nruns; ++r) {
            int kb;
            w.get(r, kb, ke, kind);
            if (kb < ke) { j0 = kb; valid = true; return; }
        }
        valid = false;
    }
    __device__ inline void first(const RunWalk& w) { seek(w, 0); }
    __device__ inline void next(const RunWalk& w) {
        j0 += TILE;
        if (j0 < ke) return;
        seek(w, r + 1);
    }
    __device__ inline bool masked(int Lk) const {
        return kind != BWA_TILE_FULL || j0 + TILE > Lk;
    }
};

// Workgroup-wide reductions of 4 ints over 256 threads (inline tile walk).
__device__ inline void wg_reduce4(int& mn_lo, int& mx_hi, int& mx_lo, int& mn_hi, int* red) {
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
    for (int i = 1; i < 4; ++i) {
        mn_lo = min(mn_lo, red[i * 4 + 0]); mx_hi = max(mx_hi, red[i * 4 + 1]);
        mx_lo = max(mx_lo, red[i * 4 + 2]); mn_hi = min(mn_hi, red[i * 4 + 3]);
    }
    __syncthreads();
    mn_lo = __builtin_amdgcn_readfirstlane(mn_lo);
    mx_hi = __builtin_amdgcn_readfirstlane(mx_hi);
    mx_lo = __builtin_amdgcn_readfirstlane(mx_lo);
    mn_hi = __builtin_amdgcn_readfirstlane(mn_hi);
}

// Set up the walk for query block qb.  lo/hi: this lane's row interval;
// row_exists: row < Lq.  Inline runs are aligned to TILE.
template <int TILE>
__device__ inline void make_walk(const AttnLaunch& p, i64 b, i64 qb, int lo, int hi,
                                 bool row_exists, RunWalk& w, int* red) {
    w.Lk = (int)p.Lk;
    w.inline_mode = !p.have_blocks;
    if (p.have_blocks) {
        const i64 lb = p.list_batch == 1 ? 0 : b;
        const i64* rp = p.row_ptr + lb * (p.n_qblocks + 1);
        i64 r0 = min(rp[qb], p.capacity), r1 = min(rp[qb + 1], p.capacity);
        w.rb = p.run_begin + lb * p.capacity;
        w.re = p.run_end + lb * p.capacity;
        w.rk = p.run_kind + lb * p.capacity;
        w.r0 = r0;
        w.nruns = max(r1 - r0, (i64)0);
        w.bkv_list = p.bkv_list;
        return;
    }
    // Inline: rows' intervals are monotone in the row index for every mask
    // this library describes, so the union of the block's intervals is
    // covered by [min lo, max hi) and the tiles inside [max lo, min hi) are
    // full.  Visiting a tile that holds no visible pair is harmless (it is
    // masked), so this walk is correct for any interval mask.
    const bool ne = row_exists && lo < hi;
    int mn_lo = ne ? lo : 0x7fffffff, mx_hi = ne ? hi : 0;
    int mx_lo = row_exists ? (ne ? lo : 0x7fffffff) : 0;
    int mn_hi = row_exists ? (ne ? hi : -1) : 0x7fffffff;
    wg_reduce4(mn_lo, mx_hi, mx_lo, mn_hi, red);
    w.nruns = 3;
    w.ik[0] = BWA_TILE_PARTIAL; w.ik[1] = BWA_TILE_FULL; w.ik[2] = BWA_TILE_PARTIAL;
    for (int i = 0; i < 3; ++i) w.ib[i] = w.ie[i] = 0;
    if (mx_hi == 0) return;  // no row of this block sees anything
    const int t0 = (mn_lo / TILE) * TILE;  // tiles j0 = t0, t0 + TILE, ... < t1
    const int t1 = mx_hi;
    // Full tiles need every existing row non-empty (mx_lo/mn_hi carry a
    // sentinel otherwise) and j0 >= max lo, j0 + TILE <= min hi.
    const bool all_rows = mx_lo != 0x7fffffff && mn_hi >= 0;
    const int f0 = all_rows ? ((mx_lo + TILE - 1) / TILE) * TILE : 0;
    const int f1 = all_rows ? (mn_hi / TILE) * TILE : 0;
    if (!all_rows || f0 >= f1) {
        w.ib[0] = t0; w.ie[0] = t1;  // one partial run
        return;
    }
    w.ib[0] = t0; w.ie[0] = f0;
    w.ib[1] = f0; w.ie[1] = f1;
    w.ib[2] = f1; w.ie[2] = t1;
}

// ---------------------------------------------------------------------------
// Softmax pieces on the 32x32 accumulator layout: lane l holds column
// (query) l%32 and rows (keys) 8*(r/4) + (l/32)*4 + r%4, r = 0..15.
// ---------------------------------------------------------------------------
template <int NKB>
__device__ inline void apply_mask(f32x16 (&s)[NKB], int j0, int lo, int hi) {
    const int hb = (threadIdx.x >> 5) & 1;
    const int lo_rel = lo - (j0 + hb * 4), hi_rel = hi - (j0 + hb * 4);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
            s[kb][r] = (off >= lo_rel && off < hi_rel) ? s[kb][r] : kNegInf;
        }
}

template <int NKB, int NDB>
__device__ inline void online_update(f32x16 (&s)[NKB], f32x16 (&acc)[NDB], float& m_run,
                                     float& l_run, float scale_l2) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
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
#pragma unroll
    for (int d = 0; d < NDB; ++d) acc[d] *= alpha;
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
template <int D, int OUT, int MODE>
__device__ inline void store_out(const AttnLaunch& p, f32x16 (&acc)[D / 32], float m_run,
                                 float l_run, float m_fixed, i64 b, i64 h, i64 row) {
    const int hb = (threadIdx.x >> 5) & 1;
    const float l = l_run + __shfl_xor(l_run, 32);
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
        if (any) lse = (MODE == BWA_MODE_FIXED_M ? m_fixed : m_run * p.scale) + __logf(l);
        p.lse[(b * p.H + h) * p.Lq + row] = lse;
    }
}

// ---------------------------------------------------------------------------
// bf16 kernel: 64-key tiles, 32x32x16 bf16 MFMA.
// ---------------------------------------------------------------------------
template <int D, int MODE, int OUT>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16(const AttnLaunch p) {
    constexpr int TILE = 64;
    constexpr int NCH = D / 8;    // 16-byte chunks per K row
    constexpr int NDB = D / 32;   // 32-wide d blocks of O^T
    constexpr int NDS = D / 16;   // 16-deep steps of Q K^T
    constexpr int KL = TILE * NCH / 256;  // K chunks loaded per thread
    constexpr int TILE_BYTES = TILE * D * 2;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][TILE_BYTES];
    __shared__ int red[16];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hb = lane >> 5;
    const i64 logical = xcd_remap(blockIdx.x, gridDim.x);
    const i64 bh = logical / p.n_qblocks;
    const i64 qb = p.n_qblocks - 1 - (logical % p.n_qblocks);
    const i64 b = bh / p.H, h = bh % p.H;
    if (p.gate) {
        const bool g = p.gate[bh] != 0;
        if (g != (MODE == BWA_MODE_FIXED_M)) return;
    }

    const i64 row = qb * kBQ + wave * 32 + l32;
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

    // Q^T operand fragments: lane holds Q[row][ds*16 + hb*8 + 0..7].
    const __bf16* qp = (const __bf16*)p.q + b * p.q_sB + row * p.q_sL + h * p.q_sH;
    uint4 qf[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
        qf[ds] = row_ok ? *(const uint4*)(qp + ds * 16 + hb * 8) : uint4{0, 0, 0, 0};

    float m_fixed = 0.0f, m_l2 = 0.0f;
    if (MODE == BWA_MODE_FIXED_M && row_ok) {
        m_fixed = p.m[bh * p.Lq + row];
        m_l2 = m_fixed * kLog2e;
    }
    const float scale_l2 = p.scale * kLog2e;

    RunWalk walk;
    make_walk<TILE>(p, b, qb, lo, hi, row_ok, walk, red);

    f32x16 acc[NDB];
#pragma unroll
    for (int d = 0; d < NDB; ++d) acc[d] = f32x16{};
    float m_run = kNegInf, l_run = 0.0f;

    const __bf16* kbase = (const __bf16*)p.k + b * p.k_sB + h * p.k_sH;
    const __bf16* vbase = (const __bf16*)p.v + b * p.v_sB + h * p.v_sH;
    const int kv_lim = (int)p.mask.kv_valid;

    // Global -> registers for one tile.
    uint4 sk[KL], sv[4];
    auto load_tile = [&](int j0) {
#pragma unroll
        for (int it = 0; it < KL; ++it) {
            const int lin = it * 256 + tid, r = lin / NCH, c = lin % NCH;
            const int j = j0 + r;
            sk[it] = (j < kv_lim) ? *(const uint4*)(kbase + (i64)j * p.k_sL + c * 8) : uint4{0, 0, 0, 0};
        }
        const int g = tid / NCH, cd = tid % NCH;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = j0 + 4 * g + e;
            sv[e] = (g < 16 && j < kv_lim) ? *(const uint4*)(vbase + (i64)j * p.v_sL + cd * 8)
                                          : uint4{0, 0, 0, 0};
        }
    };
    // Registers -> LDS (K row-major swizzled; V transposed, key-permuted, swizzled).
    auto store_tile = [&](int buf) {
        uint8_t* kl = lds[buf][0];
        uint8_t* vl = lds[buf][1];
#pragma unroll
        for (int it = 0; it < KL; ++it) {
            const int lin = it * 256 + tid, r = lin / NCH, c = lin % NCH;
            *(uint4*)(kl + r * (D * 2) + ((c ^ (r & (NCH - 1))) * 16)) = sk[it];
        }
        const int g = tid / NCH, cd = tid % NCH;
        if (g < 16) {
            const int chunk = (g >> 2) * 2 + (g & 1), half = (g >> 1) & 1;
            const uint32_t* w0 = (const uint32_t*)&sv[0];
            const uint32_t* w1 = (const uint32_t*)&sv[1];
            const uint32_t* w2 = (const uint32_t*)&sv[2];
            const uint32_t* w3 = (const uint32_t*)&sv[3];
#pragma unroll
            for (int wi = 0; wi < 4; ++wi)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int d = cd * 8 + wi * 2 + s;
                    uint2 val;
                    if (s == 0) {
                        val.x = (w0[wi] & 0xffffu) | (w1[wi] << 16);
                        val.y = (w2[wi] & 0xffffu) | (w3[wi] << 16);
                    } else {
                        val.x = (w0[wi] >> 16) | (w1[wi] & 0xffff0000u);
                        val.y = (w2[wi] >> 16) | (w3[wi] & 0xffff0000u);
                    }
                    const int cs = chunk ^ ((d ^ (d >> 3)) & 7);
                    *(uint2*)(vl + d * (TILE * 2) + cs * 16 + half * 8) = val;
                }
        }
    };
    auto compute_tile = [&](int buf, int j0, bool masked) {
        const uint8_t* kl = lds[buf][0];
        const uint8_t* vl = lds[buf][1];
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int r = kb * 32 + l32, c = ds * 2 + hb;
                const uint4 a = *(const uint4*)(kl + r * (D * 2) + ((c ^ (r & (NCH - 1))) * 16));
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[ds]), s[kb], 0, 0, 0);
            }
        }
        if (masked) apply_mask<2>(s, j0, lo, hi);
        if (MODE == BWA_MODE_FIXED_M) fixed_update<2>(s, l_run, scale_l2, m_l2);
        else online_update<2, NDB>(s, acc, m_run, l_run, scale_l2);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int kb = kk >> 1, r0 = 8 * (kk & 1);
            uint4 pb;
            pb.x = pack_bf16x2(s[kb][r0 + 0], s[kb][r0 + 1]);
            pb.y = pack_bf16x2(s[kb][r0 + 2], s[kb][r0 + 3]);
            pb.z = pack_bf16x2(s[kb][r0 + 4], s[kb][r0 + 5]);
            pb.w = pack_bf16x2(s[kb][r0 + 6], s[kb][r0 + 7]);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int d = db * 32 + l32, c = kk * 2 + hb;
                const uint4 a = *(const uint4*)(vl + d * (TILE * 2) + ((c ^ ((d ^ (d >> 3)) & 7)) * 16));
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, pb), acc[db], 0, 0, 0);
            }
        }
    };

    Cursor<TILE> cur;
    cur.first(walk);
    if (cur.valid) {
        load_tile(cur.j0);
        store_tile(0);
        __syncthreads();
        int buf = 0;
        while (true) {
            Cursor<TILE> nxt = cur;
            nxt.next(walk);
            if (nxt.valid) load_tile(nxt.j0);
            compute_tile(buf, cur.j0, cur.masked(walk.Lk));
            if (!nxt.valid) break;
            store_tile(buf ^ 1);
            __syncthreads();
            buf ^= 1;
            cur = nxt;
        }
    }
    store_out<D, OUT, MODE>(p, acc, m_run, l_run, m_fixed, b, h, row);
}

// ---------------------------------------------------------------------------
// fp32 kernel: 32-key tiles, 32x32x2 fp32 MFMA, no reduced-precision step.
// ---------------------------------------------------------------------------
template <int D, int MODE, int OUT>
__global__ __launch_bounds__(256, 1) void attn_fwd_f32(const AttnLaunch p) {
    constexpr int TILE = 32;
    constexpr int NDB = D / 32;
    constexpr int LD = D + 1;  // padded row stride (floats): conflict-free column reads
    __shared__ float ks[TILE * LD];
    __shared__ float vs[TILE * LD];
    __shared__ int red[16];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hb = lane >> 5;
    const i64 logical = xcd_remap(blockIdx.x, gridDim.x);
    const i64 bh = logical / p.n_qblocks;
    const i64 qb = p.n_qblocks - 1 - (logical % p.n_qblocks);
    const i64 b = bh / p.H, h = bh % p.H;
    if (p.gate) {
        const bool g = p.gate[bh] != 0;
        if (g != (MODE == BWA_MODE_FIXED_M)) return;
    }
    const i64 row = qb * kBQ + wave * 32 + l32;
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

    float m_fixed = 0.0f, m_l2 = 0.0f;
    if (MODE == BWA_MODE_FIXED_M && row_ok) {
        m_fixed = p.m[bh * p.Lq + row];
        m_l2 = m_fixed * kLog2e;
    }
    const float scale_l2 = p.scale * kLog2e;

    RunWalk walk;
    make_walk<TILE>(p, b, qb, lo, hi, row_ok, walk, red);

    f32x16 acc[NDB];
#pragma unroll
    for (int d = 0; d < NDB; ++d) acc[d] = f32x16{};
    float m_run = kNegInf, l_run = 0.0f;

    const float* kbase = (const float*)p.k + b * p.k_sB + h * p.k_sH;
    const float* vbase = (const float*)p.v + b * p.v_sB + h * p.v_sH;
    const int kv_lim = (int)p.mask.kv_valid;

    Cursor<TILE> cur;
    for (cur.first(walk); cur.valid; cur.next(walk)) {
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
        if (MODE == BWA_MODE_FIXED_M) fixed_update<1>(s, l_run, scale_l2, m_l2);
        else online_update<1, NDB>(s, acc, m_run, l_run, scale_l2);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int key = 8 * (t >> 2) + hb * 4 + (t & 3);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * LD + db * 32 + l32], s[0][t],
                                                               acc[db], 0, 0, 0);
        }
    }
    store_out<D, OUT, MODE>(p, acc, m_run, l_run, m_fixed, b, h, row);
}

template <int D, int MODE, int OUT>
hipError_t launch_one(const AttnLaunch& a, hipStream_t stream) {
    const i64 grid = a.n_qblocks * (i64)a.B * a.H;
    if (grid == 0) return hipSuccess;
    if (a.in_dtype == BWA_BF16)
        hipLaunchKernelGGL((attn_fwd_bf16<D, MODE, OUT>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((attn_fwd_f32<D, MODE, OUT>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnLaunch& a, hipStream_t stream) {
    if (a.mode == BWA_MODE_FIXED_M) {
        return a.out_dtype == BWA_F32 ? launch_one<D, BWA_MODE_FIXED_M, BWA_F32>(a, stream)
                                      : launch_one<D, BWA_MODE_FIXED_M, BWA_BF16>(a, stream);
    }
    return a.out_dtype == BWA_F32 ? launch_one<D, BWA_MODE_ONLINE, BWA_F32>(a, stream)
                                  : launch_one<D, BWA_MODE_ONLINE, BWA_BF16>(a, stream);
}

}  // namespace

hipError_t launch_attn_fwd(const AttnLaunch& a, hipStream_t stream) {
    if (a.D == 64) return launch_d<64>(a, stream);
    return launch_d<128>(a, stream);
}

}  // namespace bwa
