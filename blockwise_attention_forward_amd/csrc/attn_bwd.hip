// Blockwise attention backward for gfx950 (MI355X).
//
// "Add more optimal dk order optional arg" (flash-attention pull request
// 2512, description and "Sliding window perf issue") describes the backward
// pass of block-sparse attention: a program per key column computes that
// column's dK and dV over the query blocks that meet it, and each query
// block's dQ collects one contribution per key column, added in an order
// the caller may choose (ascending, descending or any permutation of the
// columns); a fixed order makes dQ repeat bit for bit.  There the key-column
// programs add into a shared dQ and wait on per-block semaphores for their
// turn.  Here no workgroup ever waits for another (gfx950 deals workgroups
// to its 8 XCDs round-robin, and a spin wait on a workgroup that has not
// been dispatched never ends):
//   * dK/dV: one workgroup per (batch, key/value head, 128-key block); it
//     walks the query tiles that meet its keys (all query heads of a
//     grouped-query head, in order) and writes dK and dV once.
//   * dQ: one workgroup per (batch, head, 256-row block); it walks the key
//     tiles of its rows in the chosen order and writes dQ once.
// Both run 8 waves, two per SIMD, so that one wave's element-wise work and
// LDS waits hide under the other's matrix products.
// The score and probability tiles are computed in both kernels (two extra
// matrix products over a pass that adds into dQ from the key-column
// programs); in exchange every output is written exactly once, no atomics
// and no waits, and the result is deterministic by construction.
//
// With P = exp(scale * Q K^T - LSE) (the forward's LSE, natural log), the
// gradients of the loss sum_i dO_i . O_i are
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - delta),  delta_i = dO_i . O_i,
//   dQ = scale * dS K,  dK = scale * dS^T Q.
// Matrix products run on the 32x32x16 bf16 matrix cores with fp32
// accumulation; P and dS are rounded to bf16 as operands.  Tiles are staged
// through registers into LDS, each tile's loads issued a tile or two before
// it is used, in an XOR swizzle of 16-byte chunks that serves both ways each
// tile is read: row by row (an operand whose rows are the tile's rows) and
// transposed (the LDS transpose read, an operand whose rows are the tile's
// columns); each read hits distinct banks.  Per-row key intervals decide which tiles are
// skipped, run unmasked (every pair visible) or compare key by key, as in
// the forward pass.

#include <utility>

#include "internal.h"

namespace bwa {
namespace {

// f(integral_constant<int, i>) for i = 0 .. N-1, each i a compile-time
// constant in the body (array indices stay registers).
template <class F, int... I>
__device__ __attribute__((always_inline)) inline void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBig = 0x7fffffff;
constexpr int kKeyBlock = 128;  // keys per dK/dV workgroup (32 per wave)
constexpr int kDqWaves = 8;     // waves per dQ workgroup (32 rows each, two per SIMD)
constexpr int kTile = 64;       // rows of a streamed Q/dO tile, keys of a streamed K/V tile
constexpr int kRing = 3;        // tile buffers in LDS
constexpr int kAhead = 4;       // LDS operand reads run this many matrix-core steps ahead (4-wave dK/dV)

__device__ inline i64 xcd_remap(i64 id, i64 n) {
    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
    // contiguous range of logical work, so that neighbouring blocks of one
    // head share that XCD's L2 while they stream the same tiles.
    const i64 q = n >> 3, r = n & 7, x = id & 7, slot = id >> 3;
    return (x < r) ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Wait for every vector-memory load of this wave.  Placed after a kernel's
// prologue loads, it settles them once: without it the loop's first use of
// those registers waits, every iteration, on the tile loads in flight (the
// wait counters of the prologue and of the loop's back edge merge at the
// loop head).
__device__ inline void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Load of wave-uniform data that no work-item writes while the kernel runs
// (the plan arrays, written by earlier launches): through the constant
// address space it becomes a scalar load, with no wait on the vector loads
// in flight.
template <class T>
__device__ inline T ld_const(const T* p, i64 i) {
    return ((const __attribute__((address_space(4))) T*)p)[i];
}

template <int D>
struct Cfg {
    static constexpr int NCH = D / 8;                // 16-byte chunks per row
    static constexpr int NDS = D / 16;               // 16-deep steps over d
    static constexpr int NDB = D / 32;               // 32-wide d blocks
    static constexpr int TILE_BYTES = kTile * D * 2;
};

// Swizzle of 16-byte chunk c of tile row r.  A 256-byte bank window holds
// one row (D = 128) or two rows (D = 64).  A row-wise operand read touches 16
// consecutive rows at one chunk; a transposed read touches 4 consecutive
// rows (aligned to 4) at 4 consecutive chunks (aligned to 4).  The XOR value
// takes 16 distinct values over any 16 consecutive rows (first read), and
// over 4 aligned rows it moves the aligned group of 4 chunks to 4 different
// groups (second read), so neither read has a bank conflict.
template <int D>
__device__ inline int bswz(int r, int c) {
    return D == 128 ? c ^ (((r & 3) << 2) | ((r >> 2) & 3)) : c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// A 64-row tile staged through registers: each of NT work-items loads 8D/NT
// chunks of 16 bytes (chunk id = it*NT + tid: row id / NCH, chunk id % NCH,
// so a row's chunks come from consecutive lanes), then stores each at its
// swizzled place in LDS.  Rows at or past `nvalid` are zeros.
template <int D, int NT = 256>
struct Staged {
    uint4 c[8 * D / NT];
};

template <int D, int NT = 256>
__device__ inline void stage_load(Staged<D, NT>& x, const __bf16* base, i64 sL, int nvalid) {
    constexpr int NCH = Cfg<D>::NCH;
#pragma unroll
    for (int it = 0; it < 8 * D / NT; ++it) {
        const int id = it * NT + (int)threadIdx.x, r = id / NCH, c = id % NCH;
        x.c[it] = r < nvalid ? *(const uint4*)(base + (i64)r * sL + c * 8) : uint4{0, 0, 0, 0};
    }
}

template <int D, int NT = 256>
__device__ inline void stage_store(const Staged<D, NT>& x, uint8_t* t) {
    constexpr int NCH = Cfg<D>::NCH;
#pragma unroll
    for (int it = 0; it < 8 * D / NT; ++it) {
        const int id = it * NT + (int)threadIdx.x, r = id / NCH, c = id % NCH;
        *(uint4*)(t + r * (D * 2) + bswz<D>(r, c) * 16) = x.c[it];
    }
}

// Operand fragment whose rows are tile rows rb*32 + l32 (16-deep step ds over
// d: the lane holds d = ds*16 + hb*8 + 0..7).
template <int D>
__device__ inline uint4 frag_rows(const uint8_t* t, int rb, int ds) {
    const int lane = threadIdx.x & 63, l32 = lane & 31, hb = lane >> 5;
    const int r = rb * 32 + l32;
    return *(const uint4*)(t + r * (D * 2) + bswz<D>(r, ds * 2 + hb) * 16);
}

// Operand fragment whose rows are tile columns d = db*32 + l32, over the 16
// tile rows of step kk in the order kk*16 + {hb*4 + 0..3, 8 + hb*4 + 0..3}
// (the order in which a 32x32 result tile holds its rows in a lane).  Two
// transposing 64-bit LDS reads: in each group of 16 lanes, lane i receives
// element i%4 of the 4-element rows addressed by lanes i/4 + 4s (s = 0..3),
// so lane 16g + 4s + u points at row base + s, columns db*32 + 16*(g&1) + 4u.
template <int D>
__device__ inline uint4 frag_cols(const uint8_t* t, int kk, int db) {
    const int lane = threadIdx.x & 63, hb = lane >> 5;
    const int g1 = (lane >> 4) & 1, s_row = (lane >> 2) & 3, u = lane & 3;
    const int c = db * 4 + g1 * 2 + (u >> 1);
    const int r0 = kk * 16 + hb * 4 + s_row, r1 = r0 + 8;
    const s16x4 x0 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + r0 * (D * 2) + bswz<D>(r0, c) * 16 + (u & 1) * 8));
    const s16x4 x1 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + r1 * (D * 2) + bswz<D>(r1, c) * 16 + (u & 1) * 8));
    uint4 out;
    out.x = __builtin_bit_cast(uint2, x0).x;
    out.y = __builtin_bit_cast(uint2, x0).y;
    out.z = __builtin_bit_cast(uint2, x1).x;
    out.w = __builtin_bit_cast(uint2, x1).y;
    return out;
}

// Keeps x where it is computed: with a masked select as its only user the
// compiler would otherwise move the arithmetic that produces it into a
// per-lane branch around the select (a branch and exec-mask updates per
// element) instead of selecting.
__device__ __attribute__((always_inline)) inline float pin(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

__device__ inline f32x16 mfma(const uint4& a, const uint4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

// Dilated band, as a bit mask over 32 consecutive positions: bit o is set
// when position base + o is congruent to res modulo g (pat holds the bits
// 0, g, 2g, ... below 32; base >= 0).  One modulo per 32 positions instead
// of one per element.
__device__ inline unsigned dil_bits(int res, int base, int g, unsigned pat) {
    const int m = ((res - base % g) % g + g) % g;
    return m < 32 ? (pat << m) : 0u;
}

__device__ inline unsigned dil_pattern(int g) {
    unsigned pat = 0u;
    for (int o = 0; o < 32; o += g) pat |= 1u << o;
    return pat;
}

// Document ids of keys j .. j+7 (j the same in every lane; clamped to the
// last key): scalar loads, so nothing waits behind the tile loads in flight.
__device__ inline void key_ids8(const BwdLaunch& p, i64 b, int j, int (&id)[8]) {
    const int* kid = p.mask.ids_kv + b * p.mask.lk;
    const int last = (int)p.mask.lk - 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) id[i] = ld_const(kid, min(j + i, last));
}

__device__ inline int wave_min(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o));
    return x;
}
__device__ inline int wave_max(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
    return x;
}

// Store 16 values of a 32x32 result tile held as C[d][n] (n = this lane's
// row or key): d = db*32 + 8*g + 4*hb + 0..3 for g = 0..3.
template <int G>
__device__ inline void store_tile(void* row_ptr, const f32x16& acc, int db, float mul) {
    const int hb = (threadIdx.x >> 5) & 1;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + hb * 4;
        const float a = acc[4 * g] * mul, b = acc[4 * g + 1] * mul, c = acc[4 * g + 2] * mul,
                    e = acc[4 * g + 3] * mul;
        if (G == BWA_F32) {
            *(f32x4*)((float*)row_ptr + d) = f32x4{a, b, c, e};
        } else {
            *(uint2*)((__bf16*)row_ptr + d) = uint2{pack_bf16x2(a, b), pack_bf16x2(c, e)};
        }
    }
}

// ---------------------------------------------------------------------------
// Planning: per-row key intervals, per-query-tile summaries, and for every
// key block the range of query tiles that meet it.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_rows_kernel(const BwdLaunch p) {
    const i64 idx = (i64)blockIdx.x * 256 + threadIdx.x;
    if (idx < p.list_batch * p.Lq) {
        const i64 b = idx / p.Lq, i = idx % p.Lq;
        int lo, hi;
        row_interval(p.mask, b, i, lo, hi);
        p.row_lo[idx] = lo;
        p.row_hi[idx] = hi;
    }
    if (idx < p.list_batch * p.nkb) {
        p.kfirst[idx] = kBig;
        p.klast[idx] = -1;
    }
}

// One wave per 64-row query tile: the envelope [env_lo, env_hi) of its rows'
// intervals (rows that see nothing left out), the part [full_lo, full_hi)
// every row sees (empty as soon as one row sees nothing), and the tile's
// index folded into the range of every key block the envelope meets.
__global__ __launch_bounds__(64) void bwd_qtiles_kernel(const BwdLaunch p) {
    const i64 t = blockIdx.x;  // over list_batch * nqt
    const i64 lb = t / p.nqt, m = t % p.nqt;
    const int lane = threadIdx.x;
    const i64 row = m * kTile + lane;
    int lo = 0, hi = 0;
    if (row < p.Lq) {
        lo = p.row_lo[lb * p.Lq + row];
        hi = p.row_hi[lb * p.Lq + row];
    }
    const bool ne = lo < hi;
    const int env_lo = wave_min(ne ? lo : kBig), env_hi = wave_max(ne ? hi : 0);
    const int full_lo = wave_max(ne ? lo : kBig), full_hi = wave_min(ne ? hi : -1);
    if (lane == 0) p.qsum[t] = int4{env_lo, env_hi, full_lo, full_hi};
    if (env_lo < env_hi) {
        const int n0 = env_lo / kKeyBlock, n1 = (env_hi - 1) / kKeyBlock;
        for (int n = n0 + lane; n <= n1; n += 64) {
            atomicMin(&p.kfirst[lb * p.nkb + n], (int)m);
            atomicMax(&p.klast[lb * p.nkb + n], (int)m);
        }
    }
}

// delta[b,h,i] = dO_i . O_i in fp32: D/8 lanes per row, 8 elements each.
template <int D, int ODT>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const BwdLaunch p) {
    constexpr int TPR = D / 8;
    const i64 r = ((i64)blockIdx.x * 256 + threadIdx.x) / TPR;  // row (b, i, h), h fastest
    const int c = (threadIdx.x % TPR) * 8;
    const i64 n = (i64)p.B * p.Lq * p.H;
    float s = 0.0f;
    const i64 h = r % p.H, bi = r / p.H, i = bi % p.Lq, b = bi / p.Lq;
    if (r < n) {
        const uint4 g = *(const uint4*)((const __bf16*)p.dout + b * p.do_sB + i * p.do_sL + h * p.do_sH + c);
        const bf16x8 gv = __builtin_bit_cast(bf16x8, g);
        float ov[8];
        if (ODT == BWA_F32) {
            const float* op = (const float*)p.o + b * p.o_sB + i * p.o_sL + h * p.o_sH + c;
            const f32x4 a = *(const f32x4*)op, e = *(const f32x4*)(op + 4);
#pragma unroll
            for (int t = 0; t < 4; ++t) { ov[t] = a[t]; ov[4 + t] = e[t]; }
        } else {
            const bf16x8 a =
                __builtin_bit_cast(bf16x8, *(const uint4*)((const __bf16*)p.o + b * p.o_sB + i * p.o_sL + h * p.o_sH + c));
#pragma unroll
            for (int t = 0; t < 8; ++t) ov[t] = (float)a[t];
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) s = __builtin_fmaf((float)gv[t], ov[t], s);
    }
#pragma unroll
    for (int o = TPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (r < n && (threadIdx.x % TPR) == 0) p.delta[(b * p.H + h) * p.Lq + i] = s;
}

struct QCursor {
    int g, m;  // query head within the group, query tile
};

// Next (g, m) after c whose rows' envelope meets keys [k0, k1).
__device__ inline bool q_next(const BwdLaunch& p, QCursor& c, i64 lb, int m0, int m1, int k0, int k1) {
    for (;;) {
        if (++c.m > m1) {
            c.m = m0;
            if (++c.g >= p.kv_group) return false;
        }
        const i32x4 s = ld_const((const i32x4*)p.qsum, lb * p.nqt + c.m);
        if (s[0] < k1 && s[1] > k0) return true;
    }
}

// ---------------------------------------------------------------------------
// dK / dV with two waves per SIMD: 8 waves = 4 key groups of 32 keys x 2 row
// halves.  The workgroup's 128 keys of K and V sit in LDS (a wave's share of
// 256 registers does not hold K, V and both accumulators); wave (kg, rh)
// computes rows rh*32 .. rh*32+31 of every 64-row query tile against keys
// kg*32 .. kg*32+31, and the two waves of a key group add their partial dK
// and dV through LDS at the end (rh 0 + rh 1, a fixed order).  Query tiles
// go through two LDS buffers, each tile's loads issued one tile ahead.
// ---------------------------------------------------------------------------
template <int D>
struct KvStage8 {
    Staged<D, 512> q, g;
    float st;  // work-items 0..255: LSE, delta, lo, hi of row tid % 64
};

template <int D>
__device__ inline void kv_load8(const BwdLaunch& p, KvStage8<D>& x, const QCursor& c, i64 b, i64 hk, i64 lb) {
    const i64 h = hk * p.kv_group + c.g;
    const i64 r0 = (i64)c.m * kTile;
    const int nq = (int)min((i64)kTile, p.mask.q_valid - r0);
    stage_load<D, 512>(x.q, (const __bf16*)p.q + b * p.q_sB + r0 * p.q_sL + h * p.q_sH, p.q_sL, nq);
    stage_load<D, 512>(x.g, (const __bf16*)p.dout + b * p.do_sB + r0 * p.do_sL + h * p.do_sH, p.do_sL, nq);
    const int wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const i64 row = r0 + lane;
    const i64 li = (b * p.H + h) * p.Lq + row;
    float v = 0.0f;
    if (row < p.Lq) {
        if (wave == 0) v = p.lse[li];
        else if (wave == 1) v = p.delta[li];
        else if (wave == 2) v = __int_as_float(p.row_lo[lb * p.Lq + row]);
        else if (wave == 3) v = __int_as_float(p.row_hi[lb * p.Lq + row]);
    }
    x.st = v;
}

template <int D>
__device__ inline void kv_store8(const BwdLaunch& p, const KvStage8<D>& x, uint8_t* qt, uint8_t* gt, float* st) {
    stage_store<D, 512>(x.q, qt);
    stage_store<D, 512>(x.g, gt);
    if (threadIdx.x < 256) st[threadIdx.x] = x.st;
}

// Rows rh*32 .. rh*32+31 of one query tile against the wave's 32 keys (K and
// V rows kg*32 + l32 of the LDS key tiles kt, vt): 2 D/16 score steps with
// the S and dP chains alternating, the element-wise work, then 4 D/32 update
// steps; LDS operand reads two steps ahead.
template <int D>
__device__ inline void kv_compute8(const BwdLaunch& p, const uint8_t* qt, const uint8_t* gt, const float* st,
                                   const uint8_t* kt, const uint8_t* vt, int kr, f32x16 (&dk)[D / 32],
                                   f32x16 (&dv)[D / 32], const QCursor& c, i64 lb, int kw0, int rh) {
    using C = Cfg<D>;
    constexpr int NS = 2 * C::NDS, NM = 4 * C::NDB, NT = NS + NM, AH = 2;
    const int lane = threadIdx.x & 63, l32 = lane & 31, hb = lane >> 5;
    const int key = kw0 + l32;
    const i32x4 s = ld_const((const i32x4*)p.qsum, lb * p.nqt + c.m);
    const bool masked = !(s[2] <= kw0 && kw0 + 32 <= s[3]);
    const float sc = p.scale * kLog2e;
    f32x16 S = {}, G = {};
    uint4 pp[2], pd[2];
    // step i: A operand (and, for the score steps, the B operand) from LDS
    struct Ops {
        uint4 a, b;
    };
    auto ld = [&](const int i) __attribute__((always_inline)) {
        Ops o;
        if (i < NS) {
            const int ds = i >> 1;
            if (i & 1) { o.a = frag_rows<D>(gt, rh, ds); o.b = frag_rows<D>(vt, kr, ds); }
            else { o.a = frag_rows<D>(qt, rh, ds); o.b = frag_rows<D>(kt, kr, ds); }
        } else {
            const int m = i - NS, k2 = m / (2 * C::NDB), w = (m / C::NDB) & 1, db = m % C::NDB;
            o.a = frag_cols<D>(w ? qt : gt, rh * 2 + k2, db);
            o.b = uint4{0, 0, 0, 0};
        }
        return o;
    };
    Ops fa[NT];
    static_for<AH>([&](auto ic) { fa[ic.value] = ld(ic.value); });
    static_for<NT>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i + AH < NT) fa[i + AH] = ld(i + AH);
        if constexpr (i < NS) {
            if constexpr (i & 1) G = mfma(fa[i].a, fa[i].b, G);
            else S = mfma(fa[i].a, fa[i].b, S);
        } else {
            constexpr int m = i - NS, k2 = m / (2 * C::NDB), w = (m / C::NDB) & 1, db = m % C::NDB;
            if constexpr (w) dk[db] = mfma(fa[i].a, pd[k2], dk[db]);
            else dv[db] = mfma(fa[i].a, pp[k2], dv[db]);
        }
        if constexpr (i == NS - 1) {
            // P and dS of this lane's rows rh*32 + 8g + 4hb + e
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int rb = rh * 32 + 8 * g + 4 * hb;
                const f32x4 L = *(const f32x4*)(st + rb);
                const f32x4 Dl = *(const f32x4*)(st + 64 + rb);
                float pv[4], dv4[4];
                if (masked) {
                    const i32x4 lo = *(const i32x4*)(st + 128 + rb);
                    const i32x4 hi = *(const i32x4*)(st + 192 + rb);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool vis = lo[e] <= key && key < hi[e];
                        const float x = pin(__builtin_amdgcn_exp2f(__builtin_fmaf(S[4 * g + e], sc, -L[e] * kLog2e)));
                        const float d = pin(x * (G[4 * g + e] - Dl[e]));
                        pv[e] = vis ? x : 0.0f;
                        dv4[e] = vis ? d : 0.0f;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[4 * g + e], sc, -L[e] * kLog2e));
                        dv4[e] = pv[e] * (G[4 * g + e] - Dl[e]);
                    }
                }
                const uint32_t a0 = pack_bf16x2(pv[0], pv[1]), a1 = pack_bf16x2(pv[2], pv[3]);
                const uint32_t b0 = pack_bf16x2(dv4[0], dv4[1]), b1 = pack_bf16x2(dv4[2], dv4[3]);
                if (g & 1) {
                    pp[g >> 1].z = a0; pp[g >> 1].w = a1;
                    pd[g >> 1].z = b0; pd[g >> 1].w = b1;
                } else {
                    pp[g >> 1].x = a0; pp[g >> 1].y = a1;
                    pd[g >> 1].x = b0; pd[g >> 1].y = b1;
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    });
}

template <int D, int G>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv8(const BwdLaunch p) {
    using C = Cfg<D>;
    // K and V of the 128 keys (two 64-row tiles each), Q / dO tiles (two
    // buffers) and the rows' statistics.  At the end the four arrays hold the
    // row-half-1 waves' partial dK and dV, one array per key group.
    __shared__ __attribute__((aligned(1024))) uint8_t ks[2][C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t vs[2][C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t qs[2][C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t gs[2][C::TILE_BYTES];
    __shared__ __attribute__((aligned(256))) float ss[2][256];  // LSE, delta, lo, hi of 64 rows

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31;
    const int kg = wave & 3, rh = wave >> 2;  // key group, row half (waves w and w+4 share a SIMD)
    const i64 logical = xcd_remap(blockIdx.x, gridDim.x);
    const i64 bhk = logical / p.nkb, kb = logical % p.nkb;
    const i64 b = bhk / p.Hk, hk = bhk % p.Hk;
    const i64 lb = p.list_batch == 1 ? 0 : b;
    const int k0 = (int)kb * kKeyBlock, kw0 = k0 + kg * 32;
    const int key = kw0 + l32;

    // The block's K and V rows (past kv_valid: zeros) into LDS.
    {
        Staged<D, 512> x;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int j0 = k0 + 64 * half;
            const int nk = (int)min((i64)kTile, p.mask.kv_valid - j0);
            stage_load<D, 512>(x, (const __bf16*)p.k + b * p.k_sB + (i64)j0 * p.k_sL + hk * p.k_sH, p.k_sL, nk);
            stage_store<D, 512>(x, ks[half]);
            stage_load<D, 512>(x, (const __bf16*)p.v + b * p.v_sB + (i64)j0 * p.v_sL + hk * p.v_sH, p.v_sL, nk);
            stage_store<D, 512>(x, vs[half]);
        }
    }
    f32x16 dk[C::NDB], dv[C::NDB];
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) { dk[d] = f32x16{}; dv[d] = f32x16{}; }

    const int m0 = ld_const(p.kfirst, lb * p.nkb + kb), m1 = ld_const(p.klast, lb * p.nkb + kb);
    QCursor cur{0, m0 - 1};
    bool have = m0 <= m1 && q_next(p, cur, lb, m0, m1, k0, k0 + kKeyBlock);
    KvStage8<D> stg;
    if (have) {
        kv_load8<D>(p, stg, cur, b, hk, lb);
        kv_store8<D>(p, stg, qs[0], gs[0], ss[0]);
    }
    wait_loads();
    int buf = 0;
    while (have) {
        // Buffer `buf` (and the key tiles) are complete, and every wave is done
        // with the other buffer.
        __syncthreads();
        QCursor nxt = cur;
        const bool more = q_next(p, nxt, lb, m0, m1, k0, k0 + kKeyBlock);
        if (more) kv_load8<D>(p, stg, nxt, b, hk, lb);
        kv_compute8<D>(p, qs[buf], gs[buf], ss[buf], ks[kg >> 1], vs[kg >> 1], kg & 1, dk, dv, cur, lb, kw0, rh);
        if (more) kv_store8<D>(p, stg, qs[buf ^ 1], gs[buf ^ 1], ss[buf ^ 1]);
        cur = nxt;
        have = more;
        buf ^= 1;
    }
    // The row-half-1 wave of each key group hands its partial sums to the
    // row-half-0 wave: lane-major, 8 D/32 x 16 floats per lane (32 KB).
    __syncthreads();
    float* red = (float*)(kg == 0 ? &ks[0][0] : kg == 1 ? &vs[0][0] : kg == 2 ? &qs[0][0] : &gs[0][0]);
    if (rh == 1) {
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                red[((2 * db) * 16 + j) * 64 + lane] = dk[db][j];
                red[((2 * db + 1) * 16 + j) * 64 + lane] = dv[db][j];
            }
    }
    __syncthreads();
    if (rh == 0) {
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                dk[db][j] += red[((2 * db) * 16 + j) * 64 + lane];
                dv[db][j] += red[((2 * db + 1) * 16 + j) * 64 + lane];
            }
        if (key < p.Lk) {
            const i64 es = G == BWA_F32 ? 4 : 2;
            char* dkr = (char*)p.dk + (b * p.dk_sB + (i64)key * p.dk_sL + hk * p.dk_sH) * es;
            char* dvr = (char*)p.dv + (b * p.dv_sB + (i64)key * p.dv_sL + hk * p.dv_sH) * es;
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
                store_tile<G>(dkr, dk[db], db, p.scale);
                store_tile<G>(dvr, dv[db], db, 1.0f);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dK / dV for masks with element terms (dilated bands, document ids): 4 waves
// x 32 keys, one wave per SIMD.  A wave keeps its keys' K and V rows as
// operands in registers and accumulates dK^T and dV^T (32 d x 32 keys per
// block of d) while 64-row tiles of Q and dO, with the rows' LSE, delta, key
// intervals and document ids, stream through LDS.  The element test needs
// registers that the two-wave form above does not have to spare.
// ---------------------------------------------------------------------------
// Loads of one query tile (Q, dO and the rows' LSE, delta and key interval)
// into registers; the work-items of wave w load statistic w.
template <int D>
struct KvStage {
    Staged<D> q, g;
    float st;
    int id;  // document id of row tid (work-items 0..63, document masks only)
};

template <int D>
__device__ inline void kv_load(const BwdLaunch& p, KvStage<D>& x, const QCursor& c, i64 b, i64 hk, i64 lb) {
    const i64 h = hk * p.kv_group + c.g;
    const i64 r0 = (i64)c.m * kTile;
    const int nq = (int)min((i64)kTile, p.mask.q_valid - r0);
    stage_load<D>(x.q, (const __bf16*)p.q + b * p.q_sB + r0 * p.q_sL + h * p.q_sH, p.q_sL, nq);
    stage_load<D>(x.g, (const __bf16*)p.dout + b * p.do_sB + r0 * p.do_sL + h * p.do_sH, p.do_sL, nq);
    const int wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const i64 row = r0 + lane;
    const i64 li = (b * p.H + h) * p.Lq + row;
    float v = 0.0f;
    if (row < p.Lq) {
        if (wave == 0) v = p.lse[li];
        else if (wave == 1) v = p.delta[li];
        else if (wave == 2) v = __int_as_float(p.row_lo[lb * p.Lq + row]);
        else v = __int_as_float(p.row_hi[lb * p.Lq + row]);
    }
    x.st = v;
    if (p.mask.seg_mode == 3 && wave == 0) x.id = row < p.Lq ? p.mask.ids_q[b * p.mask.lq + row] : -1;
}

template <int D>
__device__ inline void kv_store(const BwdLaunch& p, const KvStage<D>& x, uint8_t* qt, uint8_t* gt, float* st) {
    stage_store<D>(x.q, qt);
    stage_store<D>(x.g, gt);
    st[threadIdx.x] = x.st;
    if (p.mask.seg_mode == 3 && threadIdx.x < 64) st[256 + threadIdx.x] = __int_as_float(x.id);
}

// One 64-row query tile against the wave's 32 keys: 64 matrix-core steps in
// one stream, with the element-wise work of each 32-row chunk (P, dS and
// their bf16 packing, in four slices of 4 rows) issued between the products
// of the next phase, so that it runs while the matrix core works:
//   steps [0, NS)            S, dP of chunk 0
//   steps [NS, 2NS)          S, dP of chunk 1      + slices of chunk 0
//   steps [2NS, 2NS+NM)      dV, dK of chunk 0     + slices of chunk 1
//   steps [2NS+NM, 2NS+2NM)  dV, dK of chunk 1
// (NS = 2 D/16 score steps, NM = 4 D/32 update steps per chunk).  S and dP
// alternate between their two accumulation chains; LDS operand reads run
// kAhead steps ahead of their use.
template <int D>
__device__ inline void kv_compute(const BwdLaunch& p, const uint8_t* qt, const uint8_t* gt, const float* st,
                                  const uint4 (&kf)[D / 16], const uint4 (&vf)[D / 16], f32x16 (&dk)[D / 32],
                                  f32x16 (&dv)[D / 32], const QCursor& c, int kw0, int key_id, int key_res,
                                  unsigned dpat) {
    using C = Cfg<D>;
    constexpr int NS = 2 * C::NDS, NM = 4 * C::NDB, NT = 2 * NS + 2 * NM;
    const int lane = threadIdx.x & 63, l32 = lane & 31, hb = lane >> 5;
    const int key = kw0 + l32;
    const float sc = p.scale * kLog2e;
    f32x16 S[2] = {f32x16{}, f32x16{}}, G[2] = {f32x16{}, f32x16{}};
    uint4 pp[2][2], pd[2][2];  // bf16 P and dS per chunk and 16-row step

    auto ld = [&](const int i) __attribute__((always_inline)) {
        if (i < 2 * NS) {
            const int rc = i / NS, j = i % NS;
            return (j & 1) ? frag_rows<D>(gt, rc, j >> 1) : frag_rows<D>(qt, rc, j >> 1);
        }
        const int m = i - 2 * NS, rc = m / NM, j = m % NM;
        const int k2 = j / (2 * C::NDB), w = (j / C::NDB) & 1, db = j % C::NDB;
        return frag_cols<D>(w ? qt : gt, rc * 2 + k2, db);
    };
    // Rows rc*32 + 8g + 4hb + e of this lane: P and dS of slice g.  With a
    // dilated band the rows that see the key are those congruent to
    // key + kv_offset modulo g: a bit per row of the 32-row chunk.
    unsigned rbits[2] = {~0u, ~0u};
    if (p.mask.dilation > 1) {
#pragma unroll
        for (int rc = 0; rc < 2; ++rc) rbits[rc] = dil_bits(key_res, c.m * kTile + rc * 32, p.mask.dilation, dpat);
    }
    auto slice = [&](const int rc, const int g) __attribute__((always_inline)) {
        const int rb = rc * 32 + 8 * g + 4 * hb;
        const f32x4 L = *(const f32x4*)(st + rb);
        const f32x4 Dl = *(const f32x4*)(st + 64 + rb);
        const i32x4 lo = *(const i32x4*)(st + 128 + rb);
        const i32x4 hi = *(const i32x4*)(st + 192 + rb);
        i32x4 rid = {0, 0, 0, 0};
        if (p.mask.seg_mode == 3) rid = *(const i32x4*)(st + 256 + rb);
        float pv[4], dv4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bool vis = lo[e] <= key && key < hi[e] && ((rbits[rc] >> (8 * g + 4 * hb + e)) & 1u);
            if (p.mask.seg_mode == 3) vis = vis && rid[e] == key_id;
            const float x = pin(__builtin_amdgcn_exp2f(__builtin_fmaf(S[rc][4 * g + e], sc, -L[e] * kLog2e)));
            const float d = pin(x * (G[rc][4 * g + e] - Dl[e]));
            pv[e] = vis ? x : 0.0f;
            dv4[e] = vis ? d : 0.0f;
        }
        const uint32_t a0 = pack_bf16x2(pv[0], pv[1]), a1 = pack_bf16x2(pv[2], pv[3]);
        const uint32_t b0 = pack_bf16x2(dv4[0], dv4[1]), b1 = pack_bf16x2(dv4[2], dv4[3]);
        if (g & 1) {
            pp[rc][g >> 1].z = a0; pp[rc][g >> 1].w = a1;
            pd[rc][g >> 1].z = b0; pd[rc][g >> 1].w = b1;
        } else {
            pp[rc][g >> 1].x = a0; pp[rc][g >> 1].y = a1;
            pd[rc][g >> 1].x = b0; pd[rc][g >> 1].y = b1;
        }
    };

    uint4 fa[NT];
    static_for<kAhead>([&](auto ic) { fa[ic.value] = ld(ic.value); });
    static_for<NT>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i + kAhead < NT) fa[i + kAhead] = ld(i + kAhead);
        if constexpr (i < 2 * NS) {
            constexpr int rc = i / NS, j = i % NS;
            if constexpr (j & 1) G[rc] = mfma(fa[i], vf[j >> 1], G[rc]);
            else S[rc] = mfma(fa[i], kf[j >> 1], S[rc]);
        } else {
            constexpr int m = i - 2 * NS, rc = m / NM, j = m % NM;
            constexpr int k2 = j / (2 * C::NDB), w = (j / C::NDB) & 1, db = j % C::NDB;
            if constexpr (w) dk[db] = mfma(fa[i], pd[rc][k2], dk[db]);
            else dv[db] = mfma(fa[i], pp[rc][k2], dv[db]);
        }
        if constexpr (i >= NS && i < 2 * NS && (i - NS) % (NS / 4) == NS / 4 - 1) slice(0, (i - NS) / (NS / 4));
        if constexpr (i >= 2 * NS && i < 2 * NS + NM && (i - 2 * NS) % (NM / 4) == NM / 4 - 1)
            slice(1, (i - 2 * NS) / (NM / 4));
        __builtin_amdgcn_sched_barrier(0);
    });
}

template <int D, int G>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv(const BwdLaunch p) {
    using C = Cfg<D>;
    // Three tile buffers.  A tile's loads go to registers two iterations
    // before it is computed and land in LDS one iteration before, so each
    // load has a whole tile of compute to arrive.
    __shared__ __attribute__((aligned(1024))) uint8_t qs[kRing][C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t gs[kRing][C::TILE_BYTES];
    __shared__ __attribute__((aligned(256))) float ss[kRing][320];  // LSE, delta, lo, hi, doc id of 64 rows

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hb = lane >> 5;
    const i64 logical = xcd_remap(blockIdx.x, gridDim.x);
    const i64 bhk = logical / p.nkb, kb = logical % p.nkb;
    const i64 b = bhk / p.Hk, hk = bhk % p.Hk;
    const i64 lb = p.list_batch == 1 ? 0 : b;
    const int k0 = (int)kb * kKeyBlock, kw0 = k0 + wave * 32;
    const int key = kw0 + l32;
    const bool key_in = key < p.mask.kv_valid;  // keys past kv_valid are zeros (and masked)

    // K and V rows of this lane's key as the B operand: d = ds*16 + hb*8 + 0..7.
    uint4 kf[C::NDS], vf[C::NDS];
    const __bf16* kp = (const __bf16*)p.k + b * p.k_sB + (i64)key * p.k_sL + hk * p.k_sH;
    const __bf16* vp = (const __bf16*)p.v + b * p.v_sB + (i64)key * p.v_sL + hk * p.v_sH;
#pragma unroll
    for (int ds = 0; ds < C::NDS; ++ds) {
        kf[ds] = key_in ? *(const uint4*)(kp + ds * 16 + hb * 8) : uint4{0, 0, 0, 0};
        vf[ds] = key_in ? *(const uint4*)(vp + ds * 16 + hb * 8) : uint4{0, 0, 0, 0};
    }
    f32x16 dk[C::NDB], dv[C::NDB];
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) { dk[d] = f32x16{}; dv[d] = f32x16{}; }
    const int key_id = (p.mask.seg_mode == 3 && key < p.Lk) ? p.mask.ids_kv[b * p.mask.lk + key] : -1;
    // (key + kv_offset) mod g: the rows congruent to it see the key
    const int key_res = p.mask.dilation > 1
                            ? (int)((((i64)key + p.mask.kv_offset) % p.mask.dilation + p.mask.dilation) % p.mask.dilation)
                            : 0;
    const unsigned dpat = p.mask.dilation > 1 ? dil_pattern(p.mask.dilation) : 0u;
    wait_loads();

    const int m0 = ld_const(p.kfirst, lb * p.nkb + kb), m1 = ld_const(p.klast, lb * p.nkb + kb);
    QCursor cur{0, m0 - 1};
    bool have = m0 <= m1 && q_next(p, cur, lb, m0, m1, k0, k0 + kKeyBlock);
    // Prologue: the first tile in LDS, the second in registers.
    KvStage<D> stg;
    QCursor ahead = cur;  // the tile whose loads are in registers
    bool staged = false;
    if (have) {
        kv_load<D>(p, stg, cur, b, hk, lb);
        kv_store<D>(p, stg, qs[0], gs[0], ss[0]);
        staged = q_next(p, ahead, lb, m0, m1, k0, k0 + kKeyBlock);
        if (staged) kv_load<D>(p, stg, ahead, b, hk, lb);
    }
    int buf = 0;
    while (have) {
        // Buffer `buf` is complete, and every wave is done with the buffer of
        // the tile before it, which takes the staged tile now.
        __syncthreads();
        const int nb = buf == kRing - 1 ? 0 : buf + 1;
        if (staged) {
            kv_store<D>(p, stg, qs[nb], gs[nb], ss[nb]);
            staged = q_next(p, ahead, lb, m0, m1, k0, k0 + kKeyBlock);
            if (staged) kv_load<D>(p, stg, ahead, b, hk, lb);
        }
        kv_compute<D>(p, qs[buf], gs[buf], ss[buf], kf, vf, dk, dv, cur, kw0, key_id, key_res, dpat);
        have = q_next(p, cur, lb, m0, m1, k0, k0 + kKeyBlock);
        buf = nb;
    }
    if (key < p.Lk) {
        const i64 es = G == BWA_F32 ? 4 : 2;
        char* dkr = (char*)p.dk + (b * p.dk_sB + (i64)key * p.dk_sL + hk * p.dk_sH) * es;
        char* dvr = (char*)p.dv + (b * p.dv_sB + (i64)key * p.dv_sL + hk * p.dv_sH) * es;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            store_tile<G>(dkr, dk[db], db, p.scale);
            store_tile<G>(dvr, dv[db], db, 1.0f);
        }
    }
}

// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// dQ: 8 waves x 32 rows.  A wave keeps its rows' Q and dO as operands in
// registers and accumulates dQ^T while 64-key tiles of K and V stream
// through a ring of three LDS buffers in the chosen order.
// ---------------------------------------------------------------------------
// Key tiles of a query block in the chosen order: position r of a
// permutation of all nkt tiles, keeping the tiles in [t_lo, t_hi).
struct TCursor {
    int r, t;
};

__device__ inline int order_tile(const BwdLaunch& p, int r) {
    const int n = (int)p.nkt;
    switch (p.order) {
        case BWA_ORDER_DESC: return n - 1 - r;
        case BWA_ORDER_OUTSIDE_IN: return (r & 1) ? n - 1 - (r >> 1) : (r >> 1);
        case BWA_ORDER_CUSTOM: return ld_const(p.perm, r);
        default: return r;
    }
}

__device__ inline bool t_next(const BwdLaunch& p, TCursor& c, int t_lo, int t_hi) {
    if (p.order == BWA_ORDER_ASC) {
        if (c.r < 0) c.r = t_lo - 1;
        if (++c.r >= t_hi) return false;
        c.t = c.r;
        return true;
    }
    if (p.order == BWA_ORDER_DESC) {
        if (c.r < 0) c.r = (int)p.nkt - t_hi - 1;
        if (++c.r >= (int)p.nkt - t_lo) return false;
        c.t = (int)p.nkt - 1 - c.r;
        return true;
    }
    for (;;) {
        if (++c.r >= (int)p.nkt) return false;
        const int t = order_tile(p, c.r);
        if (t >= t_lo && t < t_hi) {
            c.t = t;
            return true;
        }
    }
}

template <int D, int NT>
struct QStage {
    Staged<D, NT> k, v;
};

template <int D, int NT>
__device__ inline void q_load(const BwdLaunch& p, QStage<D, NT>& x, int t, i64 b, i64 hk) {
    const i64 j0 = (i64)t * kTile;
    const int nk = (int)min((i64)kTile, p.mask.kv_valid - j0);
    stage_load<D, NT>(x.k, (const __bf16*)p.k + b * p.k_sB + j0 * p.k_sL + hk * p.k_sH, p.k_sL, nk);
    stage_load<D, NT>(x.v, (const __bf16*)p.v + b * p.v_sB + j0 * p.v_sL + hk * p.v_sH, p.v_sL, nk);
}

// One 64-key tile against the wave's 32 rows, with two waves per SIMD (the
// other wave's products cover this one's element-wise work): each 32-key
// half runs its S^T and dP^T products (the two chains alternating), its dS
// and its own dQ^T products in turn, so only one half's scores and dS are
// live; LDS operand reads run two steps ahead.
template <int D, bool XM>
__device__ inline void q_compute(const BwdLaunch& p, const uint8_t* kt, const uint8_t* vt,
                                     const uint4 (&qf)[D / 16], const uint4 (&gf)[D / 16], f32x16 (&dq)[D / 32],
                                     int t, int full_lo, int full_hi, int lo, int hi, float lse2, float delt, i64 b,
                                     int row, int row_id, int row_res, unsigned dpat) {
    using C = Cfg<D>;
    constexpr int NS = 2 * C::NDS, NH = 2 * C::NDB, NP = NS + NH;  // steps per half
    constexpr int AH = 2;                                            // read-ahead
    const int lane = threadIdx.x & 63, hb = lane >> 5;
    const int j0 = t * kTile;
    const bool masked = XM || !(full_lo <= j0 && j0 + kTile <= full_hi);
    const float sc = p.scale * kLog2e;
    static_for<2>([&](auto kbc) {
        constexpr int kb = decltype(kbc)::value;
        f32x16 S = {}, G = {};
        uint4 pd[2];
        auto ld = [&](const int i) __attribute__((always_inline)) {
            if (i < NS) return (i & 1) ? frag_rows<D>(vt, kb, i >> 1) : frag_rows<D>(kt, kb, i >> 1);
            const int m = i - NS;
            return frag_cols<D>(kt, kb * 2 + m / C::NDB, m % C::NDB);
        };
        uint4 fa[NP];
        static_for<AH>([&](auto ic) { fa[ic.value] = ld(ic.value); });
        static_for<NP>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i + AH < NP) fa[i + AH] = ld(i + AH);
            if constexpr (i < NS) {
                if constexpr (i & 1) G = mfma(fa[i], gf[i >> 1], G);
                else S = mfma(fa[i], qf[i >> 1], S);
            } else {
                constexpr int m = i - NS;
                dq[m % C::NDB] = mfma(fa[i], pd[m / C::NDB], dq[m % C::NDB]);
            }
            if constexpr (i == NS - 1) {
                // dilated band: the half's keys congruent to row - kv_offset mod g
                unsigned kbits = ~0u;
                if (XM && masked && p.mask.dilation > 1) kbits = dil_bits(row_res, j0 + kb * 32, p.mask.dilation, dpat);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float dsv[4];
                    int kid[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                    if (XM && masked && p.mask.seg_mode == 3) key_ids8(p, b, j0 + kb * 32 + 8 * g, kid);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(S[4 * g + e], sc, -lse2));
                        float d = pin(x * (G[4 * g + e] - delt));
                        if (masked) {
                            const int key = j0 + kb * 32 + 8 * g + 4 * hb + e;
                            bool vis = lo <= key && key < hi;
                            if (XM) {
                                vis = vis && ((kbits >> (8 * g + 4 * hb + e)) & 1u);
                                if (p.mask.seg_mode == 3) vis = vis && row_id == (hb ? kid[4 + e] : kid[e]);
                            }
                            d = vis ? d : 0.0f;
                        }
                        dsv[e] = d;
                    }
                    const uint32_t a0 = pack_bf16x2(dsv[0], dsv[1]), a1 = pack_bf16x2(dsv[2], dsv[3]);
                    if (g & 1) { pd[g >> 1].z = a0; pd[g >> 1].w = a1; }
                    else { pd[g >> 1].x = a0; pd[g >> 1].y = a1; }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    });
}

template <int D, int G, bool XM, int NW>
__global__ __launch_bounds__(NW * 64, 1) void attn_bwd_dq(const BwdLaunch p) {
    using C = Cfg<D>;
    constexpr int NT = NW * 64, RB = NW * 32;  // work-items, rows per workgroup
    __shared__ __attribute__((aligned(1024))) uint8_t ks[kRing][C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t vs[kRing][C::TILE_BYTES];
    __shared__ int red[4 * NW];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hb = lane >> 5;
    const i64 nqb = (p.Lq + RB - 1) / RB;
    const i64 logical = xcd_remap(blockIdx.x, gridDim.x);
    const i64 bh = logical / nqb;
    const i64 qb = nqb - 1 - logical % nqb;  // the blocks with the most key tiles first
    const i64 b = bh / p.H, h = bh % p.H, hk = h / p.kv_group;
    const i64 lb = p.list_batch == 1 ? 0 : b;
    const int row = (int)(qb * RB) + wave * 32 + l32;
    const bool row_ok = row < p.Lq;
    const bool row_in = row < p.mask.q_valid;  // rows past q_valid are zeros (and see nothing)

    int lo = 0, hi = 0;
    float lse2 = 0.0f, delt = 0.0f;
    if (row_ok) {
        lo = p.row_lo[lb * p.Lq + row];
        hi = p.row_hi[lb * p.Lq + row];
        const i64 li = (b * p.H + h) * p.Lq + row;
        lse2 = p.lse[li] * kLog2e;
        delt = p.delta[li];
    }
    const int row_id = (XM && p.mask.seg_mode == 3 && row_ok) ? p.mask.ids_q[b * p.mask.lq + row] : -1;
    // (row - kv_offset) mod g: the keys congruent to it are seen
    const int row_res = (XM && p.mask.dilation > 1)
                            ? (int)((((i64)row - p.mask.kv_offset) % p.mask.dilation + p.mask.dilation) % p.mask.dilation)
                            : 0;
    const unsigned dpat = (XM && p.mask.dilation > 1) ? dil_pattern(p.mask.dilation) : 0u;
    // Q and dO rows of this lane as the B operand: d = ds*16 + hb*8 + 0..7.
    uint4 qf[C::NDS], gf[C::NDS];
    const __bf16* qp = (const __bf16*)p.q + b * p.q_sB + (i64)row * p.q_sL + h * p.q_sH;
    const __bf16* gp = (const __bf16*)p.dout + b * p.do_sB + (i64)row * p.do_sL + h * p.do_sH;
#pragma unroll
    for (int ds = 0; ds < C::NDS; ++ds) {
        qf[ds] = row_in ? *(const uint4*)(qp + ds * 16 + hb * 8) : uint4{0, 0, 0, 0};
        gf[ds] = row_in ? *(const uint4*)(gp + ds * 16 + hb * 8) : uint4{0, 0, 0, 0};
    }
    f32x16 dq[C::NDB];
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) dq[d] = f32x16{};
    wait_loads();

    // Envelope and common part of the block's row intervals.
    const bool ne = lo < hi;
    int v0r = wave_min(ne ? lo : kBig), v1r = wave_max(ne ? hi : 0);
    int v2r = wave_max(ne ? lo : kBig), v3r = wave_min(ne ? hi : -1);
    if (lane == 0) {
        red[wave * 4 + 0] = v0r; red[wave * 4 + 1] = v1r;
        red[wave * 4 + 2] = v2r; red[wave * 4 + 3] = v3r;
    }
    __syncthreads();
    int env_lo = kBig, env_hi = 0, full_lo = 0, full_hi = kBig;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        env_lo = min(env_lo, red[w * 4 + 0]);
        env_hi = max(env_hi, red[w * 4 + 1]);
        full_lo = max(full_lo, red[w * 4 + 2]);
        full_hi = min(full_hi, red[w * 4 + 3]);
    }
    env_lo = uni(env_lo); env_hi = uni(env_hi); full_lo = uni(full_lo); full_hi = uni(full_hi);
    const int t_lo = env_lo < env_hi ? env_lo / kTile : 0;
    const int t_hi = env_lo < env_hi ? (env_hi + kTile - 1) / kTile : 0;

    // Same pipeline as the dK/dV kernel: loads two tiles ahead in registers,
    // stores one tile ahead into a ring of three buffers.
    TCursor cur{-1, 0};
    bool have = t_next(p, cur, t_lo, t_hi);
    QStage<D, NT> stg;
    TCursor ahead = cur;
    bool staged = false;
    if (have) {
        q_load<D, NT>(p, stg, cur.t, b, hk);
        stage_store<D, NT>(stg.k, ks[0]);
        stage_store<D, NT>(stg.v, vs[0]);
        staged = t_next(p, ahead, t_lo, t_hi);
        if (staged) q_load<D, NT>(p, stg, ahead.t, b, hk);
    }
    int buf = 0;
    while (have) {
        __syncthreads();
        const int nb = buf == kRing - 1 ? 0 : buf + 1;
        if (staged) {
            stage_store<D, NT>(stg.k, ks[nb]);
            stage_store<D, NT>(stg.v, vs[nb]);
            staged = t_next(p, ahead, t_lo, t_hi);
            if (staged) q_load<D, NT>(p, stg, ahead.t, b, hk);
        }
        q_compute<D, XM>(p, ks[buf], vs[buf], qf, gf, dq, cur.t, full_lo, full_hi, lo, hi, lse2, delt, b, row,
                         row_id, row_res, dpat);
        have = t_next(p, cur, t_lo, t_hi);
        buf = nb;
    }
    if (row_ok) {
        const i64 es = G == BWA_F32 ? 4 : 2;
        char* dqr = (char*)p.dq + (b * p.dq_sB + (i64)row * p.dq_sL + h * p.dq_sH) * es;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) store_tile<G>(dqr, dq[db], db, p.scale);
    }
}

template <int D, int G>
hipError_t launch_dg(const BwdLaunch& a, hipStream_t stream) {
    const bool xm = a.mask.dilation > 1 || a.mask.seg_mode == 3;
    const i64 nkb_total = (i64)a.B * a.Hk * a.nkb;
    if (nkb_total > 0) {
        // element masks: one wave per SIMD; interval masks: two
        if (xm) hipLaunchKernelGGL((attn_bwd_dkdv<D, G>), dim3((unsigned)nkb_total), dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((attn_bwd_dkdv8<D, G>), dim3((unsigned)nkb_total), dim3(512), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    constexpr int NW = kDqWaves;
    const i64 nqb_total = (i64)a.B * a.H * ((a.Lq + 32 * NW - 1) / (32 * NW));
    if (nqb_total > 0) {
        if (xm)
            hipLaunchKernelGGL((attn_bwd_dq<D, G, true, NW>), dim3((unsigned)nqb_total), dim3(64 * NW), 0, stream, a);
        else
            hipLaunchKernelGGL((attn_bwd_dq<D, G, false, NW>), dim3((unsigned)nqb_total), dim3(64 * NW), 0, stream, a);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BwdLaunch& a, hipStream_t stream) {
    // plan, then delta, then the two gradient kernels
    const i64 rows = max(a.list_batch * a.Lq, a.list_batch * a.nkb);
    if (rows > 0) hipLaunchKernelGGL(bwd_rows_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, a);
    if (a.list_batch * a.nqt > 0)
        hipLaunchKernelGGL(bwd_qtiles_kernel, dim3((unsigned)(a.list_batch * a.nqt)), dim3(64), 0, stream, a);
    const i64 drows = (i64)a.B * a.Lq * a.H;
    if (drows > 0) {
        const i64 blocks = (drows * (D / 8) + 255) / 256;
        if (a.o_dtype == BWA_F32) hipLaunchKernelGGL((bwd_delta_kernel<D, BWA_F32>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((bwd_delta_kernel<D, BWA_BF16>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return a.grad_dtype == BWA_F32 ? launch_dg<D, BWA_F32>(a, stream) : launch_dg<D, BWA_BF16>(a, stream);
}

}  // namespace

hipError_t launch_attn_bwd(const BwdLaunch& a, hipStream_t stream) {
    return a.D == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

static i64 pad256(i64 x) { return (x + 255) / 256 * 256; }

i64 bwd_workspace_bytes(i64 B, i64 H, i64 Lq, i64 Lk, i64 list_batch) {
    const i64 nqt = (Lq + kTile - 1) / kTile, nkb = (Lk + kKeyBlock - 1) / kKeyBlock;
    return pad256(B * H * Lq * 4) + 2 * pad256(list_batch * Lq * 4) + pad256(list_batch * nqt * 16) +
           2 * pad256(list_batch * nkb * 4);
}

void bwd_workspace_layout(BwdLaunch& a, void* ws) {
    char* w = (char*)ws;
    a.nqt = (a.Lq + kTile - 1) / kTile;
    a.nkb = (a.Lk + kKeyBlock - 1) / kKeyBlock;
    a.nkt = (a.Lk + kTile - 1) / kTile;
    a.delta = (float*)w; w += pad256((i64)a.B * a.H * a.Lq * 4);
    a.row_lo = (int*)w; w += pad256(a.list_batch * a.Lq * 4);
    a.row_hi = (int*)w; w += pad256(a.list_batch * a.Lq * 4);
    a.qsum = (int4*)w; w += pad256(a.list_batch * a.nqt * 16);
    a.kfirst = (int*)w; w += pad256(a.list_batch * a.nkb * 4);
    a.klast = (int*)w;
}

}  // namespace bwa
