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
typedef int i32x2 __attribute__((ext_vector_type(2)));
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

// (Each LDS address below is the tile's base plus one integer offset: the
// compiler tells which LDS array a read touches only through a short chain of
// address steps, and a read it cannot place waits for every copy into LDS in
// flight.)
// Operand fragment whose rows are tile rows rb*32 + l32 (16-deep step ds over
// d: the lane holds d = ds*16 + hb*8 + 0..7).
template <int D>
__device__ inline uint4 frag_rows(const uint8_t* t, int rb, int ds) {
    const int lane = threadIdx.x & 63, l32 = lane & 31, hb = lane >> 5;
    const int r = rb * 32 + l32;
    return *(const uint4*)(t + (r * (D * 2) + bswz<D>(r, ds * 2 + hb) * 16));
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
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (r0 * (D * 2) + bswz<D>(r0, c) * 16 + (u & 1) * 8)));
    const s16x4 x1 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (r1 * (D * 2) + bswz<D>(r1, c) * 16 + (u & 1) * 8)));
    uint4 out;
    out.x = __builtin_bit_cast(uint2, x0).x;
    out.y = __builtin_bit_cast(uint2, x0).y;
    out.z = __builtin_bit_cast(uint2, x1).x;
    out.w = __builtin_bit_cast(uint2, x1).y;
    return out;
}

// The lane's byte offsets of frag_rows(t, 0, ds) (ro[ds]) and of the two
// transposing reads of frag_cols(t, 0, db) (co[2 db], co[2 db + 1]) within a
// tile.  The swizzle depends on a row's index modulo 16 only, so another row
// block rb or step kk adds the constant rb*32 or kk*16 rows.  A kernel that
// reads several ring buffers computes these once and adds each buffer's base
// (a constant that the LDS read takes as its immediate offset): without that
// the compiler keeps one set of addresses per buffer alive across the loop.
template <int D>
struct FragOffs {
    int ro[D / 16], co[D / 16];
};

template <int D>
__device__ inline FragOffs<D> frag_offsets() {
    FragOffs<D> f;
    const int lane = threadIdx.x & 63, l32 = lane & 31, hb = lane >> 5;
    const int g1 = (lane >> 4) & 1, s_row = (lane >> 2) & 3, u = lane & 3;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) f.ro[ds] = l32 * (D * 2) + bswz<D>(l32, ds * 2 + hb) * 16;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        const int c = db * 4 + g1 * 2 + (u >> 1);
        const int r0 = hb * 4 + s_row, r1 = r0 + 8;
        f.co[2 * db] = r0 * (D * 2) + bswz<D>(r0, c) * 16 + (u & 1) * 8;
        f.co[2 * db + 1] = r1 * (D * 2) + bswz<D>(r1, c) * 16 + (u & 1) * 8;
    }
    return f;
}

// The offsets as new values: address arithmetic on them stays where it is
// used instead of being hoisted out of the tile loop once per buffer.
template <int D>
__device__ __attribute__((always_inline)) inline void repin(FragOffs<D>& f) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
        asm volatile("" : "+v"(f.ro[i]));
        asm volatile("" : "+v"(f.co[i]));
    }
}

template <int D>
__device__ inline uint4 frag_rows_at(const uint8_t* t, const FragOffs<D>& f, int rb, int ds) {
    return *(const uint4*)(t + (rb * 32 * (D * 2) + f.ro[ds]));
}

template <int D>
__device__ inline uint4 frag_cols_at(const uint8_t* t, const FragOffs<D>& f, int kk, int db) {
    const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (kk * 16 * (D * 2) + f.co[2 * db])));
    const s16x4 x1 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (kk * 16 * (D * 2) + f.co[2 * db + 1])));
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

// Filter bit of a document id (a multiplicative hash onto 32 bits): two
// tiles whose filters share no bit hold no row and key of one document.
__device__ inline unsigned doc_bit(int id) { return 1u << (((unsigned)id * 0x9E3779B1u) >> 27); }

typedef unsigned long long u64;

__device__ inline unsigned wave_or(unsigned x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x |= (unsigned)__shfl_xor((int)x, o);
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

// One 64-row tile (rows past nvalid read as zero) copied from HBM straight
// into LDS: lane i of a buffer load with an LDS destination fills bytes
// [16i, 16i + 16) of a 1 KB run, so each lane loads the global chunk whose
// swizzled place (bswz, its own inverse) is its slot: row r of the tile holds
// its 16-byte chunk c at r*2D + bswz(r, c)*16.  No registers, LDS stores or
// waits on the way.  The buffer range ends with the last valid row's D
// elements; loads past it return zero.  Each of the NW waves issues RUNS/NW
// loads.
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)
typedef __attribute__((address_space(3))) void lds_void;

template <int D, int NW>
struct TileCopy {
    static constexpr int RUNS = Cfg<D>::TILE_BYTES / 1024;  // 1 KB runs per tile
    static constexpr int PER_WAVE = (RUNS + NW - 1) / NW;  // loads per wave and tile
};

template <int D, int NW>
__device__ inline void tile_issue(const __bf16* base, i64 sL, int nvalid, int lds) {
    using T = TileCopy<D, NW>;
    constexpr int NCH = Cfg<D>::NCH;
    const int wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int bytes = uni(nvalid > 0 ? (int)(((i64)(nvalid - 1) * sL + D) * 2) : 0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, kRsrcFlags);
#pragma unroll
    for (int it = 0; it < T::PER_WAVE; ++it) {
        const int run = wave * T::PER_WAVE + it;
        if (T::RUNS % NW == 0 || run < T::RUNS) {
            const int slot = run * 64 + lane, r = slot / NCH, c = bswz<D>(r, slot % NCH);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(uintptr_t)(lds + run * 1024), 16,
                                                     (unsigned)(r * sL * 2 + c * 16), 0, 0, 0);
        }
    }
}

// The 64-row tiles of one head of a tensor, copied into LDS one after
// another: what every copy shares (the head's first row, the tile stride,
// this lane's offsets within a tile) is computed once, so a copy costs a
// multiply, a range and its loads.  Rows at or past `nrows` read as zero.
template <int D, int NW>
struct TileStream {
    const uint8_t* head;
    i64 tile_bytes;  // 64 rows
    int row_bytes;
    int nrows;
    unsigned voff[TileCopy<D, NW>::PER_WAVE];
};

template <int D, int NW>
__device__ inline void stream_init(TileStream<D, NW>& s, const __bf16* head, i64 sL, i64 nrows) {
    using T = TileCopy<D, NW>;
    constexpr int NCH = Cfg<D>::NCH;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    s.head = (const uint8_t*)head;
    s.tile_bytes = sL * 2 * kTile;
    s.row_bytes = (int)(sL * 2);
    s.nrows = (int)nrows;
#pragma unroll
    for (int it = 0; it < T::PER_WAVE; ++it) {
        const int slot = (wave * T::PER_WAVE + it) * 64 + lane, r = slot / NCH, c = bswz<D>(r, slot % NCH);
        s.voff[it] = (unsigned)(r * s.row_bytes + c * 16);
    }
}

template <int D, int NW>
__device__ inline void stream_issue(const TileStream<D, NW>& s, int tile, int lds) {
    using T = TileCopy<D, NW>;
    const int wave = uni(threadIdx.x >> 6);
    const int nvalid = min(max(s.nrows - tile * kTile, 0), kTile);
    const int bytes = uni(nvalid > 0 ? (nvalid - 1) * s.row_bytes + D * 2 : 0);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(s.head + tile * s.tile_bytes), 0, bytes, kRsrcFlags);
#pragma unroll
    for (int it = 0; it < T::PER_WAVE; ++it) {
        const int run = wave * T::PER_WAVE + it;
        if (T::RUNS % NW == 0 || run < T::RUNS)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(uintptr_t)(lds + run * 1024), 16, s.voff[it], 0, 0, 0);
    }
}

// 64 values of a per-row array (rows past `nrows` read as zero) copied by one
// wave: lane i's 4 bytes land at byte 4i.
__device__ inline void stat_issue(const float* head, int nrows, int tile, int lds) {
    const int r0 = tile * kTile;
    const int nr = min(max(nrows - r0, 0), kTile);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(head + r0), 0, uni(nr * 4), kRsrcFlags);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(uintptr_t)lds, 4, (unsigned)((threadIdx.x & 63) * 4), 0, 0, 0);
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
    if (p.mask.seg_mode == 3) {
        const int id = ne ? p.mask.ids_q[lb * p.mask.lq + row] : 0;
        const unsigned f = wave_or(ne ? doc_bit(id) : 0u);
        const u64 seen = __builtin_amdgcn_ballot_w64(ne);
        const int id0 = __shfl(id, seen ? __builtin_ctzll(seen) : 0);
        const bool one = seen != 0 && __builtin_amdgcn_ballot_w64(ne && id != id0) == 0;
        if (lane == 0) {
            p.qbloom[t] = f;
            p.qdoc[2 * t] = one ? 1 : 0;
            p.qdoc[2 * t + 1] = one ? id0 : 0;
        }
    }
    if (env_lo < env_hi) {
        const int n0 = env_lo / kKeyBlock, n1 = (env_hi - 1) / kKeyBlock;
        for (int n = n0 + lane; n <= n1; n += 64) {
            atomicMin(&p.kfirst[lb * p.nkb + n], (int)m);
            atomicMax(&p.klast[lb * p.nkb + n], (int)m);
        }
    }
}

// Document ids: one wave per 64-key tile, the filter of its keys' ids below
// kv_valid.
__global__ __launch_bounds__(64) void bwd_ktiles_kernel(const BwdLaunch p) {
    const i64 t = blockIdx.x;  // over list_batch * nkt
    const i64 lb = t / p.nkt, n = t % p.nkt;
    const i64 key = n * kTile + threadIdx.x;
    const bool in = key < p.mask.kv_valid;
    const int id = in ? p.mask.ids_kv[lb * p.mask.lk + key] : 0;
    const unsigned f = wave_or(in ? doc_bit(id) : 0u);
    const u64 seen = __builtin_amdgcn_ballot_w64(in);
    const int id0 = __shfl(id, 0);
    const bool one = seen != 0 && __builtin_amdgcn_ballot_w64(in && id != id0) == 0;
    if (threadIdx.x == 0) {
        p.kbloom[t] = f;
        p.kdoc[2 * t] = one ? 1 : 0;
        p.kdoc[2 * t + 1] = one ? id0 : 0;
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

// Next (g, m) after c whose rows' envelope meets keys [k0, k1) and, with
// document ids, whose filter meets the key block's filter kf.
template <bool DOC>
__device__ inline bool q_next(const BwdLaunch& p, QCursor& c, i64 lb, int m0, int m1, int k0, int k1, unsigned kf) {
    for (;;) {
        if (++c.m > m1) {
            c.m = m0;
            if (++c.g >= p.kv_group) return false;
        }
        const i32x4 s = ld_const((const i32x4*)p.qsum, lb * p.nqt + c.m);
        if (s[0] < k1 && s[1] > k0 && (!DOC || (ld_const(p.qbloom, lb * p.nqt + c.m) & kf) != 0))
            return true;
    }
}

// The filter of the document ids of keys [k0, k0 + 128).
__device__ inline unsigned key_block_filter(const BwdLaunch& p, i64 lb, int k0) {
    const i64 t = k0 / kTile;
    unsigned f = ld_const(p.kbloom, lb * p.nkt + t);
    if (t + 1 < p.nkt) f |= ld_const(p.kbloom, lb * p.nkt + t + 1);
    return f;
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
// The copies of the query tiles of one query head h of the grouped head hk:
// its Q and dO rows (rows past q_valid read as zero) and the statistic that
// wave w % 4 copies (LSE, delta, key interval lo, hi; rows past Lq read as
// zero and see nothing).
template <int D, int NW>
struct QHead {
    TileStream<D, NW> q, g;
    const float* stat;
    int gh;  // the query head within the group these are for
};

template <int D, int NW>
__device__ inline void qhead_init(const BwdLaunch& p, QHead<D, NW>& x, int g, i64 b, i64 hk, i64 lb) {
    const i64 h = hk * p.kv_group + g;
    stream_init<D, NW>(x.q, (const __bf16*)p.q + b * p.q_sB + h * p.q_sH, p.q_sL, p.mask.q_valid);
    stream_init<D, NW>(x.g, (const __bf16*)p.dout + b * p.do_sB + h * p.do_sH, p.do_sL, p.mask.q_valid);
    const int w = uni(threadIdx.x >> 6) & 3;
    const i64 li = (b * p.H + h) * p.Lq, ri = lb * p.Lq;
    x.stat = w == 0 ? p.lse + li : w == 1 ? p.delta + li
           : w == 2 ? (const float*)(p.row_lo + ri) : (const float*)(p.row_hi + ri);
    x.gh = g;
}

// The LDS of an 8-wave workgroup of the dK/dV or dQ kernel, as two arrays
// (the roles of each part are given with the kernels): ring, three pairs of
// 64-row tiles, and side, four tiles.
template <int D>
using LdsRing = uint8_t[3][2][Cfg<D>::TILE_BYTES];
template <int D>
using LdsSide = uint8_t[4 * Cfg<D>::TILE_BYTES];

// Copies of query tile c into LDS: Q and dO rows and, by waves 0..3, the
// rows' statistics (LSE at st[0..63], delta, lo, hi after it).
template <int D>
__device__ inline void kv_issue8(const BwdLaunch& p, QHead<D, 8>& x, const QCursor& c, i64 b, i64 hk, i64 lb,
                                 int qt, int gt, int st) {
    if (c.g != x.gh) qhead_init<D, 8>(p, x, c.g, b, hk, lb);
    stream_issue<D, 8>(x.q, c.m, qt);
    stream_issue<D, 8>(x.g, c.m, gt);
    const int wave = uni(threadIdx.x >> 6);
    if (wave < 4) stat_issue(x.stat, (int)p.Lq, c.m, st + wave * 256);
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
    // P and dS of this lane's rows rh*32 + 8g + 4hb + e (slice g)
    auto slice = [&](const int g) __attribute__((always_inline)) {
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
        // Slices 0 and 1 feed the first half of the update steps; slices 2
        // and 3, run between those steps, the second.
        if constexpr (i == NS - 1) {
            slice(0);
            slice(1);
        }
        if constexpr (i == NS + 1) slice(2);
        if constexpr (i == NS + NM / 4) slice(3);  // before step NS + NM / 2, the first to use them
        static_assert(NM / 4 > 1 && NM / 4 < NM / 2, "slices 2 and 3 fall between the first-half update steps");
        __builtin_amdgcn_sched_barrier(0);
    });
}

// One dK/dV block of 128 keys (`logical` = (b * Hk + hk) * nkb + key block).
// LDS: side holds K (two 64-row tiles) then V of the 128 keys; ring[x][0]
// and ring[x][1] the Q and dO tiles of buffer x (x = 0, 1); ring[2] the rows'
// statistics of both buffers.  At the end four 32 KB regions (the K, the V,
// and the two Q / dO buffers) hold the row-half-1 waves' partial dK and dV,
// one region per key group.
template <int D, int G>
__device__ __attribute__((always_inline)) inline void dkdv8_block(const BwdLaunch& p, i64 logical, LdsRing<D>& ring,
                                                                  LdsSide<D>& side) {
    using C = Cfg<D>;
    constexpr int T = C::TILE_BYTES;
    float* const ss0 = (float*)&ring[2][0][0];  // LSE, delta, lo, hi of 64 rows, per buffer (256 floats)

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31;
    const int kg = wave & 3, rh = wave >> 2;  // key group, row half (waves w and w+4 share a SIMD)
    const i64 bhk = logical / p.nkb, kb = logical % p.nkb;
    const i64 b = bhk / p.Hk, hk = bhk % p.Hk;
    const i64 lb = p.list_batch == 1 ? 0 : b;
    const int k0 = (int)kb * kKeyBlock, kw0 = k0 + kg * 32;
    const int key = kw0 + l32;

    // The block's K and V rows (past kv_valid: zeros) into LDS.
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int j0 = k0 + 64 * half;
        const int nk = (int)max((i64)0, min((i64)kTile, p.mask.kv_valid - j0));
        tile_issue<D, 8>((const __bf16*)p.k + b * p.k_sB + (i64)j0 * p.k_sL + hk * p.k_sH, p.k_sL, nk,
                         lds_opaque(&side[half * T]));
        tile_issue<D, 8>((const __bf16*)p.v + b * p.v_sB + (i64)j0 * p.v_sL + hk * p.v_sH, p.v_sL, nk,
                         lds_opaque(&side[(2 + half) * T]));
    }
    f32x16 dk[C::NDB], dv[C::NDB];
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) { dk[d] = f32x16{}; dv[d] = f32x16{}; }

    const int m0 = ld_const(p.kfirst, lb * p.nkb + kb), m1 = ld_const(p.klast, lb * p.nkb + kb);
    const unsigned kfb = ~0u;  // no document ids here
    QCursor cur{0, m0 - 1};
    bool have = m0 <= m1 && q_next<false>(p, cur, lb, m0, m1, k0, k0 + kKeyBlock, kfb);
    QHead<D, 8> qh;
    qh.gh = -1;
    if (have) kv_issue8<D>(p, qh, cur, b, hk, lb, lds_opaque(ring[0][0]), lds_opaque(ring[0][1]), lds_opaque(ss0));
    int buf = 0;
    while (have) {
        // This wave's copies of buffer `buf` (and of the key tiles) have
        // landed; after the barrier every wave's have, and every wave is done
        // with the other buffer, which the next tile's copies then fill.
        wait_loads();
        __syncthreads();
        QCursor nxt = cur;
        const bool more = q_next<false>(p, nxt, lb, m0, m1, k0, k0 + kKeyBlock, kfb);
        if (more)
            kv_issue8<D>(p, qh, nxt, b, hk, lb, lds_opaque(ring[buf ^ 1][0]), lds_opaque(ring[buf ^ 1][1]),
                         lds_opaque(ss0 + (buf ^ 1) * 256));
        kv_compute8<D>(p, ring[buf][0], ring[buf][1], ss0 + buf * 256, &side[(kg >> 1) * T], &side[(2 + (kg >> 1)) * T],
                       kg & 1, dk, dv, cur, lb, kw0, rh);
        cur = nxt;
        have = more;
        buf ^= 1;
    }
    // The row-half-1 wave of each key group hands its partial sums to the
    // row-half-0 wave: lane-major, 8 D/32 x 16 floats per lane (32 KB).
    __syncthreads();
    float* red = (float*)(kg < 2 ? &side[kg * 2 * T] : &ring[kg - 2][0][0]);
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
// Copies of query tile c into LDS: Q and dO rows, statistic w by wave w
// (LSE, delta, key interval lo, hi) and, with document ids, the rows' ids
// by every wave (the same bytes, so each wave's count of copies per tile is
// the same).
template <int D>
__device__ inline void kv_issue(const BwdLaunch& p, QHead<D, 4>& x, const QCursor& c, i64 b, i64 hk, i64 lb,
                                int qt, int gt, int st, bool doc) {
    if (c.g != x.gh) qhead_init<D, 4>(p, x, c.g, b, hk, lb);
    stream_issue<D, 4>(x.q, c.m, qt);
    stream_issue<D, 4>(x.g, c.m, gt);
    stat_issue(x.stat, (int)p.Lq, c.m, st + uni(threadIdx.x >> 6) * 256);
    if (doc)
        stat_issue((const float*)(p.mask.ids_q + b * p.mask.lq), (int)p.Lq, c.m, st + 1024);
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
template <int D, bool DOC>
__device__ inline void kv_compute(const BwdLaunch& p, const uint8_t* qt, const uint8_t* gt, const float* st,
                                  const uint4 (&kf)[D / 16], const uint4 (&vf)[D / 16], f32x16 (&dk)[D / 32],
                                  f32x16 (&dv)[D / 32], const QCursor& c, int kw0, int key_id, int key_res,
                                  unsigned dpat, bool masked) {
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
    if (masked && p.mask.dilation > 1) {
#pragma unroll
        for (int rc = 0; rc < 2; ++rc) rbits[rc] = dil_bits(key_res, c.m * kTile + rc * 32, p.mask.dilation, dpat);
    }
    auto slice = [&](const int rc, const int g) __attribute__((always_inline)) {
        const int rb = rc * 32 + 8 * g + 4 * hb;
        const f32x4 L = *(const f32x4*)(st + rb);
        const f32x4 Dl = *(const f32x4*)(st + 64 + rb);
        float pv[4], dv4[4];
        if (masked) {
            const i32x4 lo = *(const i32x4*)(st + 128 + rb);
            const i32x4 hi = *(const i32x4*)(st + 192 + rb);
            i32x4 rid = {0, 0, 0, 0};
            if (DOC) rid = *(const i32x4*)(st + 256 + rb);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bool vis = lo[e] <= key && key < hi[e] && ((rbits[rc] >> (8 * g + 4 * hb + e)) & 1u);
                if (DOC) vis = vis && rid[e] == key_id;
                const float x = pin(__builtin_amdgcn_exp2f(__builtin_fmaf(S[rc][4 * g + e], sc, -L[e] * kLog2e)));
                const float d = pin(x * (G[rc][4 * g + e] - Dl[e]));
                pv[e] = vis ? x : 0.0f;
                dv4[e] = vis ? d : 0.0f;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[rc][4 * g + e], sc, -L[e] * kLog2e));
                dv4[e] = pv[e] * (G[rc][4 * g + e] - Dl[e]);
            }
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

// DOC: document ids (the tile filters apply).
template <int D, int G, bool DOC>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv(const BwdLaunch p) {
    using C = Cfg<D>;
    // Three tile buffers; a tile's copies into LDS are issued two tiles
    // before it is computed.
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
    const int key_id = (DOC && key < p.Lk) ? p.mask.ids_kv[b * p.mask.lk + key] : -1;
    // (key + kv_offset) mod g: the rows congruent to it see the key
    const int key_res = p.mask.dilation > 1
                            ? (int)((((i64)key + p.mask.kv_offset) % p.mask.dilation + p.mask.dilation) % p.mask.dilation)
                            : 0;
    const unsigned dpat = p.mask.dilation > 1 ? dil_pattern(p.mask.dilation) : 0u;
    const unsigned kfw = DOC && kw0 / kTile < p.nkt ? ld_const(p.kbloom, lb * p.nkt + kw0 / kTile) : 0u;
    // whether the wave's keys below kv_valid share one document id (kid_w)
    const int kid_w = uni(key_id);
    const bool kone = DOC && __builtin_amdgcn_ballot_w64(key_in && key_id != kid_w) == 0;
    wait_loads();

    const int m0 = ld_const(p.kfirst, lb * p.nkb + kb), m1 = ld_const(p.klast, lb * p.nkb + kb);
    const unsigned kfb = DOC ? key_block_filter(p, lb, k0) : ~0u;
    QCursor cur{0, m0 - 1};
    bool have = m0 <= m1 && q_next<DOC>(p, cur, lb, m0, m1, k0, k0 + kKeyBlock, kfb);
    // Prologue: copies of the first two tiles.
    constexpr int LOADS = 2 * TileCopy<D, 4>::PER_WAVE + 1;  // per wave and tile, plus the document ids
    const int loads = LOADS + (DOC ? 1 : 0);
    QCursor ahead = cur;  // the last tile whose copies were issued
    bool more = have;
    int n_after = 0;      // tiles issued beyond cur
    QHead<D, 4> qh;
    qh.gh = -1;
    if (have) kv_issue<D>(p, qh, cur, b, hk, lb, lds_opaque(qs[0]), lds_opaque(gs[0]), lds_opaque(ss[0]), DOC);
    if (more) more = q_next<DOC>(p, ahead, lb, m0, m1, k0, k0 + kKeyBlock, kfb);
    if (more) {
        kv_issue<D>(p, qh, ahead, b, hk, lb, lds_opaque(qs[1]), lds_opaque(gs[1]), lds_opaque(ss[1]), DOC);
        ++n_after;
    }
    int buf = 0;
    while (have) {
        // This wave's copies of buffer `buf` have landed; after the barrier
        // every wave's have, and every wave is done with the buffer of the
        // tile before, which takes the copies two tiles ahead.
        wait_vmcnt(n_after * loads);
        __syncthreads();
        const int nb = buf == kRing - 1 ? 0 : buf + 1;
        if (more) more = q_next<DOC>(p, ahead, lb, m0, m1, k0, k0 + kKeyBlock, kfb);
        if (more) {
            const int fb = buf == 0 ? kRing - 1 : buf - 1;
            kv_issue<D>(p, qh, ahead, b, hk, lb, lds_opaque(qs[fb]), lds_opaque(gs[fb]), lds_opaque(ss[fb]), DOC);
            ++n_after;
        }
        // With document ids a wave skips a tile whose filter misses its keys' (a
        // 32-key half of one key tile: that tile's filter).
        if (!DOC || (ld_const(p.qbloom, lb * p.nqt + cur.m) & kfw) != 0) {
            // Document ids: rows all of the document of the wave's keys, every
            // row's interval holding the keys: no element test.
            bool masked = true;
            if (DOC && kone && p.mask.dilation <= 1) {
                const i32x2 qd = ld_const((const i32x2*)p.qdoc, lb * p.nqt + cur.m);
                const i32x4 sm = ld_const((const i32x4*)p.qsum, lb * p.nqt + cur.m);
                masked = !(qd[0] && qd[1] == kid_w && sm[2] <= kw0 && kw0 + 32 <= sm[3]);
            }
            kv_compute<D, DOC>(p, qs[buf], gs[buf], ss[buf], kf, vf, dk, dv, cur, kw0, key_id, key_res, dpat, masked);
        }
        have = q_next<DOC>(p, cur, lb, m0, m1, k0, k0 + kKeyBlock, kfb);
        if (have) --n_after;
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

// The next key tile of the walk whose filter, with document ids, meets the
// filter qf of the block's rows.
__device__ inline bool t_next_doc(const BwdLaunch& p, TCursor& c, int t_lo, int t_hi, i64 lb, unsigned qf) {
    for (;;) {
        if (!t_next(p, c, t_lo, t_hi)) return false;
        if ((ld_const(p.kbloom, lb * p.nkt + c.t) & qf) != 0) return true;
    }
}

template <bool DOC>
__device__ inline bool walk_next(const BwdLaunch& p, TCursor& c, int t_lo, int t_hi, i64 lb, unsigned qf) {
    if constexpr (DOC) return t_next_doc(p, c, t_lo, t_hi, lb, qf);
    else return t_next(p, c, t_lo, t_hi);
}

// One 64-key tile against the wave's 32 rows, with two waves per SIMD (the
// other wave's products cover this one's element-wise work): each 32-key
// half runs its S^T and dP^T products (the two chains alternating), its dS
// and its own dQ^T products in turn, so only one half's scores and dS are
// live.  LDS operand reads run three steps ahead (two with element tests,
// whose registers that takes).  Interleaving one half's element-wise work
// with the other half's products measured slower (the two halves' scores
// then share the registers).
template <int D, bool XM, bool DOC>
__device__ inline void q_compute(const BwdLaunch& p, const uint8_t* kt, const uint8_t* vt, const FragOffs<D>& fo,
                                     const uint4 (&qf)[D / 16], const uint8_t* gw, f32x16 (&dq)[D / 32],
                                     int t, int full_lo, int full_hi, int lo, int hi, float lse2, float delt, i64 b,
                                     int row, int row_id, int row_res, unsigned dpat, bool plain) {
    using C = Cfg<D>;
    constexpr int NS = 2 * C::NDS, NH = 2 * C::NDB, NP = NS + NH;  // steps per half
    constexpr int AH = XM ? 2 : 3;                                  // read-ahead
    const int lane = threadIdx.x & 63, hb = lane >> 5;
    const int j0 = t * kTile;
    // plain: an element-test tile whose every element is visible (one document)
    const bool masked = (XM && !plain) || !(full_lo <= j0 && j0 + kTile <= full_hi);
    const float sc = p.scale * kLog2e;
    static_for<2>([&](auto kbc) {
        constexpr int kb = decltype(kbc)::value;
        // Without element tests dP^T accumulates onto the row's -delta, so it
        // ends as dP - delta (one subtraction per element less).
        const float g0 = XM ? 0.0f : -delt, dsub = XM ? delt : 0.0f;
        f32x16 S = {}, G;
#pragma unroll
        for (int i = 0; i < 16; ++i) G[i] = g0;
        uint4 pd[2];
        // step i: the A operand, and for the dP^T steps dO's fragment as B
        struct Ops {
            uint4 a, b;
        };
        auto ld = [&](const int i) __attribute__((always_inline)) {
            Ops o;
            o.b = uint4{0, 0, 0, 0};
            if (i < NS) {
                if (i & 1) {
                    o.a = frag_rows_at<D>(vt, fo, kb, i >> 1);
                    o.b = frag_rows_at<D>(gw, fo, 0, i >> 1);
                } else {
                    o.a = frag_rows_at<D>(kt, fo, kb, i >> 1);
                }
            } else {
                const int m = i - NS;
                o.a = frag_cols_at<D>(kt, fo, kb * 2 + m / C::NDB, m % C::NDB);
            }
            return o;
        };
        Ops fa[NP];
        static_for<AH>([&](auto ic) { fa[ic.value] = ld(ic.value); });
        static_for<NP>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i + AH < NP) fa[i + AH] = ld(i + AH);
            if constexpr (i < NS) {
                if constexpr (i & 1) G = mfma(fa[i].a, fa[i].b, G);
                else S = mfma(fa[i].a, qf[i >> 1], S);
            } else {
                constexpr int m = i - NS;
                dq[m % C::NDB] = mfma(fa[i].a, pd[m / C::NDB], dq[m % C::NDB]);
            }
            if constexpr (i == NS - 1) {
                // dilated band: the half's keys congruent to row - kv_offset mod g
                unsigned kbits = ~0u;
                if (XM && masked && p.mask.dilation > 1) kbits = dil_bits(row_res, j0 + kb * 32, p.mask.dilation, dpat);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float dsv[4];
                    int kid[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                    if (DOC && masked) key_ids8(p, b, j0 + kb * 32 + 8 * g, kid);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(S[4 * g + e], sc, -lse2));
                        float d = pin(x * (XM ? G[4 * g + e] - dsub : G[4 * g + e]));
                        if (masked) {
                            const int key = j0 + kb * 32 + 8 * g + 4 * hb + e;
                            bool vis = lo <= key && key < hi;
                            if (XM) {
                                vis = vis && ((kbits >> (8 * g + 4 * hb + e)) & 1u);
                                if (DOC) vis = vis && row_id == (hb ? kid[4 + e] : kid[e]);
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

// 32 rows (rows past nvalid read as zero) copied by one wave into LDS in the
// layout of tile_issue (the first half of a 64-row tile).
template <int D>
__device__ inline void rows_issue_wave(const __bf16* base, i64 sL, int nvalid, int lds) {
    constexpr int NCH = Cfg<D>::NCH, RUNS = 32 * D * 2 / 1024;
    const int lane = threadIdx.x & 63;
    const int bytes = uni(nvalid > 0 ? (int)(((i64)(nvalid - 1) * sL + D) * 2) : 0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, kRsrcFlags);
#pragma unroll
    for (int run = 0; run < RUNS; ++run) {
        const int slot = run * 64 + lane, r = slot / NCH, c = bswz<D>(r, slot % NCH);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(uintptr_t)(lds + run * 1024), 16,
                                                 (unsigned)(r * sL * 2 + c * 16), 0, 0, 0);
    }
}

// The dQ kernel's walk over its key tiles: the tile being computed (cur),
// the last one whose copies were issued (ahead), and how many tiles beyond
// cur have copies in flight.
struct DqWalk {
    TCursor cur, ahead;
    bool more;     // ahead is a tile of the walk
    int n_after;   // tiles issued beyond cur
    int t_lo, t_hi;
};

// Copies of key tile t of the key/value head (K and V rows from kbase, vbase).
template <int D, int NW>
__device__ inline void dq_issue(const BwdLaunch& p, const __bf16* kbase, const __bf16* vbase, int t, int kl,
                                int vl) {
    const i64 j0 = (i64)t * kTile;
    const int nk = (int)max((i64)0, min((i64)kTile, p.mask.kv_valid - j0));
    tile_issue<D, NW>(kbase + j0 * p.k_sL, p.k_sL, nk, kl);
    tile_issue<D, NW>(vbase + j0 * p.v_sL, p.v_sL, nk, vl);
}

// XM: element tests; DOC: document ids (with XM; the tile filters apply).
// (XM without DOC: a dilated band.)
// One dQ block of 256 rows (`logical` = (b * H + h) * nqb + position, the
// blocks with the most key tiles first).  LDS: ring[i] holds the K and V
// tiles of ring buffer i; side the block's dO rows (each wave reads its own
// 32 as an operand).  The interval reduction borrows the third ring buffer
// before its first copy.
template <int D, int G, bool XM, int NW, bool DOC>
__device__ __attribute__((always_inline)) inline void dq_block(const BwdLaunch& p, i64 logical, LdsRing<D>& ring,
                                                               LdsSide<D>& gs) {
    using C = Cfg<D>;
    constexpr int RB = NW * 32;  // rows per workgroup
    constexpr int LOADS = 2 * TileCopy<D, NW>::PER_WAVE;
    static_assert(2 * LOADS <= 15, "wait_vmcnt covers at most 15 outstanding copies");
    static_assert(RB * D * 2 <= (int)sizeof(LdsSide<D>), "the block's dO rows fit the side array");
    int* red = (int*)&ring[2][0][0];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hb = lane >> 5;
    const i64 nqb = (p.Lq + RB - 1) / RB;
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
    const int row_id = (DOC && row_ok) ? p.mask.ids_q[b * p.mask.lq + row] : -1;
    // (row - kv_offset) mod g: the keys congruent to it are seen
    const int row_res = (XM && p.mask.dilation > 1)
                            ? (int)((((i64)row - p.mask.kv_offset) % p.mask.dilation + p.mask.dilation) % p.mask.dilation)
                            : 0;
    const unsigned dpat = (XM && p.mask.dilation > 1) ? dil_pattern(p.mask.dilation) : 0u;
    // Q rows of this lane as the B operand: d = ds*16 + hb*8 + 0..7.
    uint4 qf[C::NDS];
    const __bf16* qp = (const __bf16*)p.q + b * p.q_sB + (i64)row * p.q_sL + h * p.q_sH;
#pragma unroll
    for (int ds = 0; ds < C::NDS; ++ds) qf[ds] = row_in ? *(const uint4*)(qp + ds * 16 + hb * 8) : uint4{0, 0, 0, 0};
    // The wave's 32 dO rows (past q_valid: zeros) into its part of gs; only
    // this wave reads them, so its own wait below covers them.
    uint8_t* gw = gs + wave * 32 * (D * 2);
    {
        const i64 r0 = qb * RB + wave * 32;
        const int nrow = (int)max((i64)0, min((i64)32, p.mask.q_valid - r0));
        rows_issue_wave<D>((const __bf16*)p.dout + b * p.do_sB + r0 * p.do_sL + h * p.do_sH, p.do_sL, nrow,
                           lds_opaque(gw));
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

    // Copies run two tiles ahead of the compute.  Each step: wait for this
    // wave's copies of the tile, then at the barrier for every wave's (after
    // which every wave is also done with the previous tile's buffer, the one
    // the next copy overwrites); issue the copies two tiles ahead; compute.
    // Document ids: the filters of the block's rows and of this wave's rows
    // (a 32-row half of one query tile: that tile's filter).
    unsigned qfb = ~0u, qfw = ~0u;
    if (DOC) {
        const i64 m0 = qb * RB / kTile;
        qfb = 0u;
#pragma unroll
        for (int i = 0; i < RB / kTile; ++i)
            if (m0 + i < p.nqt) qfb |= ld_const(p.qbloom, lb * p.nqt + m0 + i);
        const i64 mw = (qb * RB + wave * 32) / kTile;
        qfw = mw < p.nqt ? ld_const(p.qbloom, lb * p.nqt + mw) : 0u;
    }
    // whether the wave's rows below q_valid share one document id (rid_w)
    const int rid_w = uni(row_id);
    const bool rone = DOC && __builtin_amdgcn_ballot_w64(row_in && row_id != rid_w) == 0;
    DqWalk wk;
    wk.t_lo = t_lo;
    wk.t_hi = t_hi;
    const __bf16* kbase = (const __bf16*)p.k + b * p.k_sB + hk * p.k_sH;
    const __bf16* vbase = (const __bf16*)p.v + b * p.v_sB + hk * p.v_sH;
    wk.cur = TCursor{-1, 0};
    bool have = walk_next<DOC>(p, wk.cur, t_lo, t_hi, lb, qfb);
    wk.ahead = wk.cur;
    wk.more = have;
    wk.n_after = 0;
    // (the barrier above: every wave has read red before ring[2] is copied to)
    if (have) dq_issue<D, NW>(p, kbase, vbase, wk.ahead.t, lds_opaque(ring[0][0]), lds_opaque(ring[0][1]));
    if (wk.more) wk.more = walk_next<DOC>(p, wk.ahead, t_lo, t_hi, lb, qfb);
    if (wk.more) {
        dq_issue<D, NW>(p, kbase, vbase, wk.ahead.t, lds_opaque(ring[1][0]), lds_opaque(ring[1][1]));
        ++wk.n_after;
    }
    const FragOffs<D> fo = frag_offsets<D>();
    int buf = 0;
    while (have) {
        wait_vmcnt(wk.n_after * LOADS);
        __syncthreads();
        if (wk.more) wk.more = walk_next<DOC>(p, wk.ahead, t_lo, t_hi, lb, qfb);
        if (wk.more) {
            const int nb = buf == 0 ? 2 : buf - 1;
            dq_issue<D, NW>(p, kbase, vbase, wk.ahead.t, lds_opaque(ring[nb][0]), lds_opaque(ring[nb][1]));
            ++wk.n_after;
        }
        if constexpr (DOC) {
            if ((ld_const(p.kbloom, lb * p.nkt + wk.cur.t) & qfw) != 0) {
                // keys all of the document of the wave's rows (and, tested
                // inside, every row's interval holding them): no element test
                bool plain = false;
                if (rone && p.mask.dilation <= 1) {
                    const i32x2 kd = ld_const((const i32x2*)p.kdoc, lb * p.nkt + wk.cur.t);
                    plain = kd[0] && kd[1] == rid_w;
                }
                q_compute<D, XM, DOC>(p, ring[buf][0], ring[buf][1], fo, qf, gw, dq, wk.cur.t, full_lo, full_hi, lo,
                                      hi, lse2, delt, b, row, row_id, row_res, dpat, plain);
            }
        } else {
            q_compute<D, XM, DOC>(p, ring[buf][0], ring[buf][1], fo, qf, gw, dq, wk.cur.t, full_lo, full_hi, lo, hi,
                                  lse2, delt, b, row, row_id, row_res, dpat, false);
        }
        have = walk_next<DOC>(p, wk.cur, t_lo, t_hi, lb, qfb);
        if (have) --wk.n_after;
        buf = buf == 2 ? 0 : buf + 1;
    }
    if (row_ok) {
        const i64 es = G == BWA_F32 ? 4 : 2;
        char* dqr = (char*)p.dq + (b * p.dq_sB + (i64)row * p.dq_sL + h * p.dq_sH) * es;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) store_tile<G>(dqr, dq[db], db, p.scale);
    }
}

// dQ for masks with element terms (dilated bands, document ids).
template <int D, int G, bool XM, int NW, bool DOC>
__global__ __launch_bounds__(NW * 64, 1) void attn_bwd_dq(const BwdLaunch p) {
    __shared__ __attribute__((aligned(1024))) LdsRing<D> ring;
    __shared__ __attribute__((aligned(1024))) LdsSide<D> side;
    dq_block<D, G, XM, NW, DOC>(p, xcd_remap(blockIdx.x, gridDim.x), ring, side);
}

// dK/dV and dQ of masks without element terms in one launch, as 8-wave
// workgroups on one LDS layout.  Per key/value head group (b, hk), in order:
// the dQ blocks of its query heads, then its dK/dV blocks; each XCD takes a
// contiguous range of that order, so a workgroup that finishes early takes
// the next block of either kind (two launches leave compute units idle at the
// end of the first when its blocks differ in length, as a window's do), and
// both kinds of one head group share the XCD's L2.
template <int D, int G>
__global__ __launch_bounds__(512, 1) void attn_bwd_fused(const BwdLaunch p) {
    __shared__ __attribute__((aligned(1024))) LdsRing<D> ring;
    __shared__ __attribute__((aligned(1024))) LdsSide<D> side;
    const i64 nqb = (p.Lq + 255) / 256;
    const i64 nq = (i64)p.kv_group * nqb, per = nq + p.nkb;
    const i64 logical = xcd_remap(blockIdx.x, gridDim.x);
    const i64 g = logical / per, r = logical % per;  // g = b * Hk + hk
    if (r < nq) {
        const i64 b = g / p.Hk, hk = g % p.Hk, h = hk * p.kv_group + r / nqb;
        dq_block<D, G, false, 8, false>(p, (b * p.H + h) * nqb + r % nqb, ring, side);
    } else {
        dkdv8_block<D, G>(p, g * p.nkb + (r - nq), ring, side);
    }
}

template <int D, int G>
hipError_t launch_dg(const BwdLaunch& a, hipStream_t stream) {
    const bool doc = a.mask.seg_mode == 3, xm = a.mask.dilation > 1 || doc;
    constexpr int NW = kDqWaves;
    static_assert(NW == 8, "the fused launch runs 8-wave dQ blocks");
    const i64 nqb = (a.Lq + 32 * NW - 1) / (32 * NW);
    if (!xm) {
        // interval masks: dK/dV and dQ blocks in one launch, two waves per SIMD
        const i64 n = (i64)a.B * a.Hk * ((i64)a.kv_group * nqb + a.nkb);
        if (n > 0) hipLaunchKernelGGL((attn_bwd_fused<D, G>), dim3((unsigned)n), dim3(512), 0, stream, a);
        return hipGetLastError();
    }
    // element masks: dK/dV with one wave per SIMD, then dQ
    const i64 nkb_total = (i64)a.B * a.Hk * a.nkb;
    if (nkb_total > 0) {
        if (doc) hipLaunchKernelGGL((attn_bwd_dkdv<D, G, true>), dim3((unsigned)nkb_total), dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((attn_bwd_dkdv<D, G, false>), dim3((unsigned)nkb_total), dim3(256), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const i64 nqb_total = (i64)a.B * a.H * nqb;
    if (nqb_total > 0) {
        if (doc)
            hipLaunchKernelGGL((attn_bwd_dq<D, G, true, NW, true>), dim3((unsigned)nqb_total), dim3(64 * NW), 0, stream, a);
        else
            hipLaunchKernelGGL((attn_bwd_dq<D, G, true, NW, false>), dim3((unsigned)nqb_total), dim3(64 * NW), 0, stream, a);
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
    if (a.mask.seg_mode == 3 && a.list_batch * a.nkt > 0)
        hipLaunchKernelGGL(bwd_ktiles_kernel, dim3((unsigned)(a.list_batch * a.nkt)), dim3(64), 0, stream, a);
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

namespace {
__global__ __launch_bounds__(256) void lse_gather_kernel(const float* src, float* dst, i64 H, i64 Lq, int g) {
    const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;  // over H * Lq, in dst order
    if (i >= H * Lq) return;
    const i64 n = Lq / g, r = i / (H * n), rest = i % (H * n), h = rest / n, a = rest % n;
    dst[i] = src[h * Lq + r + (i64)g * a];
}
}  // namespace

hipError_t launch_lse_gather(const float* src, float* dst, i64 H, i64 Lq, int g, hipStream_t stream) {
    const i64 n = H * Lq;
    if (n > 0) hipLaunchKernelGGL(lse_gather_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, src, dst, H, Lq, g);
    return hipGetLastError();
}

static i64 pad256(i64 x) { return (x + 255) / 256 * 256; }

i64 bwd_workspace_bytes(i64 B, i64 H, i64 Lq, i64 Lk, i64 list_batch) {
    const i64 nqt = (Lq + kTile - 1) / kTile, nkb = (Lk + kKeyBlock - 1) / kKeyBlock;
    const i64 nkt = (Lk + kTile - 1) / kTile;
    return pad256(B * H * Lq * 4) + 2 * pad256(list_batch * Lq * 4) + pad256(list_batch * nqt * 16) +
           2 * pad256(list_batch * nkb * 4) + pad256(list_batch * nqt * 4) + pad256(list_batch * nkt * 4) +
           pad256(list_batch * nqt * 8) + pad256(list_batch * nkt * 8);
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
    a.klast = (int*)w; w += pad256(a.list_batch * a.nkb * 4);
    a.qbloom = (unsigned*)w; w += pad256(a.list_batch * a.nqt * 4);
    a.kbloom = (unsigned*)w; w += pad256(a.list_batch * a.nkt * 4);
    a.qdoc = (int*)w; w += pad256(a.list_batch * a.nqt * 8);
    a.kdoc = (int*)w;
}

}  // namespace bwa
