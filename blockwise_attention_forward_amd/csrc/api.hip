// C ABI entry points: argument validation on the host, then one or more
// asynchronous launches on the caller's stream.  Nothing here allocates
// device memory, synchronises or keeps state between calls (the last-error
// string is thread-local; the allocation-free balanced launch caches the
// address of its static scratch per device).

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>

#include "internal.h"

using bwa::i64;

namespace {

thread_local char g_last_error[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return code;
}

int32_t ok() {
    g_last_error[0] = '\0';
    return BWA_OK;
}

int32_t hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(BWA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

constexpr i64 kMaxLen = (i64)1 << 30;  // positions are kept in int32 inside the kernels
constexpr i64 kMaxRowStride = (i64)1 << 24;

int elem_size(int32_t dt) { return dt == BWA_BF16 ? 2 : 4; }

int32_t check_tensor(const bwa_tensor* t, const char* name) {
    if (!t) return fail(BWA_ERR_NULL_ARG, "%s: tensor descriptor is NULL", name);
    if (t->dtype != BWA_F32 && t->dtype != BWA_BF16)
        return fail(BWA_ERR_BAD_DTYPE, "%s: unknown dtype code %d", name, t->dtype);
    if (t->B < 0 || t->L < 0 || t->H < 0 || t->D < 0)
        return fail(BWA_ERR_BAD_SHAPE, "%s: negative size", name);
    if (t->L > kMaxLen) return fail(BWA_ERR_UNSUPPORTED, "%s: L=%lld exceeds 2^30", name, (long long)t->L);
    if (t->D != 64 && t->D != 128)
        return fail(BWA_ERR_UNSUPPORTED, "%s: head dim %lld (supported: 64, 128)", name, (long long)t->D);
    const i64 n = t->B * t->L * t->H;
    if (n == 0) return BWA_OK;
    if (!t->ptr) return fail(BWA_ERR_NULL_ARG, "%s: data pointer is NULL", name);
    const i64 es = elem_size(t->dtype);
    if (((uintptr_t)t->ptr) % 16) return fail(BWA_ERR_BAD_STRIDE, "%s: pointer not 16-byte aligned", name);
    if ((t->sB * es) % 16 || (t->sL * es) % 16 || (t->sH * es) % 16)
        return fail(BWA_ERR_BAD_STRIDE, "%s: strides must be multiples of 16 bytes", name);
    if (t->sB < 0 || t->sL < 0 || t->sH < 0) return fail(BWA_ERR_BAD_STRIDE, "%s: negative stride", name);
    // A tile copy addresses up to 64 rows from one base with 32-bit byte
    // offsets: row strides stay below 2^24 elements.
    if (t->sL >= kMaxRowStride)
        return fail(BWA_ERR_BAD_STRIDE, "%s: row stride of %lld elements (limit 2^24)", name, (long long)t->sL);
    // No two (b, l, h) rows may share an element: broadcast views (a zero
    // stride) and strides that interleave rows are rejected.  Sufficient
    // test: taken by increasing stride, each dimension of extent > 1 steps
    // past everything the dimensions inside it span.
    struct Dim { i64 n, s; } dims[3] = {{t->B, t->sB}, {t->L, t->sL}, {t->H, t->sH}};
    std::sort(dims, dims + 3, [](const Dim& a, const Dim& b) { return a.s < b.s; });
    i64 span = t->D;  // elements one row covers
    for (const Dim& d : dims) {
        if (d.n <= 1) continue;
        if (d.s < span)
            return fail(BWA_ERR_BAD_STRIDE, "%s: overlapping layout (stride %lld over an extent of %lld elements)",
                        name, (long long)d.s, (long long)span);
        span = d.s * (d.n - 1) + span;
    }
    return BWA_OK;
}

// Resolve and validate a mask for a [B, lq] x [B, lk] problem.
int32_t resolve_mask(const bwa_mask* m, i64 B, i64 lq, i64 lk, bwa::MaskDev& out) {
    if (!m) return fail(BWA_ERR_NULL_ARG, "mask is NULL");
    if (m->causal != 0 && m->causal != 1) return fail(BWA_ERR_BAD_MASK, "causal must be 0 or 1");
    if (m->window < 0) return fail(BWA_ERR_BAD_MASK, "window must be >= 0");
    if (m->dilation < 0) return fail(BWA_ERR_BAD_MASK, "dilation must be >= 0");
    if (m->dilation > 1 && (!m->causal || m->window <= 0))
        return fail(BWA_ERR_BAD_MASK, "a dilated band needs causal = 1 and a window");
    if (m->prefix < 0) return fail(BWA_ERR_BAD_MASK, "prefix must be >= 0");
    if (m->prefix > 0 && (!m->causal || m->window > 0))
        return fail(BWA_ERR_BAD_MASK, "a prefix needs causal = 1 and no window");
    if (m->prefix > kMaxLen) return fail(BWA_ERR_BAD_MASK, "prefix out of range");
    if (m->documents != 0 && m->documents != 1) return fail(BWA_ERR_BAD_MASK, "documents must be 0 or 1");
    if (m->documents && !m->segment_ids_q) return fail(BWA_ERR_BAD_MASK, "documents needs segment ids");
    if (m->q_valid > lq) return fail(BWA_ERR_BAD_MASK, "q_valid %lld > Lq %lld", (long long)m->q_valid, (long long)lq);
    if (m->kv_valid > lk) return fail(BWA_ERR_BAD_MASK, "kv_valid %lld > Lk %lld", (long long)m->kv_valid, (long long)lk);
    if (m->kv_offset > kMaxLen || m->kv_offset < -kMaxLen)
        return fail(BWA_ERR_BAD_MASK, "kv_offset out of range");
    const bool cu = m->cu_seqlens_q != nullptr;
    const bool ids = m->segment_ids_q != nullptr;
    if (cu && ids) return fail(BWA_ERR_BAD_MASK, "give cu_seqlens or segment ids, not both");
    if (!cu && m->cu_seqlens_kv) return fail(BWA_ERR_BAD_MASK, "cu_seqlens_kv given without cu_seqlens_q");
    if (!ids && m->segment_ids_kv) return fail(BWA_ERR_BAD_MASK, "segment_ids_kv given without segment_ids_q");
    if (cu && m->num_segments <= 0) return fail(BWA_ERR_BAD_MASK, "cu_seqlens needs num_segments >= 1");
    if (!cu && m->num_segments != 0) return fail(BWA_ERR_BAD_MASK, "num_segments without cu_seqlens");
    if (ids && !m->segment_ids_kv && lq != lk)
        return fail(BWA_ERR_BAD_MASK, "segment_ids_kv may be omitted only when Lq == Lk");
    out.lq = lq;
    out.lk = lk;
    out.kv_offset = m->kv_offset;
    out.q_valid = m->q_valid < 0 ? lq : m->q_valid;
    out.kv_valid = m->kv_valid < 0 ? lk : m->kv_valid;
    out.causal = m->causal;
    out.window = m->window;
    out.dilation = m->dilation > 1 ? m->dilation : 1;
    out.prefix = m->prefix;
    out.seg_mode = cu ? 1 : (ids ? (m->documents ? 3 : 2) : 0);
    out.num_segments = cu ? m->num_segments : 0;
    out.cu_q = m->cu_seqlens_q;
    out.cu_kv = m->cu_seqlens_kv ? m->cu_seqlens_kv : m->cu_seqlens_q;
    out.ids_q = m->segment_ids_q;
    out.ids_kv = m->segment_ids_kv ? m->segment_ids_kv : m->segment_ids_q;
    (void)B;
    return BWA_OK;
}

}  // namespace

extern "C" {

const char* bwa_status_string(int32_t s) {
    switch (s) {
        case BWA_OK: return "ok";
        case BWA_ERR_NULL_ARG: return "null argument";
        case BWA_ERR_BAD_SHAPE: return "bad shape";
        case BWA_ERR_BAD_STRIDE: return "bad stride or alignment";
        case BWA_ERR_BAD_DTYPE: return "bad dtype";
        case BWA_ERR_BAD_MASK: return "bad mask";
        case BWA_ERR_UNSUPPORTED: return "unsupported";
        case BWA_ERR_CAPACITY: return "list capacity too small";
        case BWA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* bwa_last_error(void) { return g_last_error; }

int32_t bwa_version(void) { return BWATTN_VERSION; }

int32_t bwa_attn_tile(int32_t dtype, int64_t D, int32_t* bq, int32_t* bkv) {
    if (!bq || !bkv) return fail(BWA_ERR_NULL_ARG, "bq/bkv output is NULL");
    if (dtype != BWA_F32 && dtype != BWA_BF16) return fail(BWA_ERR_BAD_DTYPE, "unknown dtype %d", dtype);
    if (D != 64 && D != 128) return fail(BWA_ERR_UNSUPPORTED, "head dim %lld", (long long)D);
    *bq = bwa::attn_rows_per_block(dtype, (int)D);
    *bkv = 64;
    return ok();
}

int32_t bwa_block_mask_size(const bwa_mask* mask, int64_t B, int64_t lq, int64_t lk, int32_t bq,
                            int32_t bkv, int64_t* n_qblocks, int64_t* capacity, int64_t* list_batch) {
    if (!n_qblocks || !capacity || !list_batch) return fail(BWA_ERR_NULL_ARG, "size outputs are NULL");
    if (B < 0 || lq < 0 || lk < 0) return fail(BWA_ERR_BAD_SHAPE, "negative size");
    if (lq > kMaxLen || lk > kMaxLen) return fail(BWA_ERR_UNSUPPORTED, "length exceeds 2^30");
    if (bq <= 0 || bkv <= 0 || bq % 64 || bkv % 64 || bq > 512)
        return fail(BWA_ERR_BAD_SHAPE, "bq and bkv must be positive multiples of 64 (bq <= 512)");
    bwa::MaskDev md;
    int32_t st = resolve_mask(mask, B, lq, lk, md);
    if (st) return st;
    const i64 nqb = (lq + bq - 1) / bq, nkb = (lk + bkv - 1) / bkv;
    // runs per query block: at most 3 for one interval per row, bq + 2 for
    // segments (a run pair per segment the block meets), and for dilated
    // bands and document ids (exact classification) any number up to nkb
    const bool exact = md.dilation > 1 || md.seg_mode == 3;
    const i64 per = exact ? nkb : (md.seg_mode ? std::min<i64>(nkb, (i64)bq + 2) : std::min<i64>(nkb, 3));
    *n_qblocks = nqb;
    *capacity = std::max<i64>(nqb * per, 1);
    *list_batch = md.seg_mode >= 2 ? B : 1;
    return ok();
}

int32_t bwa_block_mask_build(const bwa_mask* mask, int64_t B, int64_t lq, int64_t lk, bwa_blocks* out,
                             void* stream) {
    if (!out) return fail(BWA_ERR_NULL_ARG, "blocks output is NULL");
    i64 nqb, cap, lb;
    int32_t st = bwa_block_mask_size(mask, B, lq, lk, out->bq, out->bkv, &nqb, &cap, &lb);
    if (st) return st;
    if (out->lq != lq || out->lk != lk || out->n_qblocks != nqb || out->batch != lb)
        return fail(BWA_ERR_BAD_SHAPE, "blocks descriptor does not match (lq, lk, n_qblocks, batch)");
    if (out->capacity < cap)
        return fail(BWA_ERR_CAPACITY, "capacity %lld < required %lld", (long long)out->capacity, (long long)cap);
    if (!out->row_ptr || !out->run_begin || !out->run_end || !out->run_kind || (lq > 0 && (!out->row_lo || !out->row_hi)))
        return fail(BWA_ERR_NULL_ARG, "blocks arrays must be non-NULL");
    // One work-item per (copy, row) and one wave per (copy, q-block): under 2^32 work-items per launch.
    if (lb * lq >= ((i64)1 << 32) - 256) return fail(BWA_ERR_UNSUPPORTED, "block list grid too large");
    bwa::BlocksLaunch a;
    resolve_mask(mask, B, lq, lk, a.mask);
    a.copies = lb;
    a.bq = out->bq;
    a.bkv = out->bkv;
    a.n_qblocks = nqb;
    a.capacity = out->capacity;
    a.row_ptr = out->row_ptr;
    a.run_begin = out->run_begin;
    a.run_end = out->run_end;
    a.run_kind = out->run_kind;
    a.row_lo = out->row_lo;
    a.row_hi = out->row_hi;
    return hip_status(bwa::launch_block_mask_build(a, (hipStream_t)stream), "block_mask_build launch");
}

int32_t bwa_fixed_m_bound(const bwa_tensor* q, const bwa_tensor* k_chunks, int32_t n_chunks,
                          const float* kmax_in, int32_t n_kmax_in, const int64_t* kv_valid, int64_t q_valid,
                          float scale,
                          float tau, float* kmax_out, float* mmax_out, float* m_out, uint8_t* gate_out,
                          void* stream) {
    int32_t st = check_tensor(q, "q");
    if (st) return st;
    if (n_chunks < 0 || n_chunks > bwa::kMaxChunks)
        return fail(BWA_ERR_BAD_SHAPE, "n_chunks must be in [0, %d]", bwa::kMaxChunks);
    if (n_chunks > 0 && !k_chunks) return fail(BWA_ERR_NULL_ARG, "k_chunks is NULL");
    if (q_valid > q->L) return fail(BWA_ERR_BAD_SHAPE, "q_valid > Lq");
    if (n_kmax_in < 0) return fail(BWA_ERR_BAD_SHAPE, "n_kmax_in < 0");
    if (n_kmax_in > 0 && !kmax_in) return fail(BWA_ERR_NULL_ARG, "kmax_in is NULL with n_kmax_in > 0");
    const i64 BH = q->B * q->H;
    if (BH > 0 && (!kmax_out || !mmax_out || !gate_out || (q->L > 0 && !m_out)))
        return fail(BWA_ERR_NULL_ARG, "bound outputs must be non-NULL");
    bwa::BoundLaunch a;
    a.Hk = n_chunks > 0 ? (int)k_chunks[0].H : (int)q->H;
    a.q = {q->ptr, q->L, q->sB, q->sL, q->sH, q_valid < 0 ? q->L : q_valid};
    for (int c = 0; c < n_chunks; ++c) {
        const bwa_tensor* k = &k_chunks[c];
        char name[32];
        snprintf(name, sizeof(name), "k_chunks[%d]", c);
        st = check_tensor(k, name);
        if (st) return st;
        if (k->dtype != q->dtype || k->B != q->B || k->D != q->D || k->H != a.Hk)
            return fail(BWA_ERR_BAD_SHAPE, "%s: dtype/B/D differ from q, or heads from k_chunks[0]", name);
        if (q->H > 0 && (k->H <= 0 || q->H % k->H))
            return fail(BWA_ERR_BAD_SHAPE, "%s: %lld key heads do not divide %lld query heads", name,
                        (long long)k->H, (long long)q->H);
        i64 valid = k->L;
        if (kv_valid && kv_valid[c] >= 0) {
            if (kv_valid[c] > k->L) return fail(BWA_ERR_BAD_SHAPE, "%s: kv_valid > L", name);
            valid = kv_valid[c];
        }
        a.k[c] = {k->ptr, k->L, k->sB, k->sL, k->sH, valid};
    }
    a.n_chunks = n_chunks;
    a.B = (int)q->B;
    a.H = (int)q->H;
    a.D = (int)q->D;
    a.dtype = q->dtype;
    a.kmax_in = n_kmax_in > 0 ? kmax_in : nullptr;
    a.n_kmax_in = n_kmax_in;
    a.scale = scale;
    a.tau = tau;
    a.kmax_out = kmax_out;
    a.mmax_out = mmax_out;
    a.m_out = m_out;
    a.gate_out = gate_out;
    return hip_status(bwa::launch_fixed_m_bound(a, (hipStream_t)stream), "fixed_m_bound launch");
}

// Balanced launch request: workgroups (one per compute unit, resolved) and workspace.
struct Balance {
    int32_t n_cus;
    void* ws;
    int64_t ws_bytes;
};

static constexpr int32_t kMaxPlannedCus = 1 << 16;

// Compute units of the current device (the balanced launch's default).
static int32_t device_cus(int32_t* n) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(BWA_ERR_HIP, "compute unit count: %s", hipGetErrorString(e));
    return BWA_OK;
}

static int32_t resolve_cus(int32_t n_cus, int32_t* out) {
    if (n_cus > kMaxPlannedCus) return fail(BWA_ERR_UNSUPPORTED, "n_cus %d > %d", n_cus, kMaxPlannedCus);
    int32_t st;
    if (n_cus <= 0 && (st = device_cus(&n_cus))) return st;
    *out = n_cus;
    return BWA_OK;
}

// A dilated band (causal, window W, dilation g, kv_offset a multiple of g) is
// g independent causal windows: row i = r + g a sees key j exactly when
// j = r + g c with c <= a + kv_offset / g and a + kv_offset / g - c <
// ceil(W / g).  When the lengths, kv_offset and the valid counts are
// multiples of g, each batch element runs as one launch whose batch index is
// the residue r, on strided views of q, k, v, o and lse: every key it
// computes is visible, where the band's own walk computes g keys per visible
// one.  Other dilated calls (and fixed-m modes, carried partials and
// segments) take the element-test kernels.
static bool band_splits(const bwa::MaskDev& m, i64 Lq, i64 Lk) {
    const i64 g = m.dilation;
    return g > 1 && m.seg_mode == 0 && m.prefix == 0 && m.causal && m.window > 0 && Lq % g == 0 && Lk % g == 0 &&
           m.kv_offset % g == 0 && m.q_valid % g == 0 && m.kv_valid % g == 0;
}

// The mask of each residue class's window.
static bwa::MaskDev band_window(const bwa::MaskDev& m, i64 Lq, i64 Lk) {
    const i64 g = m.dilation;
    bwa::MaskDev s = m;
    s.lq = Lq / g;
    s.lk = Lk / g;
    s.kv_offset = m.kv_offset / g;
    s.q_valid = m.q_valid / g;
    s.kv_valid = m.kv_valid / g;
    s.window = (int)((m.window + g - 1) / g);
    s.dilation = 1;
    return s;
}

static bool dilated_as_windows(const bwa::AttnLaunch& a) {
    return band_splits(a.mask, a.Lq, a.Lk) && a.mode == BWA_MODE_ONLINE && !a.lse_prev && !a.split_next;
}

static hipError_t launch_dilated(const bwa::AttnLaunch& a, int32_t bq, hipStream_t stream) {
    const i64 g = a.mask.dilation;
    const i64 ei = a.in_dtype == BWA_BF16 ? 2 : 4, eo = a.out_dtype == BWA_BF16 ? 2 : 4;
    for (i64 b = 0; b < a.B; ++b) {
        bwa::AttnLaunch s = a;
        s.B = (int)g;
        s.Lq = a.Lq / g;
        s.Lk = a.Lk / g;
        s.q = (const char*)a.q + b * a.q_sB * ei; s.q_sB = a.q_sL; s.q_sL = a.q_sL * g;
        s.k = (const char*)a.k + b * a.k_sB * ei; s.k_sB = a.k_sL; s.k_sL = a.k_sL * g;
        s.v = (const char*)a.v + b * a.v_sB * ei; s.v_sB = a.v_sL; s.v_sL = a.v_sL * g;
        s.o = (char*)a.o + b * a.o_sB * eo; s.o_sB = a.o_sL; s.o_sL = a.o_sL * g;
        s.lse = a.lse + b * a.lse_sB; s.lse_sB = a.lse_sL; s.lse_sL = a.lse_sL * g;
        s.mask = band_window(a.mask, a.Lq, a.Lk);
        s.have_blocks = 0;  // the walk follows the window inline
        s.n_qblocks = (s.Lq + bq - 1) / bq;
        const hipError_t e = bwa::launch_attn_fwd(s, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

static int32_t attn_fwd_impl(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v, const bwa_mask* mask,
                             const bwa_blocks* blocks, float scale, int32_t mode, const float* m,
                             const uint8_t* gate, const bwa_tensor* o_prev, const float* lse_prev, bwa_tensor* o,
                             float* lse, void* stream, const Balance* bal = nullptr) {
    int32_t st;
    if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) ||
        (st = check_tensor(o, "o")))
        return st;
    if (k->dtype != q->dtype || v->dtype != q->dtype)
        return fail(BWA_ERR_BAD_DTYPE, "q, k and v must share a dtype");
    if (o->dtype != BWA_F32 && o->dtype != q->dtype)
        return fail(BWA_ERR_BAD_DTYPE, "o must be fp32 or q's dtype");
    if (k->B != q->B || v->B != q->B || k->D != q->D || v->D != q->D || v->H != k->H)
        return fail(BWA_ERR_BAD_SHAPE, "q, k, v disagree on B or D, or k and v on H");
    if (q->H > 0 && (k->H <= 0 || q->H % k->H))
        return fail(BWA_ERR_BAD_SHAPE, "%lld key/value heads do not divide %lld query heads", (long long)k->H,
                    (long long)q->H);
    if (k->L != v->L) return fail(BWA_ERR_BAD_SHAPE, "k and v lengths differ");
    if (o->B != q->B || o->L != q->L || o->H != q->H || o->D != q->D)
        return fail(BWA_ERR_BAD_SHAPE, "o must have q's shape");
    if (mode != BWA_MODE_ONLINE && mode != BWA_MODE_FIXED_M && mode != BWA_MODE_GATED)
        return fail(BWA_ERR_BAD_SHAPE, "unknown mode %d", mode);
    const i64 B = q->B, H = q->H, Lq = q->L, Lk = k->L;
    const i64 rows = B * H * Lq;
    if (rows > 0 && !lse) return fail(BWA_ERR_NULL_ARG, "lse is NULL");
    if (mode != BWA_MODE_ONLINE && rows > 0 && !m) return fail(BWA_ERR_NULL_ARG, "fixed-m and gated modes need m");
    if (mode == BWA_MODE_GATED && rows > 0 && !gate) return fail(BWA_ERR_NULL_ARG, "gated mode needs gate");
    bwa::AttnLaunch a;
    memset(&a, 0, sizeof(a));
    if ((st = resolve_mask(mask, B, Lq, Lk, a.mask))) return st;
    int32_t bq, bkv;
    bwa_attn_tile(q->dtype, q->D, &bq, &bkv);
    if (blocks) {
        if (blocks->bq != bq || blocks->bkv <= 0 || blocks->bkv % bkv)
            return fail(BWA_ERR_BAD_SHAPE, "blocks built with bq=%d bkv=%d; need bq=%d, bkv a multiple of %d",
                        blocks->bq, blocks->bkv, bq, bkv);
        if (blocks->lq != Lq || blocks->lk != Lk || blocks->n_qblocks != (Lq + bq - 1) / bq)
            return fail(BWA_ERR_BAD_SHAPE, "blocks describe a different problem size");
        if (blocks->batch != 1 && blocks->batch != B) return fail(BWA_ERR_BAD_SHAPE, "blocks batch must be 1 or B");
        if (a.mask.seg_mode >= 2 && blocks->batch != B)
            return fail(BWA_ERR_BAD_SHAPE, "per-token segment ids need one list copy per batch element");
        if (!blocks->row_ptr || !blocks->run_begin || !blocks->run_end || !blocks->run_kind ||
            (Lq > 0 && (!blocks->row_lo || !blocks->row_hi)))
            return fail(BWA_ERR_NULL_ARG, "blocks arrays must be non-NULL");
        a.have_blocks = 1;
        a.row_ptr = blocks->row_ptr;
        a.run_begin = blocks->run_begin;
        a.run_end = blocks->run_end;
        a.run_kind = blocks->run_kind;
        a.row_lo = blocks->row_lo;
        a.row_hi = blocks->row_hi;
        a.list_batch = blocks->batch;
        a.capacity = blocks->capacity;
        a.bkv_list = blocks->bkv;
    }
    // One workgroup of up to 512 work-items per (b, h, q-block); a launch holds under 2^32 work-items.
    if (B * H * ((Lq + bq - 1) / bq) >= ((i64)1 << 23)) return fail(BWA_ERR_UNSUPPORTED, "grid too large");
    a.q = q->ptr; a.k = k->ptr; a.v = v->ptr;
    a.q_sB = q->sB; a.q_sL = q->sL; a.q_sH = q->sH;
    a.k_sB = k->sB; a.k_sL = k->sL; a.k_sH = k->sH;
    a.v_sB = v->sB; a.v_sL = v->sL; a.v_sH = v->sH;
    a.o = o->ptr; a.o_sB = o->sB; a.o_sL = o->sL; a.o_sH = o->sH;
    a.lse = lse;
    a.lse_sB = H * Lq; a.lse_sH = Lq; a.lse_sL = 1;
    a.B = (int)B; a.H = (int)H; a.D = (int)q->D;
    a.kv_group = H > 0 ? (int)(H / k->H) : 1;
    a.Lq = Lq; a.Lk = Lk;
    a.in_dtype = q->dtype;
    a.out_dtype = o->dtype;
    a.scale = scale;
    a.mode = mode;
    a.m = m;
    a.gate = gate;
    a.n_qblocks = (Lq + bq - 1) / bq;
    if (o_prev) {
        if ((st = check_tensor(o_prev, "o_prev"))) return st;
        if (o_prev->dtype != BWA_F32) return fail(BWA_ERR_BAD_DTYPE, "o_prev must be fp32");
        if (o_prev->B != q->B || o_prev->L != q->L || o_prev->H != q->H || o_prev->D != q->D)
            return fail(BWA_ERR_BAD_SHAPE, "o_prev must have q's shape");
        if (rows > 0 && !lse_prev) return fail(BWA_ERR_NULL_ARG, "lse_prev is NULL");
        if (o_prev->ptr == o->ptr &&
            (o->dtype != BWA_F32 || o_prev->sB != o->sB || o_prev->sL != o->sL || o_prev->sH != o->sH))
            return fail(BWA_ERR_BAD_STRIDE, "o may alias o_prev only as the same fp32 tensor (same strides)");
        a.o_prev = (const float*)o_prev->ptr;
        a.op_sB = o_prev->sB; a.op_sL = o_prev->sL; a.op_sH = o_prev->sH;
        a.lse_prev = rows > 0 ? lse_prev : nullptr;
    }
    if (bal) {
        if (q->dtype != BWA_BF16) return fail(BWA_ERR_UNSUPPORTED, "the balanced launch computes bf16 inputs only");
        if (a.mask.dilation > 1 || a.mask.seg_mode == 3)
            return fail(BWA_ERR_UNSUPPORTED, "the balanced launch takes no dilated bands or document ids");
        const i64 units = B * H * a.n_qblocks;
        const bwa::SplitPlan sp = bwa::split_plan(units, bal->n_cus, Lk);
        const i64 need = bwa::split_workspace_bytes(sp, bq, (int)q->D);
        if (units > 0) {
            if (!bal->ws) return fail(BWA_ERR_NULL_ARG, "workspace is NULL");
            if ((uintptr_t)bal->ws % 256) return fail(BWA_ERR_BAD_STRIDE, "workspace not 256-byte aligned");
            if (bal->ws_bytes < need)
                return fail(BWA_ERR_CAPACITY, "workspace of %lld bytes; %lld needed", (long long)bal->ws_bytes,
                            (long long)need);
            bwa::split_workspace_layout(a, bal->ws, sp, bq, (int)q->D);
        }
    }
    if (dilated_as_windows(a)) return hip_status(launch_dilated(a, bq, (hipStream_t)stream), "attn_fwd launch");
    return hip_status(bwa::launch_attn_fwd(a, (hipStream_t)stream), "attn_fwd launch");
}

int32_t bwa_attn_fwd(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v, const bwa_mask* mask,
                     const bwa_blocks* blocks, float scale, int32_t mode, const float* m,
                     const uint8_t* gate, bwa_tensor* o, float* lse, void* stream) {
    return attn_fwd_impl(q, k, v, mask, blocks, scale, mode, m, gate, nullptr, nullptr, o, lse, stream);
}

int32_t bwa_attn_fwd_carry(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v, const bwa_mask* mask,
                           const bwa_blocks* blocks, float scale, int32_t mode, const float* m,
                           const uint8_t* gate, const bwa_tensor* o_prev, const float* lse_prev, bwa_tensor* o,
                           float* lse, void* stream) {
    if (!o_prev) return fail(BWA_ERR_NULL_ARG, "o_prev is NULL");
    return attn_fwd_impl(q, k, v, mask, blocks, scale, mode, m, gate, o_prev, lse_prev, o, lse, stream);
}

int32_t bwa_attn_fwd_balanced_workspace(int32_t dtype, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                                        int32_t n_cus, int64_t* bytes, int64_t* cut_blocks, int32_t* pieces) {
    if (!bytes) return fail(BWA_ERR_NULL_ARG, "bytes output is NULL");
    if (B < 0 || H < 0 || Lq < 0 || Lk < 0) return fail(BWA_ERR_BAD_SHAPE, "negative size");
    int32_t bq, bkv, st;
    if ((st = bwa_attn_tile(dtype, D, &bq, &bkv))) return st;
    if ((st = resolve_cus(n_cus, &n_cus))) return st;
    const i64 units = B * H * ((Lq + bq - 1) / bq);
    const bwa::SplitPlan sp = bwa::split_plan(units, n_cus, Lk);
    *bytes = units > 0 ? bwa::split_workspace_bytes(sp, bq, (int)D) : 0;
    if (cut_blocks) *cut_blocks = units > 0 ? sp.tail : 0;
    if (pieces) *pieces = sp.s;
    return ok();
}

int32_t bwa_attn_fwd_balanced(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v, const bwa_mask* mask,
                              const bwa_blocks* blocks, float scale, int32_t mode, const float* m,
                              const uint8_t* gate, int32_t n_cus, void* workspace, int64_t workspace_bytes,
                              bwa_tensor* o, float* lse, void* stream) {
    Balance bal;
    int32_t st;
    if ((st = resolve_cus(n_cus, &bal.n_cus))) return st;
    bal.ws = workspace;
    bal.ws_bytes = workspace_bytes;
    return attn_fwd_impl(q, k, v, mask, blocks, scale, mode, m, gate, nullptr, nullptr, o, lse, stream, &bal);
}

int32_t bwa_attn_fwd_balanced_noalloc(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v,
                                      const bwa_mask* mask, const bwa_blocks* blocks, float scale, int32_t mode,
                                      const float* m, const uint8_t* gate, int32_t n_cus, bwa_tensor* o, float* lse,
                                      void* stream) {
    Balance bal;
    int32_t st;
    if ((st = resolve_cus(n_cus, &bal.n_cus))) return st;
    // The plan's workspace must fit the static scratch; checked before any
    // launch (shapes as validated again by attn_fwd_impl).
    if (q && k && q->dtype == BWA_BF16 && (q->D == 64 || q->D == 128) && q->B >= 0 && q->H >= 0 && q->L >= 0 &&
        k->L >= 0) {
        const i64 bq = bwa::attn_rows_per_block(q->dtype, (int)q->D);
        const i64 units = q->B * q->H * ((q->L + bq - 1) / bq);
        const i64 need = units > 0 ? bwa::split_workspace_bytes(bwa::split_plan(units, bal.n_cus, k->L), (int)bq,
                                                                  (int)q->D)
                                   : 0;
        if (need > bwa::kNoAllocScratchBytes)
            return fail(BWA_ERR_CAPACITY,
                        "the balanced plan needs %lld bytes of workspace; the static scratch holds %lld "
                        "(use bwa_attn_fwd_balanced with a workspace)",
                        (long long)need, (long long)bwa::kNoAllocScratchBytes);
    }
    void* ws = nullptr;
    if ((st = hip_status(bwa::noalloc_scratch(&ws), "static scratch address"))) return st;
    bal.ws = ws;
    bal.ws_bytes = bwa::kNoAllocScratchBytes;
    return attn_fwd_impl(q, k, v, mask, blocks, scale, mode, m, gate, nullptr, nullptr, o, lse, stream, &bal);
}

int32_t bwa_attn_fwd_balanced_carry(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v,
                                    const bwa_mask* mask, const bwa_blocks* blocks, float scale, int32_t mode,
                                    const float* m, const uint8_t* gate, const bwa_tensor* o_prev,
                                    const float* lse_prev, int32_t n_cus, void* workspace, int64_t workspace_bytes,
                                    bwa_tensor* o, float* lse, void* stream) {
    if (!o_prev) return fail(BWA_ERR_NULL_ARG, "o_prev is NULL");
    Balance bal;
    int32_t st;
    if ((st = resolve_cus(n_cus, &bal.n_cus))) return st;
    bal.ws = workspace;
    bal.ws_bytes = workspace_bytes;
    return attn_fwd_impl(q, k, v, mask, blocks, scale, mode, m, gate, o_prev, lse_prev, o, lse, stream, &bal);
}

// The backward pass of a dilated band that splits into strided windows (as
// the forward does; order ascending): one pass per batch element over g
// residue classes, with the element's LSE gathered into the workspace in the
// windows' row order first.  Its workspace: the windows' own, after the
// gathered LSE.
static i64 bwd_split_bytes(const bwa::MaskDev& m, i64 H, i64 Lq, i64 Lk) {
    if (!band_splits(m, Lq, Lk)) return 0;
    const i64 g = m.dilation;
    return (H * Lq * 4 + 255) / 256 * 256 + bwa::bwd_workspace_bytes(g, H, Lq / g, Lk / g, 1);
}

int32_t bwa_attn_bwd_workspace(const bwa_mask* mask, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t* bytes,
                               int64_t* n_kv_tiles) {
    if (!bytes) return fail(BWA_ERR_NULL_ARG, "bytes output is NULL");
    if (B < 0 || H < 0 || Lq < 0 || Lk < 0) return fail(BWA_ERR_BAD_SHAPE, "negative size");
    if (Lq > kMaxLen || Lk > kMaxLen) return fail(BWA_ERR_UNSUPPORTED, "length exceeds 2^30");
    bwa::MaskDev md;
    int32_t st = resolve_mask(mask, B, Lq, Lk, md);
    if (st) return st;
    const i64 lb = md.seg_mode >= 2 ? B : 1;
    *bytes = std::max(bwa::bwd_workspace_bytes(B, H, Lq, Lk, lb), bwd_split_bytes(md, H, Lq, Lk));
    if (n_kv_tiles) *n_kv_tiles = (Lk + 63) / 64;
    return ok();
}

static hipError_t launch_bwd_split(const bwa::BwdLaunch& a, void* workspace, hipStream_t stream) {
    const i64 g = a.mask.dilation;
    const i64 eg = a.grad_dtype == BWA_BF16 ? 2 : 4, eo = a.o_dtype == BWA_BF16 ? 2 : 4;
    float* lse_w = (float*)workspace;
    void* ws = (char*)workspace + (a.H * a.Lq * 4 + 255) / 256 * 256;
    for (i64 b = 0; b < a.B; ++b) {
        hipError_t e = bwa::launch_lse_gather(a.lse + b * a.H * a.Lq, lse_w, a.H, a.Lq, (int)g, stream);
        if (e != hipSuccess) return e;
        bwa::BwdLaunch s = a;
        s.B = (int)g;
        s.Lq = a.Lq / g;
        s.Lk = a.Lk / g;
        s.q = (const char*)a.q + b * a.q_sB * 2; s.q_sB = a.q_sL; s.q_sL = a.q_sL * g;
        s.k = (const char*)a.k + b * a.k_sB * 2; s.k_sB = a.k_sL; s.k_sL = a.k_sL * g;
        s.v = (const char*)a.v + b * a.v_sB * 2; s.v_sB = a.v_sL; s.v_sL = a.v_sL * g;
        s.o = (const char*)a.o + b * a.o_sB * eo; s.o_sB = a.o_sL; s.o_sL = a.o_sL * g;
        s.dout = (const char*)a.dout + b * a.do_sB * 2; s.do_sB = a.do_sL; s.do_sL = a.do_sL * g;
        s.dq = (char*)a.dq + b * a.dq_sB * eg; s.dq_sB = a.dq_sL; s.dq_sL = a.dq_sL * g;
        s.dk = (char*)a.dk + b * a.dk_sB * eg; s.dk_sB = a.dk_sL; s.dk_sL = a.dk_sL * g;
        s.dv = (char*)a.dv + b * a.dv_sB * eg; s.dv_sB = a.dv_sL; s.dv_sL = a.dv_sL * g;
        s.lse = lse_w;
        s.mask = band_window(a.mask, a.Lq, a.Lk);
        s.list_batch = 1;
        bwa::bwd_workspace_layout(s, ws);
        e = bwa::launch_attn_bwd(s, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

int32_t bwa_attn_bwd(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v, const bwa_tensor* o,
                     const float* lse, const bwa_tensor* dout, const bwa_mask* mask, float scale, int32_t order,
                     const int32_t* kv_order, void* workspace, int64_t workspace_bytes, bwa_tensor* dq,
                     bwa_tensor* dk, bwa_tensor* dv, void* stream) {
    int32_t st;
    if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) ||
        (st = check_tensor(o, "o")) || (st = check_tensor(dout, "dout")) || (st = check_tensor(dq, "dq")) ||
        (st = check_tensor(dk, "dk")) || (st = check_tensor(dv, "dv")))
        return st;
    if (q->dtype != BWA_BF16) return fail(BWA_ERR_UNSUPPORTED, "the backward pass computes bf16 inputs only");
    if (k->dtype != q->dtype || v->dtype != q->dtype) return fail(BWA_ERR_BAD_DTYPE, "q, k and v must share a dtype");
    if (dout->dtype != BWA_BF16) return fail(BWA_ERR_BAD_DTYPE, "dout must be bf16");
    if (dk->dtype != dq->dtype || dv->dtype != dq->dtype)
        return fail(BWA_ERR_BAD_DTYPE, "dq, dk and dv must share a dtype");
    if (k->B != q->B || v->B != q->B || k->D != q->D || v->D != q->D || v->H != k->H || k->L != v->L)
        return fail(BWA_ERR_BAD_SHAPE, "q, k, v disagree on B or D, or k and v on H or L");
    if (q->H > 0 && (k->H <= 0 || q->H % k->H))
        return fail(BWA_ERR_BAD_SHAPE, "%lld key/value heads do not divide %lld query heads", (long long)k->H,
                    (long long)q->H);
    auto same = [](const bwa_tensor* a, const bwa_tensor* b) {
        return a->B == b->B && a->L == b->L && a->H == b->H && a->D == b->D;
    };
    if (!same(o, q) || !same(dout, q) || !same(dq, q)) return fail(BWA_ERR_BAD_SHAPE, "o, dout and dq must have q's shape");
    if (!same(dk, k) || !same(dv, k)) return fail(BWA_ERR_BAD_SHAPE, "dk and dv must have k's shape");
    if (order < BWA_ORDER_ASC || order > BWA_ORDER_CUSTOM) return fail(BWA_ERR_BAD_SHAPE, "unknown order %d", order);
    const i64 B = q->B, H = q->H, Lq = q->L, Lk = k->L;
    bwa::BwdLaunch a;
    memset(&a, 0, sizeof(a));
    if ((st = resolve_mask(mask, B, Lq, Lk, a.mask))) return st;
    if (B * H * Lq > 0 && !lse) return fail(BWA_ERR_NULL_ARG, "lse is NULL");
    if (order == BWA_ORDER_CUSTOM && Lk > 0 && !kv_order)
        return fail(BWA_ERR_NULL_ARG, "BWA_ORDER_CUSTOM needs kv_order");
    // One 256-work-item workgroup per (b, h, 128 rows) and per (b, h_kv, 128 keys); the delta pass
    // runs D/8 work-items per row: each launch holds under 2^32 work-items.
    if (B * H * ((Lq + 127) / 128) >= ((i64)1 << 23) || B * k->H * ((Lk + 127) / 128) >= ((i64)1 << 23) ||
        B * H * Lq * (q->D / 8) >= ((i64)1 << 32) - 256)
        return fail(BWA_ERR_UNSUPPORTED, "grid too large");
    a.list_batch = a.mask.seg_mode >= 2 ? B : 1;
    const bool split = order == BWA_ORDER_ASC && band_splits(a.mask, Lq, Lk);
    const i64 need = split ? bwd_split_bytes(a.mask, H, Lq, Lk) : bwa::bwd_workspace_bytes(B, H, Lq, Lk, a.list_batch);
    if (!workspace) return fail(BWA_ERR_NULL_ARG, "workspace is NULL");
    if ((uintptr_t)workspace % 256) return fail(BWA_ERR_BAD_STRIDE, "workspace not 256-byte aligned");
    if (workspace_bytes < need)
        return fail(BWA_ERR_CAPACITY, "workspace of %lld bytes; %lld needed", (long long)workspace_bytes,
                    (long long)need);
    a.q = q->ptr; a.k = k->ptr; a.v = v->ptr; a.o = o->ptr; a.dout = dout->ptr;
    a.q_sB = q->sB; a.q_sL = q->sL; a.q_sH = q->sH;
    a.k_sB = k->sB; a.k_sL = k->sL; a.k_sH = k->sH;
    a.v_sB = v->sB; a.v_sL = v->sL; a.v_sH = v->sH;
    a.o_sB = o->sB; a.o_sL = o->sL; a.o_sH = o->sH;
    a.do_sB = dout->sB; a.do_sL = dout->sL; a.do_sH = dout->sH;
    a.lse = lse;
    a.dq = dq->ptr; a.dq_sB = dq->sB; a.dq_sL = dq->sL; a.dq_sH = dq->sH;
    a.dk = dk->ptr; a.dk_sB = dk->sB; a.dk_sL = dk->sL; a.dk_sH = dk->sH;
    a.dv = dv->ptr; a.dv_sB = dv->sB; a.dv_sL = dv->sL; a.dv_sH = dv->sH;
    a.B = (int)B; a.H = (int)H; a.Hk = (int)k->H; a.D = (int)q->D;
    a.kv_group = H > 0 ? (int)(H / k->H) : 1;
    a.Lq = Lq; a.Lk = Lk;
    a.o_dtype = o->dtype;
    a.grad_dtype = dq->dtype;
    a.scale = scale;
    a.order = order;
    a.perm = order == BWA_ORDER_CUSTOM ? kv_order : nullptr;
    if (split) return hip_status(launch_bwd_split(a, workspace, (hipStream_t)stream), "attn_bwd launch");
    bwa::bwd_workspace_layout(a, workspace);
    return hip_status(bwa::launch_attn_bwd(a, (hipStream_t)stream), "attn_bwd launch");
}

int32_t bwa_lse_merge(int32_t n_parts, const bwa_tensor* o_parts, const float* const* lse_parts,
                      bwa_tensor* o_out, float* lse_out, void* stream) {
    if (n_parts < 1 || n_parts > bwa::kMaxParts)
        return fail(BWA_ERR_BAD_SHAPE, "n_parts must be in [1, %d]", bwa::kMaxParts);
    if (!o_parts || !lse_parts) return fail(BWA_ERR_NULL_ARG, "o_parts/lse_parts is NULL");
    int32_t st = check_tensor(o_out, "o_out");
    if (st) return st;
    bwa::MergeLaunch a;
    memset(&a, 0, sizeof(a));
    const i64 rows = o_out->B * o_out->L * o_out->H;
    for (int t = 0; t < n_parts; ++t) {
        char name[32];
        snprintf(name, sizeof(name), "o_parts[%d]", t);
        if ((st = check_tensor(&o_parts[t], name))) return st;
        const bwa_tensor& p = o_parts[t];
        if (p.dtype != BWA_F32) return fail(BWA_ERR_BAD_DTYPE, "%s must be fp32", name);
        if (p.B != o_out->B || p.L != o_out->L || p.H != o_out->H || p.D != o_out->D)
            return fail(BWA_ERR_BAD_SHAPE, "%s shape differs from o_out", name);
        if (rows > 0 && !lse_parts[t]) return fail(BWA_ERR_NULL_ARG, "lse_parts[%d] is NULL", t);
        a.o[t] = (const float*)p.ptr;
        a.lse[t] = lse_parts[t];
        a.sB[t] = p.sB; a.sL[t] = p.sL; a.sH[t] = p.sH;
    }
    // One 256-work-item workgroup per 64 tokens of a (b, h); a launch holds under 2^32 work-items.
    if (o_out->B * o_out->H * ((o_out->L + 63) / 64) >= ((i64)1 << 24))
        return fail(BWA_ERR_UNSUPPORTED, "merge grid too large");
    a.n_parts = n_parts;
    a.B = (int)o_out->B; a.H = (int)o_out->H; a.D = (int)o_out->D;
    a.L = o_out->L;
    a.out = o_out->ptr; a.out_sB = o_out->sB; a.out_sL = o_out->sL; a.out_sH = o_out->sH;
    a.out_dtype = o_out->dtype;
    a.lse_out = lse_out;
    return hip_status(bwa::launch_lse_merge(a, (hipStream_t)stream), "lse_merge launch");
}

}  // extern "C"
