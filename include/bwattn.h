/*
 * bwattn.h -- C ABI of the blockwise attention forward library (MI355X, gfx950).
 *
 * The library computes blockwise scaled-dot-product attention forward with
 * online softmax or with a fixed per-query bound in place of the running max,
 * the log-sum-exp merge of key-chunk partials, the fixed-m bound and gate,
 * the tile run lists that let the attention kernel skip whole tiles, and the
 * deterministic backward pass of the same attention.
 *
 * Pages the operations follow (cited by title and section):
 *  [FIXEDM]  "Fixed-m softmax for 2D-ring x Ulysses attention (WAN 2.2)"
 *            (maxdiffusion pull request 452): description, Result, Notes, Tests.
 *  [SPLASH]  "Let splash attention exceed 524,288 tokens when packing is off"
 *            (maxtext pull request 4929): description, Effect, review.
 *  [DKORDER] "Add more optimal dk order optional arg" (flash-attention pull
 *            request 2512): description (the backward pass and the order of
 *            the key columns), "Sliding window perf issue", "A simplish fix".
 *  [H3]      sglang pull request 47566 (H3 packed sequence): Motivation,
 *            Modifications.
 *  [ULYRING] maxdiffusion pull request 404 (ulysses_ring review): padding
 *            mask from global positions; validation of the layout.
 *
 * Conventions shared by every entry point
 *  - Tensors are token-major [B, L, H, D] with the last dimension contiguous;
 *    strides are in elements.  Base pointers and the B/L/H strides must be
 *    multiples of 16 bytes, and no two (b, l, h) rows may share an element:
 *    taken by increasing stride, each dimension of extent > 1 must step past
 *    everything the dimensions inside it span (so broadcast views with a zero
 *    stride, and L or H strides under D, return BWA_ERR_BAD_STRIDE; any
 *    permutation of B, L, H and padded row pitches are fine).  The L stride
 *    must be below 2^24 elements (BWA_ERR_BAD_STRIDE otherwise).  Per-row
 *    statistics (lse, m) are dense fp32 [B, H, L].
 *  - Every pointer inside a tensor or mask, and every output pointer, is a
 *    device pointer unless the argument says "host".  The caller allocates
 *    and owns every buffer; the library allocates no device memory and keeps
 *    no state between calls.
 *  - Every call is asynchronous on the given stream (a hipStream_t; NULL is
 *    the null stream) and never synchronises.  Argument errors are detected
 *    on the host before any launch and return a nonzero status with nothing
 *    enqueued; bwa_last_error() then describes the problem.  A failed launch
 *    returns BWA_ERR_HIP.  No C++ exception crosses the ABI.
 *  - Unsupported input returns BWA_ERR_UNSUPPORTED; there is no fallback to
 *    any other implementation.
 *  - Calls are deterministic: the same inputs give the same bits.
 */
#ifndef BWATTN_H
#define BWATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BWATTN_VERSION 3

/* Status codes. */
enum {
    BWA_OK = 0,
    BWA_ERR_NULL_ARG = 1,     /* a required pointer is NULL */
    BWA_ERR_BAD_SHAPE = 2,    /* sizes disagree or are negative */
    BWA_ERR_BAD_STRIDE = 3,   /* misaligned pointer or stride */
    BWA_ERR_BAD_DTYPE = 4,    /* dtype code unknown or not allowed here */
    BWA_ERR_BAD_MASK = 5,     /* inconsistent mask description */
    BWA_ERR_UNSUPPORTED = 6,  /* valid input this build does not handle (e.g. D not 64/128) */
    BWA_ERR_CAPACITY = 7,     /* caller-provided list storage too small */
    BWA_ERR_HIP = 8           /* the HIP runtime reported an error */
};

/* Element types. */
enum { BWA_F32 = 0, BWA_BF16 = 1 };

/* Attention modes. */
enum {
    BWA_MODE_ONLINE = 0,  /* running row max and rescale [FIXEDM description] */
    BWA_MODE_FIXED_M = 1, /* precomputed per-row bound m in place of the max [FIXEDM] */
    BWA_MODE_GATED = 2    /* per head: fixed-m where gate != 0, online elsewhere [FIXEDM Notes] */
};

/* Tile kinds in run lists [DKORDER "Sliding window perf issue"]. */
enum { BWA_TILE_SKIP = 0, BWA_TILE_FULL = 1, BWA_TILE_PARTIAL = 2 };

/* Orders in which a query block's key tiles add into dQ [DKORDER description]. */
enum {
    BWA_ORDER_ASC = 0,         /* ascending key tiles */
    BWA_ORDER_DESC = 1,        /* descending */
    BWA_ORDER_OUTSIDE_IN = 2,  /* tiles 0, n-1, 1, n-2, ... of all n key tiles */
    BWA_ORDER_CUSTOM = 3       /* the caller's permutation of the n key tiles */
};

/* A dense [B, L, H, D] tensor; d-stride is 1; strides in elements. */
typedef struct bwa_tensor {
    void* ptr;       /* device pointer to element [0,0,0,0] */
    int32_t dtype;   /* BWA_F32 or BWA_BF16 */
    int32_t reserved;
    int64_t B, L, H, D;
    int64_t sB, sL, sH;
} bwa_tensor;

/*
 * Mask description.  Query row i sits at position i and key j at position
 * j + kv_offset; write d = i - (j + kv_offset).  Key j is visible to row i
 * iff all of:
 *   j < kv_valid and i < q_valid         -- padding at the end of the global
 *                                           sequence [ULYRING]; alignment rows
 *                                           are zeroed [H3 Modifications]
 *   seg_q(i) == seg_kv(j)                -- packing / varlen [SPLASH; H3];
 *                                           documents [DKORDER masks]
 *   causal, no prefix => d >= 0
 *   causal, prefix P  => d >= 0 or j + kv_offset < P   (prefix-LM: the first
 *                                           P positions are seen by every row)
 *   window W > 0      => d < W when causal (a band of W keys ending at the
 *                        row), |d| < W when not (a two-sided band)
 *   dilation g >= 2   => d mod g == 0 (a dilated band; needs causal and W)
 * A row with no visible key gets O = 0 and LSE = -inf.  (The [DKORDER]
 * tables name sliding_window, prefix_lm, dilated_sliding_window and
 * document masks without defining them; these are the plainest readings.)
 * A dilated band is g causal windows of ceil(W / g) keys over the residue
 * classes of rows and keys; when Lq, Lk, kv_offset, q_valid and kv_valid are
 * multiples of g and there are no segments, bwa_attn_fwd (online mode,
 * without a carried partial) and bwa_attn_bwd (ascending order) compute it
 * that way, on strided views, so that they compute visible keys only; the
 * results agree with the band's own walk to rounding.
 *
 * Segments come either from cumulative lengths (cu_seqlens_q/kv, shared by
 * every batch element; segment s covers [cu[s], cu[s+1]); positions covered
 * by no segment see nothing) or from per-token segment ids ([B][L]; equal
 * ids see each other).  With documents == 0 the ids must be non-decreasing
 * along L (contiguous segments), and segments become per-row key intervals
 * before any attention tile runs, so no per-token table is held on chip and
 * the sequence length is bounded by memory only; one segment covering every
 * token gives exactly the unsegmented result [SPLASH description].  With
 * documents == 1 the ids may come in any order (a document's tokens need not
 * be contiguous): tiles that mix documents compare ids key by key.  Leave
 * both NULL for an unsegmented mask.
 */
typedef struct bwa_mask {
    int32_t causal;                 /* 0 or 1 */
    int32_t window;                 /* 0 = no window; see above */
    int64_t kv_offset;              /* key j is at position j + kv_offset (ring hop, bottom-right) */
    int64_t q_valid;                /* rows >= q_valid see nothing; < 0 means Lq */
    int64_t kv_valid;               /* keys >= kv_valid are invisible; < 0 means Lk */
    int32_t num_segments;           /* segments in cu_seqlens (0 when not used) */
    int32_t dilation;               /* 0 or 1 = none; >= 2 needs causal and window */
    const int32_t* cu_seqlens_q;    /* device [num_segments + 1], non-decreasing */
    const int32_t* cu_seqlens_kv;   /* device [num_segments + 1]; NULL = cu_seqlens_q */
    const int32_t* segment_ids_q;   /* device [B][Lq], or NULL */
    const int32_t* segment_ids_kv;  /* device [B][Lk]; NULL = segment_ids_q (needs Lq == Lk) */
    int64_t prefix;                 /* 0 = none; > 0 needs causal and no window */
    int32_t documents;              /* 0: ids non-decreasing; 1: ids in any order */
    int32_t reserved;
} bwa_mask;

/*
 * Tile run lists and per-row key intervals ([DKORDER]: partial and full
 * tiles; "A simplish fix": one ordered list).  For every query block of bq
 * rows, the key blocks of bkv keys that hold at least one visible pair are
 * listed in ascending order as maximal runs [begin, end) of one kind:
 * FULL (every pair visible) or PARTIAL.  Tiles are clipped to
 * [0, lq) x [0, lk).  row_lo/row_hi hold each row's visible keys [lo, hi)
 * ((0, 0) when the row sees nothing).  All arrays are device memory owned by
 * the caller and sized with bwa_block_mask_size.
 */
typedef struct bwa_blocks {
    int32_t bq, bkv;      /* tile sizes the lists are built for */
    int64_t lq, lk;       /* problem size the lists describe */
    int64_t batch;        /* list copies: 1 (shared by all batch elements) or B */
    int64_t n_qblocks;    /* ceil(lq / bq) */
    int64_t capacity;     /* run slots per copy */
    int64_t* row_ptr;     /* [batch][n_qblocks + 1] CSR offsets into the runs */
    int32_t* run_begin;   /* [batch][capacity] first key block of the run */
    int32_t* run_end;     /* [batch][capacity] one past the last key block */
    uint8_t* run_kind;    /* [batch][capacity] BWA_TILE_FULL or BWA_TILE_PARTIAL */
    int32_t* row_lo;      /* [batch][lq] */
    int32_t* row_hi;      /* [batch][lq] */
} bwa_blocks;

/* Human-readable name of a status code (static string). */
const char* bwa_status_string(int32_t status);

/* Detail of the last failure in the calling thread (static per thread). */
const char* bwa_last_error(void);

/* BWATTN_VERSION of the built library. */
int32_t bwa_version(void);

/* Tile sizes the attention kernel uses for (dtype, D): *bq rows per query
 * block (256 for bf16 with D = 128, else 128), key tiles of *bkv (64).  Lists
 * passed to bwa_attn_fwd must be built with this bq and a bkv that is a
 * multiple of this bkv.  Host only. */
int32_t bwa_attn_tile(int32_t dtype, int64_t D, int32_t* bq, int32_t* bkv);

/*
 * Storage needed by bwa_block_mask_build (host only, no launch, reads no
 * device memory).  Outputs: *n_qblocks = ceil(lq / bq); *list_batch = copies
 * (B with per-token segment ids, else 1); *capacity = run slots per copy that
 * is always enough: 3 per query block without segments (a partial edge, a
 * full middle, a partial edge), min(n_kblocks, bq + 2) per query block with
 * segments.
 */
int32_t bwa_block_mask_size(const bwa_mask* mask, int64_t B, int64_t lq, int64_t lk,
                            int32_t bq, int32_t bkv, int64_t* n_qblocks,
                            int64_t* capacity, int64_t* list_batch);

/*
 * Build tile run lists and row intervals for mask on a [B, lq] x [B, lk]
 * problem ([DKORDER]; the forward analogue of its partial/full block lists).
 * out->bq, bkv, lq, lk, batch, n_qblocks and capacity must hold the values
 * from bwa_block_mask_size (capacity may be larger) and its pointers the
 * caller's device buffers.  bq and bkv must be positive multiples of 64,
 * bq at most 512.
 * Results are exact integers (bit-exact against any correct implementation).
 * Preconditions checked on the device only by construction: cu_seqlens and
 * segment ids non-decreasing; violating them gives unspecified (but
 * in-bounds) lists.
 */
int32_t bwa_block_mask_build(const bwa_mask* mask, int64_t B, int64_t lq, int64_t lk,
                             bwa_blocks* out, void* stream);

/*
 * Fixed-m bound and gate [FIXEDM description and Notes].
 *   kmax[b,h]  = max over chunks c and keys j < kv_valid[c] of ||k_c[b,j,h,:]||_2,
 *                folded with max over s of kmax_in[s][b][h], s < n_kmax_in
 *                (per-shard max||k|| values of shards this call does not see,
 *                e.g. other ring ranks', promoted to the global bound);
 *   m[b,h,i]   = scale * ||q[b,i,h,:]||_2 * kmax[b,h]   (natural-log units);
 *   mmax[b,h]  = max over i < q_valid of m[b,h,i]   (0 when q_valid == 0);
 *   gate[b,h]  = 1 if mmax[b,h] <= tau and mmax[b,h] <= 58 ln 2 (= 40.2025)
 *                else 0   (a tie passes; compared in fp32).
 * The second term is the largest bound for which the fixed-m body of
 * bwa_attn_fwd is provably accurate in its own arithmetic (heads whose bound
 * cannot be proven safe keep online softmax [FIXEDM description]): with
 * |s_ij| <= m_i, a row's terms 2^32 exp(s - m_i) all lie in
 * [2^(32 - 2 m_i log2 e), 2^32]; at 2 m_i log2 e <= 116 the largest is at least
 * 2^-84, so up to 2^30 keys flushed under the fp32/bf16 normal range 2^-126
 * carry at most 2^-12 of its weight.  A tau above 40.2 (the page's 106.5)
 * therefore still sends heads with 40.2 < mmax <= tau to the online loop.
 * q: [B, Lq, H, D]; k_chunks: host array of n_chunks tensors [B, Lk_c, H, D]
 * with q's dtype, B, H and D; kv_valid: host array [n_chunks] (NULL = all
 * keys valid; entries < 0 mean Lk_c); kmax_in: device [n_kmax_in][B][H]
 * (NULL when n_kmax_in == 0); q_valid < 0 means Lq.  Outputs are device arrays: kmax_out [B][H],
 * mmax_out [B][H], m_out [B][H][Lq] (fp32), gate_out [B][H] (uint8).
 * Norms are fp32 sums of squares (bf16 products are exact in fp32).
 */
int32_t bwa_fixed_m_bound(const bwa_tensor* q, const bwa_tensor* k_chunks, int32_t n_chunks,
                          const float* kmax_in, int32_t n_kmax_in, const int64_t* kv_valid, int64_t q_valid,
                          float scale, float tau, float* kmax_out, float* mmax_out,
                          float* m_out, uint8_t* gate_out, void* stream);

/*
 * Blockwise attention forward on one key chunk.
 *   O[b,i,h,:] = sum_j p_ij v[b,j,h,:] / sum_j p_ij over visible keys j,
 *   LSE[b,h,i] = ln sum_j exp(scale * q_i . k_j)  (natural log),
 * computed tile by tile over the listed key blocks with
 *   BWA_MODE_ONLINE : a running row max and rescale of the partial sums,
 *   BWA_MODE_FIXED_M: p_ij = 2^32 exp(scale * q_i . k_j - m[b,h,i]) with the
 *                     caller's per-row bound m (from bwa_fixed_m_bound); no
 *                     max and no rescale [FIXEDM description]; the factor
 *                     2^32 cancels in O and is taken out of LSE.  The result
 *                     is exact in real arithmetic whenever m bounds the row's
 *                     scores, and accurate in this arithmetic whenever in
 *                     addition m_i <= 58 ln 2 (the gate of
 *                     bwa_fixed_m_bound); m is trusted, not checked.
 * q: [B, Lq, H, D]; k, v: [B, Lk, H, D]; q, k, v share a dtype (BWA_BF16
 * computes Q K^T and P V on bf16 matrix cores with fp32 accumulation and
 * rounds P to bf16; BWA_F32 computes in fp32 throughout).  D is 64 or 128.
 * o: [B, Lq, H, D] in fp32 or in q's dtype; lse: device fp32 [B][H][Lq].
 * mask: required.  blocks: run lists from bwa_block_mask_build for this mask
 * and shape (bq and bkv as bwa_attn_tile requires), or NULL to derive the
 * tile walk from the mask inside the kernel (always correct; per-token
 * segment ids then cost a per-row binary search).
 * gate: device uint8 [B][H] or NULL.  When given, an online call processes
 * only heads with gate == 0 and a fixed-m call only heads with gate != 0;
 * the other heads' outputs are left untouched, so a gated pair of calls on
 * the same outputs covers every head with one branch-free body each
 * [FIXEDM Notes].  BWA_MODE_GATED (gate and m required) does both in one
 * launch: each query block runs the fixed-m loop if its head passed the gate
 * and the online loop otherwise (two separate loops, one per workgroup), so
 * a single failing head does not leave a small second grid.
 * Rows with no visible key (padding, alignment rows) get O = 0 and
 * LSE = -inf and cost no tile work [H3 Modifications].
 */
int32_t bwa_attn_fwd(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v,
                     const bwa_mask* mask, const bwa_blocks* blocks, float scale,
                     int32_t mode, const float* m, const uint8_t* gate,
                     bwa_tensor* o, float* lse, void* stream);

/*
 * bwa_attn_fwd with a carried partial [FIXEDM Notes: hop partials combine in
 * LSE space; the next step there is to fold the combine into the hop itself].
 * Computes this call's attention over k/v exactly as bwa_attn_fwd does and
 * merges it, in the epilogue, with a partial (o_prev, lse_prev) over other,
 * disjoint key chunks of the same queries:
 *   lse = ln(e^lse_this + e^lse_prev)
 *   o   = e^(lse_this - lse) o_this + e^(lse_prev - lse) o_prev
 * so a ring of hops needs no separate merge pass: each hop carries the
 * running partial forward and the last hop can write the final output in
 * bf16.  A side whose LSE is -inf has weight 0 (its O rows are not read);
 * a row that both sides leave empty gets O = 0, LSE = -inf.
 * o_prev: device fp32 tensor of q's shape (non-NULL); lse_prev: device fp32
 * [B][H][Lq].  o may be the same tensor as o_prev (same pointer, fp32, same
 * strides) and lse may be lse_prev: each row is read before it is written,
 * by the same thread; any other overlap is not allowed.  With a gate, only
 * the rows this call writes are merged.  Errors as for bwa_attn_fwd, plus
 * BWA_ERR_NULL_ARG (o_prev or lse_prev NULL), BWA_ERR_BAD_DTYPE (o_prev not
 * fp32), BWA_ERR_BAD_SHAPE, BWA_ERR_BAD_STRIDE (partial alias of o).
 */
int32_t bwa_attn_fwd_carry(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v,
                           const bwa_mask* mask, const bwa_blocks* blocks, float scale,
                           int32_t mode, const float* m, const uint8_t* gate,
                           const bwa_tensor* o_prev, const float* lse_prev,
                           bwa_tensor* o, float* lse, void* stream);

/*
 * bwa_attn_fwd with the work balanced over the compute units.  Computes the
 * same O and LSE as bwa_attn_fwd (within rounding: see below).  The plain
 * launch runs one workgroup per (b, h, query block); the device deals
 * workgroups round-robin to its 8 XCDs, so each XCD runs an equal,
 * contiguous share of the blocks in launch order (head-major, the last query
 * block of a head first), in rounds of one block per compute unit.  XCDs do
 * not run at the same speed, and a share that is not a multiple of the
 * XCD's units leaves a last, partial round, so units idle at the end.  Here
 * n_cus workgroups (one per compute unit) loop over 8 queues holding the
 * same shares: first a share's whole rounds of blocks, then the blocks of
 * its last partial round, each cut along its key tiles into `pieces` equal
 * pieces; a workgroup whose queue is empty takes items from another XCD's.
 * The pieces' partials (fp32, in the workspace) are merged in LSE space
 * ([FIXEDM Notes]: the combine of partials over disjoint key ranges) by a
 * second kernel, in piece order.  No workgroup waits for another.
 *   - q, k, v must be BWA_BF16; every other argument, the outputs, gate and
 *     mode behave as in bwa_attn_fwd (blocks may be NULL).
 *   - n_cus: workgroups to launch (>= 1), normally the device's compute-unit
 *     count, which <= 0 selects.  Any value gives a correct result.
 *   - workspace: device memory of at least the bytes
 *     bwa_attn_fwd_balanced_workspace reports for the same dtype, B, H, Lq,
 *     Lk, D and n_cus, 256-byte aligned, owned by the caller.  The call
 *     clears what it uses; calls that share a workspace must be ordered
 *     (same stream), since a running call owns it.
 *   - Rounding: whole blocks give bwa_attn_fwd's bits.  A cut block's rows
 *     combine `pieces` partials, so they can differ from bwa_attn_fwd in the
 *     last bits (in the online mode each piece also rounds its
 *     probabilities to bf16 against its own running max); the result does
 *     not depend on the order in which workgroups take items, so it is
 *     deterministic for given sizes and n_cus.
 * Errors as for bwa_attn_fwd, plus BWA_ERR_NULL_ARG (workspace NULL),
 * BWA_ERR_UNSUPPORTED (fp32 inputs; n_cus > 65536), BWA_ERR_BAD_STRIDE
 * (workspace alignment), BWA_ERR_CAPACITY (workspace too small).
 */
int32_t bwa_attn_fwd_balanced(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v,
                              const bwa_mask* mask, const bwa_blocks* blocks, float scale,
                              int32_t mode, const float* m, const uint8_t* gate,
                              int32_t n_cus, void* workspace, int64_t workspace_bytes,
                              bwa_tensor* o, float* lse, void* stream);

/*
 * bwa_attn_fwd_balanced for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation with the same plan and bits, its
 * workspace taken from a static device array of 64 MiB that the library
 * holds on each device it runs on until the process ends (the array's
 * address is looked up on the first call on a device).  The call itself
 * allocates nothing.  Arguments, results and errors as for
 * bwa_attn_fwd_balanced without the workspace, plus BWA_ERR_CAPACITY when
 * the plan's workspace (bwa_attn_fwd_balanced_workspace) exceeds 64 MiB,
 * reported before anything is enqueued.  Every call on a device shares that
 * device's array: calls that may overlap on one device (other streams,
 * other threads) race and must be ordered by the caller.
 */
int32_t bwa_attn_fwd_balanced_noalloc(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v,
                                      const bwa_mask* mask, const bwa_blocks* blocks, float scale,
                                      int32_t mode, const float* m, const uint8_t* gate, int32_t n_cus,
                                      bwa_tensor* o, float* lse, void* stream);

/*
 * bwa_attn_fwd_balanced with a carried partial, merged as in
 * bwa_attn_fwd_carry [FIXEDM Notes]: whole blocks merge it in their epilogue,
 * cut blocks as one more part of the piece merge.  Arguments, aliasing rules
 * and errors as for bwa_attn_fwd_carry and bwa_attn_fwd_balanced.
 */
int32_t bwa_attn_fwd_balanced_carry(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v,
                                    const bwa_mask* mask, const bwa_blocks* blocks, float scale,
                                    int32_t mode, const float* m, const uint8_t* gate,
                                    const bwa_tensor* o_prev, const float* lse_prev,
                                    int32_t n_cus, void* workspace, int64_t workspace_bytes,
                                    bwa_tensor* o, float* lse, void* stream);

/*
 * Plan of bwa_attn_fwd_balanced for q of dtype/B/H/Lq/D, keys of length Lk
 * and n_cus (<= 0: the current device's compute-unit count, which this call
 * then queries).  Host outputs: *bytes, the workspace size (required);
 * *cut_blocks, how many query blocks are cut, and *pieces, into how many
 * pieces each (both optional, may be NULL).  With U blocks dealt to 8 shares
 * of floor(U/8) or floor(U/8) + 1 (the first U mod 8 shares) and
 * c = max(1, n_cus / 8), a share of u blocks cuts its last u mod c;
 * pieces = min(4, floor(ceil(Lk / 64) / 8)), and nothing is cut when that is
 * below 2.
 * The workspace holds 256 bytes of queue counters plus
 * cut_blocks * pieces * rows-per-block * (D + 1) * 4 bytes of partials.
 */
int32_t bwa_attn_fwd_balanced_workspace(int32_t dtype, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                                        int32_t n_cus, int64_t* bytes, int64_t* cut_blocks, int32_t* pieces);

/*
 * Backward pass of bwa_attn_fwd [DKORDER description: a program per key
 * column computes that column's dK and dV, and each query block's dQ
 * collects one contribution per key column in an order the caller chooses;
 * a fixed order makes dQ repeat bit for bit].  For the loss
 * sum_i dout_i . O_i, with P = exp(scale * Q K^T - LSE) over the visible
 * pairs (0 elsewhere):
 *   dV = P^T dout,  dS = P o (dout V^T - delta),  delta_i = dout_i . O_i,
 *   dQ = scale * dS K,  dK = scale * dS^T Q,
 * and with grouped-query heads a key/value head's dK and dV sum over the
 * query heads that read it.
 *   - q, k, v: BWA_BF16, shapes and mask as for bwa_attn_fwd (D 64 or 128).
 *     o: the forward output (fp32 or bf16, q's shape); lse: the forward's
 *     device fp32 [B][H][Lq]; dout: the upstream gradient, BWA_BF16, q's
 *     shape.  dq (q's shape), dk and dv (k's shape): outputs, all fp32 or all
 *     bf16; every element is written (keys no row sees and rows that see
 *     nothing get 0).
 *   - order: BWA_ORDER_*.  A query block adds the contributions of its key
 *     tiles (64 keys each; n = ceil(Lk / 64) of them) into dQ in the order
 *     of the tiles' positions in the permutation: ascending, descending,
 *     outside-in, or kv_order (device int32 [n], required only for
 *     BWA_ORDER_CUSTOM; it must be a permutation of 0..n-1: entries out of
 *     range are ignored, a repeated entry is added twice).  dK and dV always
 *     add query tiles in ascending order.  The order changes only dQ's
 *     rounding; every order is deterministic.
 *   - workspace: device memory of at least bwa_attn_bwd_workspace bytes for
 *     the same B, H, Lq, Lk and mask, 256-byte aligned, owned by the caller;
 *     calls that share it must be ordered (same stream).
 * No workgroup waits for another and nothing is accumulated with atomics:
 * the key-column kernel writes dK and dV, a query-block kernel recomputes
 * the probabilities and writes dQ.  P and dS are rounded to bf16 as
 * matrix-core operands; accumulation is fp32.
 * Errors as for bwa_attn_fwd, plus BWA_ERR_UNSUPPORTED (q not bf16),
 * BWA_ERR_BAD_DTYPE (dout not bf16, o or the gradients not fp32/bf16, or
 * the gradients of mixed dtypes), BWA_ERR_BAD_SHAPE (an unknown order),
 * BWA_ERR_NULL_ARG (workspace, lse or kv_order missing), BWA_ERR_BAD_STRIDE
 * (workspace alignment), BWA_ERR_CAPACITY (workspace too small).
 */
int32_t bwa_attn_bwd(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v, const bwa_tensor* o,
                     const float* lse, const bwa_tensor* dout, const bwa_mask* mask, float scale,
                     int32_t order, const int32_t* kv_order, void* workspace, int64_t workspace_bytes,
                     bwa_tensor* dq, bwa_tensor* dk, bwa_tensor* dv, void* stream);

/*
 * Workspace of bwa_attn_bwd for B, H query heads, Lq, Lk and mask (host
 * only, no launch).  *bytes = pad(B*H*Lq*4) + 2 pad(c*Lq*4)
 * + pad(c*ceil(Lq/64)*16) + 2 pad(c*ceil(Lk/128)*4) + pad(c*ceil(Lq/64)*4)
 * + pad(c*ceil(Lk/64)*4) + pad(c*ceil(Lq/64)*8) + pad(c*ceil(Lk/64)*8),
 * pad = round up to 256, c = B with per-token segment ids, else 1 (the last
 * four hold document-id summaries of the query and key tiles).  For a
 * dilated band computed as strided windows (see the mask description),
 * *bytes is the larger of that and pad(H*Lq*4) plus the same formula for B =
 * g, Lq / g, Lk / g, c = 1 (one batch element's LSE in the windows' row order,
 * then the windows' own workspace).  *n_kv_tiles (optional) = the
 * number of 64-key tiles, the length of a BWA_ORDER_CUSTOM permutation.
 */
int32_t bwa_attn_bwd_workspace(const bwa_mask* mask, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                               int64_t* bytes, int64_t* n_kv_tiles);

/*
 * Log-sum-exp merge of attention partials over disjoint key chunks
 * [FIXEDM Notes: the fallback merge in LSE space, invariant to the overshoot]:
 *   lse[b,h,i] = ln sum_t exp(lse_t[b,h,i])            (-inf if all are -inf)
 *   O[b,i,h,:] = sum_t exp(lse_t - lse) O_t[b,i,h,:]    (0 if lse is -inf)
 * A part whose lse_t is -inf on a row has weight 0 there and its O_t row is
 * not used (it may hold anything, NaN included).
 * n_parts in [1, 16]; o_parts: host array of n_parts fp32 tensors of one
 * shape; lse_parts: host array of n_parts device pointers to fp32 [B][H][L];
 * o_out: same B, L, H, D in fp32 or bf16 (may alias no input); lse_out:
 * device fp32 [B][H][L] (may be NULL).
 */
int32_t bwa_lse_merge(int32_t n_parts, const bwa_tensor* o_parts, const float* const* lse_parts,
                      bwa_tensor* o_out, float* lse_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BWATTN_H */
