"""GPU parity at the full workload sizes, against the fp64 oracle.

Workloads (synthetic stand-ins for the pages' models and data, see synth):
  * tiny     B=1 H=2 L=256 D=64 fp32, dense, and split in 2 KV chunks + LSE merge
  * varlen   H3 packed request, cu_seqlens [0, 33002, 33024], 24 heads
  * window   causal bands W in {512, 1024, 2048} on 4096^2, 4096x8192, 8192^2
  * dit      one rank's share of ring2 x uly2 video-DiT attention (2 KV hops,
             fixed-m with a sink head on online fallback, LSE merge), with the
             plain and the balanced launch (the bench's)
  * long     1,048,576-token causal attention, single segment and packed
  * page     the flash-attention tables' named masks (prefix_lm, dilated
             sliding window, document) and a two-sided band at their shapes

Large outputs are checked on a seeded sample of 512 query rows per head
(always holding the first and last valid rows, segment-boundary rows and an
invalid row where one exists); integer outputs (run lists, row intervals,
gates, zero rows) are checked exactly.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_close, gpu_rows, mask_for_batch, np64, oracle_attention

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import blockwise_attention_forward_amd as bw  # noqa: E402

DEV = "cuda"
BF16 = torch.bfloat16


def _lists_match_oracle(bl, mask, Lq, Lk, bq, bkv, qblocks=None):
    """GPU run lists and row intervals equal the oracle's (interval method)."""
    lo, hi = oracle.row_intervals(Lq, Lk, mask)
    assert np.array_equal(bl.row_lo[:Lq].cpu().numpy(), lo)
    assert np.array_equal(bl.row_hi[:Lq].cpu().numpy(), hi)
    rp, b, e, k = bl.host()
    nqb = (Lq + bq - 1) // bq
    qblocks = np.arange(nqb) if qblocks is None else np.asarray(qblocks)
    kinds = oracle.block_kinds_intervals(lo, hi, Lq, Lk, bq, bkv, qblocks=qblocks)
    for n, qb in enumerate(qblocks):
        got = (b[rp[qb]:rp[qb + 1]], e[rp[qb]:rp[qb + 1]], k[rp[qb]:rp[qb + 1]])
        w = oracle.runs_from_kinds(kinds[n:n + 1])
        assert np.array_equal(got[0], w[1]) and np.array_equal(got[1], w[2]) and np.array_equal(got[2], w[3]), qb
    return kinds


def _gpu_tile_counts(bl, Lq, Lk, bq, bkv):
    rp, b, e, k = bl.host()
    n_tiles = int((e - b).astype(np.int64).sum())
    n_partial = int(((e - b) * (k == bw.BWA_TILE_PARTIAL)).astype(np.int64).sum())
    return n_tiles, n_partial


# ------------------------------------------------------------------- tiny
def test_tiny_dense_and_two_chunk_merge():
    t = synth.make_tiny(DEV)
    q, k, v, scale = t["q"], t["k"], t["v"], t["scale"]
    o_ref, l_ref = oracle_attention(q, k, v, {}, scale)
    o, l = bw.bwa_attn_fwd(q, k, v, {}, scale=scale)
    assert_close(o, l, o_ref, l_ref, torch.float32, "tiny")
    parts = [bw.bwa_attn_fwd(q, k[:, a:e], v[:, a:e], {"kv_offset": a}, scale=scale) for a, e in t["chunks"]]
    om, lm = bw.bwa_lse_merge([p[0] for p in parts], [p[1] for p in parts], out_dtype=torch.float32)
    assert_close(om, lm, o_ref, l_ref, torch.float32, "tiny merged")


# ------------------------------------------------------------------- varlen
def test_varlen_packed_request():
    w = synth.make_varlen(DEV)
    q, k, v, mask, scale = w["q"], w["k"], w["v"], w["mask"], w["scale"]
    L = q.shape[1]
    bl128 = bw.bwa_block_mask_build(mask, 1, L, L, 128, 128)
    kinds = _lists_match_oracle(bl128, mask, L, L, 128, 128)
    assert (kinds != oracle.SKIP).sum() == 66564 and (kinds == oracle.PARTIAL).sum() == 515
    bq, _ = bw.bwa_attn_tile(BF16, 128)
    blocks = bw.bwa_block_mask_build(mask, 1, L, L, bq, 128)
    _lists_match_oracle(blocks, mask, L, L, bq, 128)
    o, l = bw.bwa_attn_fwd(q, k, v, mask, blocks=blocks, scale=scale)
    o2, l2 = bw.bwa_attn_fwd(q, k, v, mask, scale=scale)
    assert torch.equal(o, o2) and torch.equal(l, l2)
    # the 22 alignment rows are written as zeros with LSE -inf, in every head
    assert torch.all(o[:, 33002:] == 0) and torch.all(torch.isneginf(l[:, :, 33002:]))
    rows = synth.sample_rows(L, 512, seed=21, must=[0, 127, 128, 255, 256, 32895, 32896, 33001, 33002, 33023])
    o_ref, l_ref = oracle_attention(q, k, v, mask, scale, rows)
    assert_close(*gpu_rows(o, l, rows), o_ref, l_ref, BF16, "varlen")


# ------------------------------------------------------------------- window
WINDOW_COUNTS = {(4096, 4096): (150, 252, 408), (4096, 8192): (160, 288, 544), (8192, 8192): (310, 540, 952)}


@pytest.mark.parametrize("W", [512, 1024, 2048])
@pytest.mark.parametrize("Lq,Lk", [(4096, 4096), (4096, 8192), (8192, 8192)])
def test_sliding_window(Lq, Lk, W):
    w = synth.make_window(Lq, Lk, W, DEV)
    q, k, v, mask, scale = w["q"], w["k"], w["v"], w["mask"], w["scale"]
    bl128 = bw.bwa_block_mask_build(mask, 1, Lq, Lk, 128, 128)
    want = oracle.block_lists(mask, Lq, Lk, 128, 128)  # element predicate, brute force
    got = bl128.host()
    for g, x in zip(got, want):
        assert np.array_equal(g, x)
    n_tiles, _ = _gpu_tile_counts(bl128, Lq, Lk, 128, 128)
    assert n_tiles == WINDOW_COUNTS[(Lq, Lk)][(512, 1024, 2048).index(W)]
    bq, _ = bw.bwa_attn_tile(BF16, 128)
    blocks = bw.bwa_block_mask_build(mask, 1, Lq, Lk, bq, 128)
    _lists_match_oracle(blocks, mask, Lq, Lk, bq, 128)
    o, l = bw.bwa_attn_fwd(q, k, v, mask, blocks=blocks, scale=scale)
    rows = synth.sample_rows(Lq, 512, seed=22, must=[0, 1, W - 1, W, Lq - 1])
    o_ref, l_ref = oracle_attention(q, k, v, mask, scale, rows)
    assert_close(*gpu_rows(o, l, rows), o_ref, l_ref, BF16, f"window {Lq}x{Lk} W={W}")


# ------------------------------------------------------------------- dit share
# ------------------------------------------------------------- page masks
@pytest.mark.parametrize("kind", synth.PAGE_MASKS)
@pytest.mark.parametrize("Lq,Lk", [(4096, 4096), (4096, 8192), (8192, 8192)])
def test_page_masks(kind, Lq, Lk):
    # the flash-attention tables' prefix_lm, dilated_sliding_window and
    # document masks (and a two-sided band) at their shapes: run lists exact,
    # sampled rows against the oracle, run lists and inline walk bit-equal
    w = synth.make_page_mask(kind, Lq, Lk, DEV)
    q, k, v, mask, scale = w["q"], w["k"], w["v"], w["mask"], w["scale"]
    m0 = mask_for_batch(mask, 0)
    bq, _ = bw.bwa_attn_tile(BF16, 128)
    blocks = bw.bwa_block_mask_build(mask, 1, Lq, Lk, bq, 128)
    rp, be, en, kd = blocks.host()
    want = oracle.block_lists(m0, Lq, Lk, bq, 128)
    assert all(np.array_equal(x, y) for x, y in zip((rp, be, en, kd), want))
    o, l = bw.bwa_attn_fwd(q, k, v, mask, blocks=blocks, scale=scale)
    o2, l2 = bw.bwa_attn_fwd(q, k, v, mask, scale=scale)
    assert torch.equal(o, o2) and torch.equal(l, l2)
    rows = synth.sample_rows(Lq, 256, seed=29, must=[0, 1, 63, 64, Lq // 4 - 1, Lq // 4, Lq - 1])
    o_ref, l_ref = oracle_attention(q, k, v, m0, scale, rows)
    assert_close(*gpu_rows(o, l, rows), o_ref, l_ref, BF16, f"{kind} {Lq}x{Lk}")


@pytest.mark.parametrize("kind", synth.PAGE_MASKS)
def test_page_masks_gated(kind):
    # The page masks with the fixed-m bound and gate (bench --mode gated), plain
    # launch: every head passes on these inputs; the fixed-m body with the
    # element tests (dilated bands walk their band here, not the strided
    # windows) matches the oracle, and the gated launch gives the fixed-m bits.
    Lq = Lk = 4096
    w = synth.make_page_mask(kind, Lq, Lk, DEV)
    q, k, v, mask, scale = w["q"], w["k"], w["v"], w["mask"], w["scale"]
    m0 = mask_for_batch(mask, 0)
    qv, kvv = int(mask.get("q_valid", Lq)), int(mask.get("kv_valid", Lk))
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, [k], scale, 106.5, kv_valid=[kvv], q_valid=qv)
    assert gate.all().item()
    bq, _ = bw.bwa_attn_tile(BF16, 128)
    blocks = bw.bwa_block_mask_build(mask, 1, Lq, Lk, bq, 128)
    o, l = bw.bwa_attn_fwd(q, k, v, mask, blocks=blocks, scale=scale, mode=bw.BWA_MODE_GATED, m=m, gate=gate)
    o2, l2 = bw.bwa_attn_fwd(q, k, v, mask, blocks=blocks, scale=scale, mode=bw.BWA_MODE_FIXED_M, m=m)
    assert torch.equal(o, o2) and torch.equal(l, l2)
    rows = synth.sample_rows(Lq, 256, seed=31, must=[0, 1, 63, 64, Lq // 4 - 1, Lq // 4, Lq - 1])
    o_ref, l_ref = oracle_attention(q, k, v, m0, scale, rows)
    assert_close(*gpu_rows(o, l, rows), o_ref, l_ref, BF16, f"{kind} gated")


@pytest.fixture(scope="module")
def dit():
    return synth.make_dit_share(DEV)


def _hops(d, mode, m=None, gate=None, balanced=False, parts_out=None):
    q = d["q"]
    B, Lq, H, D = q.shape
    bq, _ = bw.bwa_attn_tile(BF16, D)
    attn = bw.bwa_attn_fwd_balanced if balanced else bw.bwa_attn_fwd
    parts = []
    for k, v, off in zip(d["k_chunks"], d["v_chunks"], d["kv_offsets"]):
        mask = {"kv_offset": off}
        blocks = bw.bwa_block_mask_build(mask, B, Lq, k.shape[1], bq, 128)
        parts.append(attn(q, k, v, mask, blocks=blocks, scale=d["scale"], mode=mode, m=m, gate=gate,
                          out_dtype=torch.float32))
    if parts_out is not None:
        parts_out.extend(parts)
    return bw.bwa_lse_merge([p[0] for p in parts], [p[1] for p in parts], out_dtype=BF16)


def _cut_blocks(B, H, Lq, Lk, D):
    """(b, h, first row, end row) of the query blocks the balanced launch cuts
    on this device: per XCD share, the blocks past its last whole round."""
    nbytes, cut, pieces = bw.bwa_attn_fwd_balanced_workspace(BF16, B, H, Lq, Lk, D, plan=True)
    bq, _ = bw.bwa_attn_tile(BF16, D)
    nqb = (Lq + bq - 1) // bq
    U = B * H * nqb
    c = max(1, torch.cuda.get_device_properties(0).multi_processor_count // 8)
    q_, r_ = divmod(U, 8)
    out = []
    for x in range(8):
        u = q_ + (1 if x < r_ else 0)
        a = x * q_ + min(x, r_)
        d = (u // c) * c if pieces > 1 else u
        for unit in range(a + d, a + u):
            bh, qb = unit // nqb, nqb - 1 - unit % nqb
            out.append((bh // H, bh % H, qb * bq, min(Lq, (qb + 1) * bq)))
    assert len(out) == cut
    return out


def _check_balanced_vs_plain(o_b, l_b, o_p, l_p, cut):
    """Rows of whole blocks: the plain launch's bits.  Rows of cut blocks: one
    LSE-space combine more, with probabilities rounded to bf16 against each
    piece's own running max in the online body: bf16 rounding level of P."""
    cut_rows = torch.zeros(l_p.shape, dtype=torch.bool, device=DEV)  # [B, H, L]
    for b, h, r0, r1 in cut:
        cut_rows[b, h, r0:r1] = True
    assert cut_rows.any() and not cut_rows.all()
    assert torch.equal(l_b[~cut_rows], l_p[~cut_rows])
    oc = cut_rows.permute(0, 2, 1)
    assert torch.equal(o_b[~oc], o_p[~oc])
    fin = torch.isfinite(l_p) & cut_rows
    assert torch.equal(torch.isneginf(l_b), torch.isneginf(l_p))
    assert bool(((l_b[fin] - l_p[fin]).abs() <= 1e-5 + 1e-6 * l_p[fin].abs()).all())
    err = (o_b[oc].float() - o_p[oc].float()).abs()
    assert err.max().item() <= 4e-3 and err.mean().item() <= 3e-4, (err.max().item(), err.mean().item())


def _dit_oracle(d, rows):
    k = torch.cat(d["k_chunks"], dim=1)
    v = torch.cat(d["v_chunks"], dim=1)
    return oracle_attention(d["q"], k, v, {}, d["scale"], rows)


def test_dit_bound_gate_and_promotion(dit):
    q, ks, scale = dit["q"], dit["k_chunks"], dit["scale"]
    H = q.shape[2]
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, ks, scale, 106.5)
    g = gate[0].cpu().numpy()
    assert g[dit["sink_head"]] == 0 and g.sum() == H - 1
    for h in range(H):
        km, mr, mm, gh = oracle.fixed_m_bound(np64(q[0, :, h]), [np64(c[0, :, h]) for c in ks], scale, 106.5)
        np.testing.assert_allclose(kmax[0, h].item(), km, rtol=1e-6)
        np.testing.assert_allclose(np64(m[0, h]), mr, rtol=2e-6)
        np.testing.assert_allclose(mmax[0, h].item(), mm, rtol=2e-6)
        assert bool(g[h]) == gh
    # a caller's per-shard max||k|| promoted to the global bound: the bound
    # over chunk 0 alone with both shards' maxima equals the two-chunk bound
    per = torch.stack([bw.bwa_fixed_m_bound(q, [c], scale, 106.5)[0] for c in ks])
    k2, mm2, m2, g2 = bw.bwa_fixed_m_bound(q, [ks[0]], scale, 106.5, kmax_in=per)
    assert torch.equal(k2, kmax) and torch.equal(m2, m) and torch.equal(g2, gate) and torch.equal(mm2, mmax)


def test_dit_gated_and_online_hops(dit):
    q = dit["q"]
    Lq = q.shape[1]
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, dit["k_chunks"], dit["scale"], 106.5)
    o_g, l_g = _hops(dit, bw.BWA_MODE_GATED, m=m, gate=gate)
    o_o, l_o = _hops(dit, bw.BWA_MODE_ONLINE)
    rows = synth.sample_rows(Lq, 512, seed=23, must=[0, 1, 127, 128, Lq - 41, Lq - 1])
    o_ref, l_ref = _dit_oracle(dit, rows)
    assert_close(*gpu_rows(o_g, l_g, rows), o_ref, l_ref, BF16, "dit gated")
    assert_close(*gpu_rows(o_o, l_o, rows), o_ref, l_ref, BF16, "dit online")


def test_dit_balanced_hops(dit):
    # The bench's launch: each hop through the balanced launch (per-XCD queues,
    # cut blocks of each XCD's last partial round), then the merge.  Sampled
    # rows cover the cut blocks; whole blocks match the plain launch bit for bit.
    q = dit["q"]
    B, Lq, H, D = q.shape
    Lc = dit["k_chunks"][0].shape[1]
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, dit["k_chunks"], dit["scale"], 106.5)
    cut = _cut_blocks(B, H, Lq, Lc, D)
    parts_b, parts_p = [], []
    o, l = _hops(dit, bw.BWA_MODE_GATED, m=m, gate=gate, balanced=True, parts_out=parts_b)
    _hops(dit, bw.BWA_MODE_GATED, m=m, gate=gate, parts_out=parts_p)
    for (ob, lb), (op, lp) in zip(parts_b, parts_p):
        _check_balanced_vs_plain(ob, lb, op, lp, cut)
    must = [0, Lq - 1] + sorted({r0 for _, _, r0, _ in cut} | {r1 - 1 for _, _, _, r1 in cut})[:24]
    rows = synth.sample_rows(Lq, 512, seed=27, must=must)
    o_ref, l_ref = _dit_oracle(dit, rows)
    assert_close(*gpu_rows(o, l, rows), o_ref, l_ref, BF16, "dit balanced hops")


def test_varlen_balanced():
    w = synth.make_varlen(DEV)
    q, k, v, mask, scale = w["q"], w["k"], w["v"], w["mask"], w["scale"]
    B, L, H, D = q.shape
    bq, _ = bw.bwa_attn_tile(BF16, D)
    blocks = bw.bwa_block_mask_build(mask, 1, L, L, bq, 128)
    cut = _cut_blocks(B, H, L, L, D)
    o, l = bw.bwa_attn_fwd_balanced(q, k, v, mask, blocks=blocks, scale=scale)
    o_p, l_p = bw.bwa_attn_fwd(q, k, v, mask, blocks=blocks, scale=scale)
    _check_balanced_vs_plain(o, l, o_p, l_p, cut)
    assert torch.all(o[:, 33002:] == 0) and torch.all(torch.isneginf(l[:, :, 33002:]))
    must = [0, 33001, 33002, 33023] + sorted({r0 for _, _, r0, _ in cut} | {r1 - 1 for _, _, _, r1 in cut})[:24]
    rows = synth.sample_rows(L, 512, seed=28, must=must)
    o_ref, l_ref = oracle_attention(q, k, v, mask, scale, rows)
    assert_close(*gpu_rows(o, l, rows), o_ref, l_ref, BF16, "varlen balanced")


def test_varlen_gated_balanced():
    # The packed request with the fixed-m bound and gate (bench --mode gated):
    # the alignment rows stay zero with LSE -inf, the rest matches the oracle.
    w = synth.make_varlen(DEV)
    q, k, v, mask, scale = w["q"], w["k"], w["v"], w["mask"], w["scale"]
    B, L, H, D = q.shape
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, [k], scale, 106.5, q_valid=mask["q_valid"])
    assert gate.all().item()
    bq, _ = bw.bwa_attn_tile(BF16, D)
    blocks = bw.bwa_block_mask_build(mask, 1, L, L, bq, 128)
    o, l = bw.bwa_attn_fwd_balanced(q, k, v, mask, blocks=blocks, scale=scale, mode=bw.BWA_MODE_GATED, m=m,
                                    gate=gate)
    assert torch.all(o[:, 33002:] == 0) and torch.all(torch.isneginf(l[:, :, 33002:]))
    rows = synth.sample_rows(L, 512, seed=30, must=[0, 127, 128, 33001, 33002, 33023])
    o_ref, l_ref = oracle_attention(q, k, v, mask, scale, rows)
    assert_close(*gpu_rows(o, l, rows), o_ref, l_ref, BF16, "varlen gated")


def _hops_carry(d, mode, m=None, gate=None, balanced=False):
    """The hops chained by the carried partial: hop 0 writes fp32, the last hop the bf16 result."""
    q = d["q"]
    B, Lq, H, D = q.shape
    bq, _ = bw.bwa_attn_tile(BF16, D)
    o = lse = None
    n = len(d["k_chunks"])
    for t, (k, v, off) in enumerate(zip(d["k_chunks"], d["v_chunks"], d["kv_offsets"])):
        mask = {"kv_offset": off}
        blocks = bw.bwa_block_mask_build(mask, B, Lq, k.shape[1], bq, 128)
        kw = dict(mask=mask, blocks=blocks, scale=d["scale"], mode=mode, m=m, gate=gate,
                  out_dtype=BF16 if t == n - 1 else torch.float32)
        if balanced:
            carry = {} if t == 0 else dict(o_prev=o, lse_prev=lse)
            o, lse = bw.bwa_attn_fwd_balanced(q, k, v, **kw, **carry)
        elif t == 0:
            o, lse = bw.bwa_attn_fwd(q, k, v, **kw)
        else:
            o, lse = bw.bwa_attn_fwd_carry(q, k, v, o, lse, **kw)
    return o, lse


def test_dit_hops_chained_by_carry(dit):
    q = dit["q"]
    Lq = q.shape[1]
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, dit["k_chunks"], dit["scale"], 106.5)
    o, l = _hops_carry(dit, bw.BWA_MODE_GATED, m=m, gate=gate)
    assert o.dtype == BF16
    rows = synth.sample_rows(Lq, 512, seed=26, must=[0, 1, 127, 128, Lq - 41, Lq - 1])
    o_ref, l_ref = _dit_oracle(dit, rows)
    assert_close(*gpu_rows(o, l, rows), o_ref, l_ref, BF16, "dit carried hops")
    # and every row agrees with the separate merge pass to bf16 rounding
    o_m, l_m = _hops(dit, bw.BWA_MODE_GATED, m=m, gate=gate)
    assert (l - l_m).abs().max().item() <= 1e-5
    assert (o.float() - o_m.float()).abs().max().item() <= 2 ** -7


def test_dit_balanced_hops_chained_by_carry(dit):
    # the bench's carried-hops step with its launch (balanced)
    q = dit["q"]
    Lq = q.shape[1]
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, dit["k_chunks"], dit["scale"], 106.5)
    o, l = _hops_carry(dit, bw.BWA_MODE_GATED, m=m, gate=gate, balanced=True)
    assert o.dtype == BF16
    B, _, H, D = q.shape
    cut = _cut_blocks(B, H, Lq, dit["k_chunks"][0].shape[1], D)
    must = [0, Lq - 1] + sorted({r0 for _, _, r0, _ in cut})[:24]
    rows = synth.sample_rows(Lq, 512, seed=30, must=must)
    o_ref, l_ref = _dit_oracle(dit, rows)
    assert_close(*gpu_rows(o, l, rows), o_ref, l_ref, BF16, "dit balanced carried hops")
    o_p, l_p = _hops_carry(dit, bw.BWA_MODE_GATED, m=m, gate=gate)
    assert (l - l_p).abs().max().item() <= 1e-5
    assert (o.float() - o_p.float()).abs().max().item() <= 2 ** -7


def test_dit_all_heads_eligible():
    d = synth.make_dit_share(DEV, seed=1013, sink=False)
    q = d["q"]
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, d["k_chunks"], d["scale"], 106.5)
    assert torch.all(gate == 1)
    o, l = _hops(d, bw.BWA_MODE_FIXED_M, m=m)  # branch-free fixed-m body for every head
    rows = synth.sample_rows(q.shape[1], 512, seed=24, must=[0, q.shape[1] - 1])
    o_ref, l_ref = _dit_oracle(d, rows)
    assert_close(*gpu_rows(o, l, rows), o_ref, l_ref, BF16, "dit all eligible")


def test_dit_ragged_padded_last_shard(dit):
    # padding only at the end of the global sequence: the last shard's tail
    q, ks, vs = dit["q"], dit["k_chunks"], dit["v_chunks"]
    Lc = ks[1].shape[1]
    n_valid = Lc - 1000
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, ks, dit["scale"], 106.5, kv_valid=[Lc, n_valid])
    parts = []
    for t, (k, v) in enumerate(zip(ks, vs)):
        mask = {"kv_offset": t * Lc, "kv_valid": Lc if t == 0 else n_valid}
        parts.append(bw.bwa_attn_fwd(q, k, v, mask, scale=dit["scale"], mode=bw.BWA_MODE_GATED, m=m, gate=gate,
                                     out_dtype=torch.float32))
    o, l = bw.bwa_lse_merge([p[0] for p in parts], [p[1] for p in parts])
    rows = synth.sample_rows(q.shape[1], 128, seed=25, must=[0, q.shape[1] - 1])
    k_all = torch.cat([ks[0], ks[1][:, :n_valid]], dim=1)
    v_all = torch.cat([vs[0], vs[1][:, :n_valid]], dim=1)
    o_ref, l_ref = oracle_attention(q, k_all, v_all, {}, dit["scale"], rows)
    assert_close(*gpu_rows(o, l, rows), o_ref, l_ref, BF16, "dit padded shard")


# ------------------------------------------------------------------- 1M tokens
@pytest.fixture(scope="module")
def long():
    return synth.make_long_causal(DEV)


@pytest.mark.timeout(900)
def test_long_causal_single_segment(long):
    q, k, v, scale = long["q"], long["k"], long["v"], long["scale"]
    L = q.shape[1]
    bq, _ = bw.bwa_attn_tile(BF16, 128)
    plain = {"causal": True}
    seg1 = {"causal": True, "cu_seqlens_q": [0, L], "cu_seqlens_kv": [0, L]}
    b0 = bw.bwa_block_mask_build(plain, 1, L, L, bq, 128)
    b1 = bw.bwa_block_mask_build(seg1, 1, L, L, bq, 128)
    for x, y in zip(b0.host(), b1.host()):
        assert np.array_equal(x, y)
    o0, l0 = bw.bwa_attn_fwd(q, k, v, plain, blocks=b0, scale=scale)
    o1, l1 = bw.bwa_attn_fwd(q, k, v, seg1, blocks=b1, scale=scale)
    torch.cuda.synchronize()
    # one segment through the segmented path gives the unsegmented bits
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    bl128 = bw.bwa_block_mask_build(plain, 1, L, L, 128, 128)
    n_tiles, n_partial = _gpu_tile_counts(bl128, L, L, 128, 128)
    assert n_tiles == 8192 * 8193 // 2 and n_partial == 8192
    qbs = np.unique(np.concatenate([[0, 1, 8191], np.random.default_rng(3).choice(8192, 61, replace=False)]))
    _lists_match_oracle(bl128, plain, L, L, 128, 128, qblocks=qbs)
    rows = synth.sample_rows(L, 512, seed=26, must=[0, 1, 255, 256, L - 1])
    o_ref, l_ref = oracle_attention(q, k, v, plain, scale, rows)
    assert_close(*gpu_rows(o0, l0, rows), o_ref, l_ref, BF16, "1M causal")


@pytest.mark.timeout(900)
def test_long_causal_gated_balanced(long):
    # The fixed-m bound and gate on the 1M causal workload, the balanced launch
    # (the bench's --mode gated): every head passes the gate on these inputs
    # and runs the fixed-m body; the result is the oracle's within tolerance.
    q, k, v, scale = long["q"], long["k"], long["v"], long["scale"]
    L = q.shape[1]
    mask = {"causal": True}
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, [k], scale, 106.5)
    assert gate.all().item()
    bq, _ = bw.bwa_attn_tile(BF16, 128)
    blocks = bw.bwa_block_mask_build(mask, 1, L, L, bq, 128)
    o, l = bw.bwa_attn_fwd_balanced(q, k, v, mask, blocks=blocks, scale=scale, mode=bw.BWA_MODE_GATED, m=m,
                                    gate=gate)
    rows = synth.sample_rows(L, 512, seed=29, must=[0, 1, 255, 256, L - 1])
    o_ref, l_ref = oracle_attention(q, k, v, mask, scale, rows)
    assert_close(*gpu_rows(o, l, rows), o_ref, l_ref, BF16, "1M causal gated")


@pytest.mark.timeout(900)
def test_long_causal_packed(long):
    q, k, v, scale = long["q"], long["k"], long["v"], long["scale"]
    L, H = q.shape[1], q.shape[2]
    cu = synth.long_causal_segments(L)
    mask = {"causal": True, "cu_seqlens_q": cu, "cu_seqlens_kv": cu}
    bq, _ = bw.bwa_attn_tile(BF16, 128)
    blocks = bw.bwa_block_mask_build(mask, 1, L, L, bq, 128)
    o, l = bw.bwa_attn_fwd(q, k, v, mask, blocks=blocks, scale=scale)
    bl128 = bw.bwa_block_mask_build(mask, 1, L, L, 128, 128)
    qbs = np.unique(np.concatenate([[0, 8191], [c // 128 for c in cu[1:-1]],
                                    np.random.default_rng(4).choice(8192, 48, replace=False)]))
    _lists_match_oracle(bl128, mask, L, L, 128, 128, qblocks=qbs)
    must = [0, L - 1] + [c for c in cu[1:-1]] + [c - 1 for c in cu[1:-1]]
    rows = synth.sample_rows(L, 512, seed=27, must=must)
    # The oracle runs each sampled row inside its own segment (keys of other
    # segments are invisible by the definition): same rule, fewer keys.
    seg = np.searchsorted(np.asarray(cu), rows, side="right") - 1
    got_o, got_l = gpu_rows(o, l, rows)
    ref_o = np.zeros_like(got_o)
    ref_l = np.zeros_like(got_l)
    for s in np.unique(seg):
        a, e = cu[s], cu[s + 1]
        sel = np.nonzero(seg == s)[0]
        oo, ll = oracle_attention(q[:, a:e], k[:, a:e], v[:, a:e], {"causal": True}, scale, rows[sel] - a)
        ref_o[:, sel] = oo
        ref_l[:, :, sel] = ll
    assert_close(got_o, got_l, ref_o, ref_l, BF16, "1M packed")
