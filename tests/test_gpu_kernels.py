"""GPU parity of every entry point against the fp64 oracle at small sizes.

Sizes span several 128-row query blocks and 64-key tiles with ragged tails;
every mask kind, both dtypes, both head dims, online and fixed-m, with and
without precomputed run lists.  All calls go through the C ABI.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_close, mask_for_batch, np64, oracle_attention

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts too
    pytest.skip("needs a GPU", allow_module_level=True)

import blockwise_attention_forward_amd as bw  # noqa: E402

DEV = "cuda"


def _rand(shape, seed, dtype):
    return synth.normal(shape, seed, DEV, dtype)


def test_tiny_fp32_dense_and_chunk_merge():
    t = synth.make_tiny(DEV)
    q, k, v, scale = t["q"], t["k"], t["v"], t["scale"]
    o, lse = bw.bwa_attn_fwd(q, k, v, {}, scale=scale)
    o_ref, l_ref = oracle_attention(q, k, v, {}, scale)
    assert_close(o, lse, o_ref, l_ref, torch.float32, "tiny fp32")
    parts = []
    for a, e in t["chunks"]:
        parts.append(bw.bwa_attn_fwd(q, k[:, a:e], v[:, a:e], {"kv_offset": a}, scale=scale))
    om, lm = bw.bwa_lse_merge([p[0] for p in parts], [p[1] for p in parts], out_dtype=torch.float32)
    assert_close(om, lm, o_ref, l_ref, torch.float32, "tiny fp32 merged")


# document ids in any order, one row per batch element (two elements)
_DOCS = np.random.Generator(np.random.PCG64(404)).integers(0, 4, size=(2, 333)).astype(np.int32)

MASKS = [
    {},
    {"causal": True},
    {"causal": True, "window": 100},
    {"causal": True, "window": 1},
    {"causal": True, "kv_offset": 37},
    {"causal": True, "kv_offset": -120, "window": 200},
    {"q_valid": 290, "kv_valid": 301},
    {"q_valid": 0},
    {"kv_valid": 0},
    {"cu_seqlens_q": [0, 70, 200, 333], "cu_seqlens_kv": [0, 70, 200, 333]},
    {"cu_seqlens_q": [0, 150, 333], "cu_seqlens_kv": [0, 150, 333], "causal": True, "q_valid": 300},
    {"cu_seqlens_q": [5, 100, 300], "cu_seqlens_kv": [0, 60, 333], "causal": True, "window": 50},
    {"causal": True, "prefix": 100},                      # prefix-LM
    {"causal": True, "prefix": 300, "kv_offset": 40, "q_valid": 320},
    {"window": 60},                                       # two-sided band
    {"window": 50, "kv_offset": -40, "kv_valid": 310},
    {"causal": True, "window": 90, "dilation": 3},        # dilated band
    {"causal": True, "window": 200, "dilation": 70, "kv_offset": 20},
    {"segment_ids_q": _DOCS, "segment_ids_kv": _DOCS, "documents": True},
    {"segment_ids_q": _DOCS, "segment_ids_kv": _DOCS, "documents": True, "causal": True, "q_valid": 300},
]


def _contiguous_part(mask):
    """The terms of a mask that bound each row's keys to one interval: what
    the library's per-row intervals hold (dilation and document ids drop)."""
    m = dict(mask)
    m.pop("dilation", None)
    if m.pop("documents", False):
        m.pop("segment_ids_q", None)
        m.pop("segment_ids_kv", None)
    return m


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_masks_against_oracle(mi, D, dtype):
    mask = MASKS[mi]
    B, H, Lq, Lk = 2, 3, 333, 333
    q = _rand((B, Lq, H, D), 10 + mi, dtype)
    k = _rand((B, Lk, H, D), 20 + mi, dtype)
    v = _rand((B, Lk, H, D), 30 + mi, dtype)
    scale = 1 / math.sqrt(D)
    o_ref, l_ref = oracle_attention(q, k, v, mask, scale)
    o1, l1 = bw.bwa_attn_fwd(q, k, v, mask, scale=scale)
    assert_close(o1, l1, o_ref, l_ref, dtype, f"inline walk {mask}")
    bq, bkv = bw.bwa_attn_tile(dtype, D)
    blocks = bw.bwa_block_mask_build(mask, B, Lq, Lk, bq, 128)
    o2, l2 = bw.bwa_attn_fwd(q, k, v, mask, blocks=blocks, scale=scale)
    assert_close(o2, l2, o_ref, l_ref, dtype, f"run lists {mask}")
    # the two tile walks visit the same tiles in the same order
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# Masks whose rows see many keys: the plain bf16 launch runs whole blocks
# (rows with few keys, as in the suite above, run half blocks).
LONG_ROW_MASKS = [
    {},
    {"causal": True, "kv_offset": 300 - 9000},
    {"causal": True, "kv_offset": 300 - 9000, "window": 5000, "dilation": 3},
    {"window": 2500, "kv_offset": 4000},
]


# Dilated bands whose lengths, kv_offset and valid counts are multiples of the
# dilation g run as g strided causal windows (one launch per batch element,
# the residue class as its batch index); the others walk the band with the
# element test.  (g, window, Lq, Lk, kv_offset, q_valid, kv_valid)
DILATED_SPLIT = [
    (2, 100, 768, 768, 0, 768, 768),
    (3, 257, 768, 960, -192, 720, 900),
    (4, 1024, 768, 768, 0, 768, 768),
    (4, 301, 512, 1024, -512, 512, 1000),
    (5, 64, 640, 640, 0, 600, 640),
    (4, 130, 768, 768, 2, 768, 768),  # kv_offset not a multiple of g: the element test
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("ci", range(len(DILATED_SPLIT)))
def test_dilated_band_as_strided_windows(ci, D, dtype):
    g, w, Lq, Lk, off, qv, kvv = DILATED_SPLIT[ci]
    B, H, Hk = 2, 4, 2
    mask = {"causal": True, "window": w, "dilation": g, "kv_offset": off, "q_valid": qv, "kv_valid": kvv}
    q = _rand((B, Lq, H, D), 40 + ci, dtype)
    k = _rand((B, Lk, Hk, D), 50 + ci, dtype)
    v = _rand((B, Lk, Hk, D), 60 + ci, dtype)
    scale = 1 / math.sqrt(D)
    o_ref, l_ref = oracle_attention(q, k, v, mask, scale)
    o, lse = bw.bwa_attn_fwd(q, k, v, mask, scale=scale)
    assert_close(o, lse, o_ref, l_ref, dtype, f"dilated {DILATED_SPLIT[ci]}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mi", range(len(LONG_ROW_MASKS)))
def test_whole_block_launch_long_rows(mi, D):
    mask = LONG_ROW_MASKS[mi]
    B, H, Lq, Lk = 1, 2, 300, 9000
    q = _rand((B, Lq, H, D), 40 + mi, torch.bfloat16)
    k = _rand((B, Lk, H, D), 50 + mi, torch.bfloat16)
    v = _rand((B, Lk, H, D), 60 + mi, torch.bfloat16)
    scale = 1 / math.sqrt(D)
    o_ref, l_ref = oracle_attention(q, k, v, mask, scale)
    o, l = bw.bwa_attn_fwd(q, k, v, mask, scale=scale)
    assert_close(o, l, o_ref, l_ref, torch.bfloat16, f"whole blocks {mask}")


@pytest.mark.parametrize("Lq,Lk", [(1, 1), (5, 700), (700, 5), (129, 64), (64, 129)])
def test_shapes(Lq, Lk):
    B, H, D = 1, 2, 128
    q, k, v = (_rand((B, L, H, D), s, torch.bfloat16) for L, s in ((Lq, 1), (Lk, 2), (Lk, 3)))
    for mask in ({}, {"causal": True, "kv_offset": Lq - Lk}):
        o_ref, l_ref = oracle_attention(q, k, v, mask, 0.1)
        o, l = bw.bwa_attn_fwd(q, k, v, mask, scale=0.1)
        assert_close(o, l, o_ref, l_ref, torch.bfloat16, f"{Lq}x{Lk} {mask}")


def test_empty_inputs():
    q = _rand((1, 0, 2, 128), 1, torch.bfloat16)
    k = _rand((1, 10, 2, 128), 2, torch.bfloat16)
    o, l = bw.bwa_attn_fwd(q, k, k, {})
    assert o.shape[1] == 0
    q = _rand((1, 50, 2, 128), 1, torch.bfloat16)
    k0 = _rand((1, 0, 2, 128), 2, torch.bfloat16)
    o, l = bw.bwa_attn_fwd(q, k0, k0, {})
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))


def test_segment_ids_per_batch_and_strided_views():
    B, H, L, D = 2, 2, 300, 128
    ids = np.stack([np.sort(np.random.default_rng(s).integers(0, 4, L)) for s in (1, 2)]).astype(np.int32)
    mask = {"segment_ids_q": ids, "segment_ids_kv": ids, "causal": True}
    qkv = _rand((B, L, 3 * H, D), 5, torch.bfloat16)  # packed projection: strided views
    q, k, v = qkv[:, :, :H], qkv[:, :, H:2 * H], qkv[:, :, 2 * H:]
    o_ref, l_ref = oracle_attention(q, k, v, mask, 0.09)
    o, l = bw.bwa_attn_fwd(q, k, v, mask, scale=0.09)
    assert_close(o, l, o_ref, l_ref, torch.bfloat16, "segment ids, inline")
    bq, _ = bw.bwa_attn_tile(torch.bfloat16, D)
    blocks = bw.bwa_block_mask_build(mask, B, L, L, bq, 64)
    o2, l2 = bw.bwa_attn_fwd(q, k, v, mask, blocks=blocks, scale=0.09)
    assert torch.equal(o, o2) and torch.equal(l, l2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_head_major_and_padded_layouts(dtype):
    # K/V rows whose L stride is exactly D (head-major views of [B, H, L, D])
    # or wider than a token (padded pitch) read every valid row, and rows past
    # kv_valid as nothing; the same results as contiguous token-major copies.
    B, H, Lq, Lk, D = 1, 2, 300, 333, 128
    q = _rand((B, H, Lq, D), 11, dtype).transpose(1, 2)
    k = _rand((B, H, Lk, D), 12, dtype).transpose(1, 2)
    vp = _rand((B, Lk, H, D + 64), 13, dtype)[..., :D]  # row pitch H * (D + 64)
    mask = {"causal": True, "kv_offset": Lq - Lk, "kv_valid": 301}
    o_ref, l_ref = oracle_attention(q, k, vp, mask, 0.1)
    o, l = bw.bwa_attn_fwd(q, k, vp, mask, scale=0.1)
    assert_close(o, l, o_ref, l_ref, dtype, "head-major / padded")
    o2, l2 = bw.bwa_attn_fwd(q.contiguous(), k.contiguous(), vp.contiguous(), mask, scale=0.1)
    assert torch.equal(o, o2) and torch.equal(l, l2)


def test_overlapping_layouts_are_rejected():
    q = _rand((1, 200, 2, 128), 1, torch.bfloat16)
    k1 = _rand((1, 1, 2, 128), 2, torch.bfloat16)
    kx = k1.expand(1, 200, 2, 128)  # one key broadcast along L: stride 0
    with pytest.raises(bw.BwaError) as e:
        bw.bwa_attn_fwd(q, kx, kx, {})
    assert e.value.status == 3
    with pytest.raises(bw.BwaError):
        bw.bwa_attn_fwd(q, k1.expand(1, 200, 2, 128).contiguous(), kx, {})
    with pytest.raises(bw.BwaError):
        bw.bwa_fixed_m_bound(q, [kx], 0.1, 106.5)


@pytest.mark.parametrize("mi", range(len(MASKS)))
@pytest.mark.parametrize("bq,bkv", [(128, 128), (128, 64), (64, 192)])
def test_block_lists_bit_exact(mi, bq, bkv):
    mask = MASKS[mi]
    Lq = Lk = 333
    bl = bw.bwa_block_mask_build(mask, 1, Lq, Lk, bq, bkv)
    rp, b, e, k = bl.host()
    m0 = mask_for_batch(mask, 0)
    want = oracle.block_lists(m0, Lq, Lk, bq, bkv)
    assert np.array_equal(rp, want[0]) and np.array_equal(b, want[1])
    assert np.array_equal(e, want[2]) and np.array_equal(k, want[3])
    lo, hi = oracle.row_intervals_bruteforce(Lq, Lk, _contiguous_part(m0))
    assert np.array_equal(bl.row_lo[:Lq].cpu().numpy(), lo)
    assert np.array_equal(bl.row_hi[:Lq].cpu().numpy(), hi)


@pytest.mark.parametrize("Hk", [1, 2, 6])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_grouped_query_heads(Hk, dtype):
    # 6 query heads on Hk key/value heads (multi-query at 1, one each at 6),
    # plain and balanced launch, fixed-m bound per key head
    B, H, Lq, Lk, D = 2, 6, 333, 401, 128
    scale = 1 / math.sqrt(D)
    q = _rand((B, Lq, H, D), 60, dtype)
    k = _rand((B, Lk, Hk, D), 61, dtype)
    v = _rand((B, Lk, Hk, D), 62, dtype)
    mask = {"causal": True, "kv_offset": 68}
    o_ref, l_ref = oracle_attention(q, k, v, mask, scale)
    o, l = bw.bwa_attn_fwd(q, k, v, mask, scale=scale, out_dtype=torch.float32)
    assert_close(o, l, o_ref, l_ref, dtype, f"gqa Hk={Hk}")
    if dtype == torch.bfloat16:
        bq, _ = bw.bwa_attn_tile(dtype, D)
        blocks = bw.bwa_block_mask_build(mask, B, Lq, Lk, bq, 64)
        ob, lb = bw.bwa_attn_fwd_balanced(q, k, v, mask, blocks=blocks, scale=scale, n_cus=16,
                                          out_dtype=torch.float32)
        assert_close(ob, lb, o_ref, l_ref, dtype, f"gqa balanced Hk={Hk}")
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, [k], scale, 106.5)
    for b in range(B):
        for h in range(H):
            km, mr, mm, gh = oracle.fixed_m_bound(np64(q[b, :, h]), [np64(k[b, :, oracle.kv_head(h, H, Hk)])],
                                                  scale, 106.5)
            np.testing.assert_allclose(kmax[b, h].item(), km, rtol=1e-6)
            np.testing.assert_allclose(np64(m[b, h]), mr, rtol=2e-6)
            assert bool(gate[b, h].item()) == gh
    o2, l2 = bw.bwa_attn_fwd(q, k, v, mask, scale=scale, mode=bw.BWA_MODE_FIXED_M, m=m, out_dtype=torch.float32)
    assert_close(o2, l2, o_ref, l_ref, dtype, f"gqa fixed-m Hk={Hk}")


def test_document_lists_per_batch_and_balanced_refusal():
    # document ids differ per batch element: one list copy each; the balanced
    # launch does not take element-test masks
    B, H, L, D = 2, 2, 333, 128
    mask = {"segment_ids_q": _DOCS, "segment_ids_kv": _DOCS, "documents": True, "causal": True}
    bq, _ = bw.bwa_attn_tile(torch.bfloat16, D)
    bl = bw.bwa_block_mask_build(mask, B, L, L, bq, 64)
    assert bl.struct.batch == B
    for b in range(B):
        rp, be, en, kd = bl.host(b)
        want = oracle.block_lists(mask_for_batch(mask, b), L, L, bq, 64)
        assert all(np.array_equal(x, y) for x, y in zip((rp, be, en, kd), want))
    q, k, v = (_rand((B, L, H, D), 70 + s, torch.bfloat16) for s in range(3))
    with pytest.raises(bw.BwaError) as e:
        bw.bwa_attn_fwd_balanced(q, k, v, mask, blocks=bl, n_cus=16)
    assert e.value.status == 6


def test_fixed_m_bound_and_gate():
    B, H, D = 2, 4, 128
    q = _rand((B, 300, H, D), 40, torch.bfloat16)
    ks = [_rand((B, n, H, D), 41 + i, torch.bfloat16) for i, n in enumerate((200, 170))]
    ks[1][1, 7, 2] *= 50  # sink key in (b=1, h=2)
    kv_valid = [200, 160]
    ks[1][0, 165, 0] *= 1e3  # past kv_valid: must not enter the bound
    kmax_in = torch.zeros(2, B, H, device=DEV)
    kmax_in[0, 0, 3] = 400.0  # promoted to the global bound of (b=0, h=3)
    scale = 1 / math.sqrt(D)
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, ks, scale, 106.5, kmax_in=kmax_in, kv_valid=kv_valid,
                                               q_valid=290)
    for b in range(B):
        for h in range(H):
            km, mr, mm, g = oracle.fixed_m_bound(np64(q[b, :, h]), [np64(c[b, :, h]) for c in ks], scale,
                                                 106.5, q_valid=290, kv_valid=kv_valid,
                                                 kmax_in=np64(kmax_in[:, b, h]))
            np.testing.assert_allclose(kmax[b, h].item(), km, rtol=1e-6)
            np.testing.assert_allclose(np64(m[b, h]), mr, rtol=2e-6)
            np.testing.assert_allclose(mmax[b, h].item(), mm, rtol=2e-6)
            assert bool(gate[b, h].item()) == g
    assert gate[1, 2].item() == 0 and gate[0, 3].item() == 0


@pytest.mark.parametrize("B,L,H,D,dtype", [
    (3, 50, 4, 128, torch.bfloat16),   # several batch elements inside one workgroup's row stretch
    (2, 1500, 5, 64, torch.bfloat16),  # stretches straddle batch boundaries
    (2, 9, 300, 64, torch.float32),    # more heads than the per-head LDS table
    (1, 4097, 3, 128, torch.float32),
])
def test_fixed_m_bound_batch_and_head_layouts(B, L, H, D, dtype):
    q = _rand((B, L, H, D), 44, dtype)
    ks = [_rand((B, L + 3, H, D), 45, dtype), _rand((B, max(L // 2, 1), H, D), 46, dtype)]
    for b in range(B):
        ks[b % 2][b, 1, b % H] *= 20.0  # a distinct maximum per batch element
        q[b, L - 1, (b + 1) % H] *= 7.0
    scale = 1 / math.sqrt(D)
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, ks, scale, 106.5)
    for b in range(B):
        for h in range(H):
            km, mr, mm, g = oracle.fixed_m_bound(np64(q[b, :, h]), [np64(c[b, :, h]) for c in ks], scale, 106.5)
            np.testing.assert_allclose(kmax[b, h].item(), km, rtol=1e-6)
            np.testing.assert_allclose(np64(m[b, h]), mr, rtol=2e-6)
            np.testing.assert_allclose(mmax[b, h].item(), mm, rtol=2e-6)
            assert bool(gate[b, h].item()) == g


@pytest.mark.parametrize("D", [64, 128])
def test_fixed_m_attention_and_gated_pair(D):
    B, H, Lq, Lk = 1, 4, 300, 400
    scale = 1 / math.sqrt(D)
    q = _rand((B, Lq, H, D), 50, torch.bfloat16)
    k = _rand((B, Lk, H, D), 51, torch.bfloat16)
    v = _rand((B, Lk, H, D), 52, torch.bfloat16)
    k[0, 11, 1] *= 50  # head 1 fails the gate
    for mask in ({}, {"causal": True, "kv_offset": -100}):
        kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, [k], scale, 106.5)
        assert gate[0].tolist() == [1, 0, 1, 1]
        o_ref, l_ref = oracle_attention(q, k, v, mask, scale)
        # every head in fixed-m mode: exact for the eligible heads
        o, l = bw.bwa_attn_fwd(q, k, v, mask, scale=scale, mode=bw.BWA_MODE_FIXED_M, m=m,
                               out_dtype=torch.float32)
        for h in (0, 2, 3):
            assert_close(o[:, :, h:h + 1], l[:, h:h + 1], o_ref[:, :, h:h + 1], l_ref[:, h:h + 1],
                         torch.bfloat16, f"fixed-m head {h}")
        # gated pair: fixed-m on passing heads, online on the failing head
        o2 = torch.full_like(o, float("nan"))
        l2 = torch.full_like(l, float("nan"))
        bw.bwa_attn_fwd(q, k, v, mask, scale=scale, mode=bw.BWA_MODE_FIXED_M, m=m, gate=gate, o=o2, lse=l2)
        bw.bwa_attn_fwd(q, k, v, mask, scale=scale, mode=bw.BWA_MODE_ONLINE, gate=gate, o=o2, lse=l2)
        assert_close(o2, l2, o_ref, l_ref, torch.bfloat16, "gated pair")
        # one gated launch: the same two loops chosen per workgroup, same bits
        o3, l3 = bw.bwa_attn_fwd(q, k, v, mask, scale=scale, mode=bw.BWA_MODE_GATED, m=m, gate=gate,
                                 out_dtype=torch.float32)
        assert torch.equal(o3, o2) and torch.equal(l3, l2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_fixed_m_rows_far_below_their_bound(dtype):
    # Rows whose every key points away from the query with the largest norm:
    # all scores sit near -m_i, about 2 m_i below the bound.  Head 0's bound
    # is just under the largest one the fixed-m arithmetic proves safe, so it
    # passes the gate and its rows sit ~72 below m_i; head 1's bound (~100)
    # is under the page's 106.5 but out of that range, so it fails the gate
    # and takes the online loop.  Both must match the oracle, in fixed-m,
    # gated and balanced launches.
    B, H, Lq, Lk, D = 1, 2, 300, 700, 128
    scale = 1 / math.sqrt(D)
    g = torch.Generator(device="cpu").manual_seed(60)
    qdir = torch.randn(H, D, generator=g, dtype=torch.float64)
    qdir /= qdir.norm(dim=1, keepdim=True)
    a = torch.rand(Lk, H, generator=g, dtype=torch.float64) * 0.1 + 0.9
    a[0] = 1.0
    k = (-a[:, :, None] * qdir[None]).unsqueeze(0)
    m_target = torch.tensor([0.99 * oracle.fixed_m_safe_max(), 100.0], dtype=torch.float64)
    qn = (m_target / scale) * (0.95 + 0.05 * torch.rand(Lq, H, generator=g, dtype=torch.float64))
    q = (qn[:, :, None] * qdir[None]).unsqueeze(0)
    q, k = q.to(DEV, dtype), k.to(DEV, dtype)
    v = _rand((B, Lk, H, D), 61, dtype)
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, [k], scale, 106.5)
    assert gate[0].tolist() == [1, 0] and mmax[0, 1].item() < 106.5
    for h in range(H):
        assert oracle.fixed_m_bound(np64(q[0, :, h]), [np64(k[0, :, h])], scale, 106.5)[3] == (h == 0)
    o_ref, l_ref = oracle_attention(q, k, v, {}, scale)
    s_max = (np64(q[0, :, 0]) @ np64(k[0, :, 0]).T).max(axis=1) * scale
    assert np.all(np64(m[0, 0]) - s_max > 70.0)
    o, l = bw.bwa_attn_fwd(q, k, v, {}, scale=scale, mode=bw.BWA_MODE_FIXED_M, m=m, gate=gate,
                           out_dtype=torch.float32)
    assert_close(o[:, :, :1], l[:, :1], o_ref[:, :, :1], l_ref[:, :1], dtype, "fixed-m, rows far below m")
    o2, l2 = bw.bwa_attn_fwd(q, k, v, {}, scale=scale, mode=bw.BWA_MODE_GATED, m=m, gate=gate,
                             out_dtype=torch.float32)
    assert_close(o2, l2, o_ref, l_ref, dtype, "gated")
    assert torch.equal(o2[:, :, :1], o[:, :, :1]) and torch.equal(l2[:, :1], l[:, :1])
    if dtype == torch.bfloat16:
        o3, l3 = bw.bwa_attn_fwd_balanced(q, k, v, {}, scale=scale, mode=bw.BWA_MODE_GATED, m=m, gate=gate,
                                          n_cus=16, out_dtype=torch.float32)
        assert_close(o3, l3, o_ref, l_ref, dtype, "gated, balanced")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", [{}, {"causal": True}])
def test_online_reference_moves_mid_walk(D, mask):
    """Online softmax with rows whose max jumps far past their running
    reference (by much more than the lazy margin) after earlier tiles have
    been accumulated, in the middle and in the ragged last tile of the key
    walk: the rare rescale, and the redo of a half's exponentials in the
    online-only launches, against the oracle (plain and balanced launches)."""
    B, H, L = 1, 3, 700
    dtype = torch.bfloat16
    q = _rand((B, L, H, D), 90, dtype)
    k = _rand((B, L, H, D), 91, dtype)
    v = _rand((B, L, H, D), 92, dtype)
    k[0, 300, 0] *= 30
    k[0, 333, 1] *= 12
    k[0, 20, 2] *= 8
    k[0, 690, 2] *= 60
    scale = 1 / math.sqrt(D)
    o_ref, l_ref = oracle_attention(q, k, v, mask, scale)
    o1, l1 = bw.bwa_attn_fwd(q, k, v, mask, scale=scale, mode=bw.BWA_MODE_ONLINE)
    assert_close(o1, l1, o_ref, l_ref, dtype, f"plain {mask}")
    o2, l2 = bw.bwa_attn_fwd_balanced(q, k, v, mask, scale=scale, mode=bw.BWA_MODE_ONLINE, n_cus=4)
    assert_close(o2, l2, o_ref, l_ref, dtype, f"balanced {mask}")


@pytest.mark.parametrize("n_parts", [1, 2, 3])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_lse_merge_against_oracle(n_parts, out_dtype):
    B, L, H, D = 2, 77, 3, 128
    g = torch.Generator(device=DEV).manual_seed(60 + n_parts)
    os_ = [torch.randn(B, L, H, D, device=DEV, generator=g) for _ in range(n_parts)]
    ls = [torch.randn(B, H, L, device=DEV, generator=g) * 5 for _ in range(n_parts)]
    for t in range(n_parts):
        ls[t][0, 0, :10] = -float("inf")  # rows some chunk did not see
    ls[0][1, 2, 5] = -float("inf")
    if n_parts > 1:
        for t in range(n_parts):
            ls[t][1, 1, 3] = -float("inf")  # row no chunk saw
            os_[t][1, 3, 1] = 0
    o, l = bw.bwa_lse_merge(os_, ls, out_dtype=out_dtype)
    ref_o, ref_l = oracle.lse_merge([(np64(a).transpose(0, 2, 1, 3), np64(b)) for a, b in zip(os_, ls)])
    ref_o = ref_o.transpose(0, 2, 1, 3)
    got_l = np64(l)
    assert np.array_equal(np.isneginf(got_l), np.isneginf(ref_l))
    f = np.isfinite(ref_l)
    np.testing.assert_allclose(got_l[f], ref_l[f], atol=1e-5, rtol=0)
    tol = 1e-5 if out_dtype == torch.float32 else 1e-2
    np.testing.assert_allclose(np64(o), ref_o, atol=tol, rtol=0 if out_dtype == torch.float32 else 8e-3)


@pytest.mark.parametrize("D", [64, 128])
def test_lse_merge_dead_parts_and_strided_views(D):
    # A part whose LSE is -inf on a row has weight 0 there: its O row is not
    # used, so NaN in it must not reach the result.  Parts are strided views.
    B, L, H = 2, 300, 3
    g = torch.Generator(device=DEV).manual_seed(66)
    big = [torch.randn(B, L, H + 1, 2 * D, device=DEV, generator=g) for _ in range(2)]
    os_ = [x[:, :, 1:, :D] for x in big]
    ls = [torch.randn(B, H, L, device=DEV, generator=g) * 3 for _ in range(2)]
    ls[1][0, 1, 100:180] = -float("inf")
    os_[1][0, 100:180, 1] = float("nan")
    ls[0][1, 2, 250:] = -float("inf")
    ls[1][1, 2, 250:] = -float("inf")
    os_[0][1, 250:, 2] = float("nan")
    out = torch.empty(B, L, H + 2, D, device=DEV)[:, :, 2:]
    o, l = bw.bwa_lse_merge(os_, ls, o_out=out, out_dtype=torch.float32)
    clean = [torch.where(torch.isneginf(lt).permute(0, 2, 1)[..., None], torch.zeros_like(ot), ot)
             for ot, lt in zip(os_, ls)]
    ref_o, ref_l = oracle.lse_merge([(np64(a).transpose(0, 2, 1, 3), np64(b)) for a, b in zip(clean, ls)])
    ref_o = ref_o.transpose(0, 2, 1, 3)
    got_o, got_l = np64(o), np64(l)
    assert np.all(np.isfinite(got_o))
    assert np.array_equal(np.isneginf(got_l), np.isneginf(ref_l))
    assert np.all(got_o[1, 250:, 2] == 0)
    f = np.isfinite(ref_l)
    np.testing.assert_allclose(got_l[f], ref_l[f], atol=1e-5, rtol=0)
    np.testing.assert_allclose(got_o, ref_o, atol=1e-5, rtol=0)


@pytest.mark.parametrize("D,dtype", [(128, torch.bfloat16), (64, torch.bfloat16), (128, torch.float32)])
@pytest.mark.parametrize("mode", ["online", "fixed", "gated"])
def test_attn_fwd_carry_two_chunks(D, dtype, mode):
    # Two key chunks of one causal sequence: chunk 0 = keys [0, 200), chunk 1 =
    # keys [200, 370).  Hop 0 writes an fp32 partial, hop 1 merges into it.
    B, H, Lq, L0, L1 = 2, 3, 300, 200, 170
    scale = 1 / math.sqrt(D)
    q = _rand((B, Lq, H, D), 80, dtype)
    k = _rand((B, L0 + L1, H, D), 81, dtype)
    v = _rand((B, L0 + L1, H, D), 82, dtype)
    k[1, 5, 2] *= 30  # head 2 of batch 1 fails the gate
    ks, vs = [k[:, :L0], k[:, L0:]], [v[:, :L0], v[:, L0:]]
    masks = [{"causal": True, "kv_offset": 0, "q_valid": 290}, {"causal": True, "kv_offset": L0, "q_valid": 290}]
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, ks, scale, 106.5, q_valid=290)
    args = {"online": dict(mode=bw.BWA_MODE_ONLINE),
            "fixed": dict(mode=bw.BWA_MODE_FIXED_M, m=m),
            "gated": dict(mode=bw.BWA_MODE_GATED, m=m, gate=gate)}[mode]
    o_ref, l_ref = oracle_attention(q, k, v, {"causal": True, "q_valid": 290}, scale)
    heads = [0, 1, 2] if mode != "fixed" else [0, 1]  # fixed-m is exact only for heads that pass the gate
    if mode == "fixed":
        assert gate[0].tolist() == [1, 1, 1] and gate[1, 2].item() == 0
    o0, l0 = bw.bwa_attn_fwd(q, ks[0], vs[0], masks[0], scale=scale, out_dtype=torch.float32, **args)
    for out_dtype in (torch.float32, dtype):
        o, l = bw.bwa_attn_fwd_carry(q, ks[1], vs[1], o0, l0, masks[1], scale=scale, out_dtype=out_dtype, **args)
        assert_close(o[:, :, heads], l[:, heads], o_ref[:, :, heads], l_ref[:, heads], dtype, f"carry {mode}")
    # same result as two partials merged by bwa_lse_merge
    o1, l1 = bw.bwa_attn_fwd(q, ks[1], vs[1], masks[1], scale=scale, out_dtype=torch.float32, **args)
    om, lm = bw.bwa_lse_merge([o0, o1], [l0, l1], out_dtype=torch.float32)
    oc, lc = bw.bwa_attn_fwd_carry(q, ks[1], vs[1], o0, l0, masks[1], scale=scale, out_dtype=torch.float32, **args)
    assert torch.equal(torch.isneginf(lc), torch.isneginf(lm))
    fin = torch.isfinite(lm)
    assert (lc[fin] - lm[fin]).abs().max().item() <= 1e-5
    assert (oc - om).abs().max().item() <= 1e-5
    # in place: the carried partial is overwritten by the merged result
    oi, li = o0.clone(), l0.clone()
    bw.bwa_attn_fwd_carry(q, ks[1], vs[1], oi, li, masks[1], scale=scale, o=oi, lse=li, **args)
    assert torch.equal(oi, oc) and torch.equal(li, lc)


def test_attn_fwd_carry_dead_sides_and_nan():
    # Rows the carried partial never saw (lse_prev = -inf) ignore its O rows,
    # NaN included; rows neither side sees come out 0 / -inf.
    B, H, Lq, Lk, D = 1, 2, 200, 150, 128
    scale = 1 / math.sqrt(D)
    q = _rand((B, Lq, H, D), 90, torch.bfloat16)
    k = _rand((B, Lk, H, D), 91, torch.bfloat16)
    v = _rand((B, Lk, H, D), 92, torch.bfloat16)
    mask = {"causal": True, "kv_offset": 40, "q_valid": 190}  # rows < 40 see nothing in this chunk
    o_prev = torch.randn(B, Lq, H, D, device=DEV)
    l_prev = torch.randn(B, H, Lq, device=DEV)
    l_prev[0, 0, 100:] = -float("inf")
    o_prev[0, 100:, 0] = float("nan")
    l_prev[0, 1, :30] = -float("inf")  # rows 0..29 of head 1: empty on both sides
    o, l = bw.bwa_attn_fwd_carry(q, k, v, o_prev, l_prev, mask, scale=scale, out_dtype=torch.float32)
    cur_o, cur_l = oracle_attention(q, k, v, mask, scale)
    prev_o = np64(o_prev).transpose(0, 2, 1, 3)
    prev_o[np.isneginf(np64(l_prev))] = 0.0
    ref_o, ref_l = oracle.lse_merge([(cur_o.transpose(0, 2, 1, 3), cur_l), (prev_o, np64(l_prev))])
    got_o, got_l = np64(o), np64(l)
    assert np.all(np.isfinite(got_o))
    assert np.array_equal(np.isneginf(got_l), np.isneginf(ref_l))
    assert np.all(got_o[0, :30, 1] == 0) and np.all(np.isneginf(got_l[0, 1, :30]))
    f = np.isfinite(ref_l)
    np.testing.assert_allclose(got_l[f], ref_l[f], atol=1e-3, rtol=0)
    np.testing.assert_allclose(got_o, ref_o.transpose(0, 2, 1, 3), atol=2e-2, rtol=0)


def test_deterministic_repeat():
    B, H, L, D = 1, 4, 500, 128
    q, k, v = (_rand((B, L, H, D), s, torch.bfloat16) for s in (70, 71, 72))
    mask = {"causal": True, "window": 200}
    outs = [bw.bwa_attn_fwd(q, k, v, mask) for _ in range(2)]
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mode", ["online", "fixed", "gated"])
@pytest.mark.parametrize("balanced", [False, True])
def test_keys_past_kv_valid_never_reach_the_result(D, mode, balanced):
    # Keys at and past kv_valid hold NaN and Inf: their rows fall outside the
    # K/V copy ranges and read as zero, and the mask hides them, so the call
    # equals attention over the truncated keys (the oracle's "padded keys
    # masked equals truncated keys").
    B, H, Lq, Lk, kv_valid = 1, 2, 300, 700, 530
    scale = 1 / math.sqrt(D)
    q = _rand((B, Lq, H, D), 90, torch.bfloat16)
    k = _rand((B, Lk, H, D), 91, torch.bfloat16)
    v = _rand((B, Lk, H, D), 92, torch.bfloat16)
    k[:, kv_valid:] = float("nan")
    v[:, kv_valid:] = float("inf")
    kt, vt = k[:, :kv_valid].contiguous(), v[:, :kv_valid].contiguous()
    mask = {"kv_valid": kv_valid}
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, [k], scale, 106.5, kv_valid=[kv_valid])
    assert gate.all().item()
    args = {"online": dict(mode=bw.BWA_MODE_ONLINE),
            "fixed": dict(mode=bw.BWA_MODE_FIXED_M, m=m),
            "gated": dict(mode=bw.BWA_MODE_GATED, m=m, gate=gate)}[mode]
    call = bw.bwa_attn_fwd_balanced if balanced else bw.bwa_attn_fwd
    o, l = call(q, k, v, mask, scale=scale, **args)
    assert torch.isfinite(o).all() and torch.isfinite(l).all()
    o_ref, l_ref = oracle_attention(q, kt, vt, {}, scale)
    assert_close(o, l, o_ref, l_ref, torch.bfloat16, f"kv_valid {mode}")
