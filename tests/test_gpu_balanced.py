"""GPU parity of the balanced launch (bwa_attn_fwd_balanced) through the C ABI.

One workgroup per compute unit takes whole query blocks, then pieces of the
last blocks cut along their key tiles, from a queue; a second kernel merges
the pieces in LSE space.  Checked here, with workgroup counts that give
several queue rounds and cut blocks at these sizes: the result against the
fp64 oracle; rows of whole blocks bit-identical to the plain launch and rows
of cut blocks close to it; determinism whatever the workspace held before;
pieces without tiles and blocks that see nothing; gate-skipped heads left
untouched; every mode and both head dims; workspace reuse and size errors.
"""

import math

import numpy as np
import pytest
import torch

import synth
from helpers import assert_close, oracle_attention

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts too
    pytest.skip("needs a GPU", allow_module_level=True)

import blockwise_attention_forward_amd as bw  # noqa: E402

DEV = "cuda"


def _rand(shape, seed):
    return synth.normal(shape, seed, DEV, torch.bfloat16)


def _blocks(mask, B, Lq, Lk, D, bkv=64):
    bq, _ = bw.bwa_attn_tile(torch.bfloat16, D)
    return bw.bwa_block_mask_build(mask, B, Lq, Lk, bq, bkv)


def _plan(B, H, Lq, Lk, D, n_cus):
    return bw.bwa_attn_fwd_balanced_workspace(torch.bfloat16, B, H, Lq, Lk, D, n_cus, plan=True)


def _tail_rows(B, H, Lq, D, n_cus, pieces):
    """Boolean [B, H, Lq]: rows of the cut query blocks.  Blocks in launch
    order (head-major, query blocks last-first within a head) are dealt to 8
    XCD shares of q or q + 1 contiguous blocks; with c = n_cus // 8 workgroups
    per XCD, a share's blocks past its last whole round of c are cut (when
    the plan cuts at all, pieces > 1)."""
    bq, _ = bw.bwa_attn_tile(torch.bfloat16, D)
    nqb = (Lq + bq - 1) // bq
    U = B * H * nqb
    if n_cus <= 0:
        n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    c = max(1, n_cus // 8)
    q, r = divmod(U, 8)
    tail = np.zeros((B, H, Lq), dtype=bool)
    n_cut = 0
    for x in range(8):
        u = q + (1 if x < r else 0)
        a = x * q + min(x, r)
        d = (u // c) * c if pieces > 1 else u
        for unit in range(a + d, a + u):
            bh, qb = unit // nqb, nqb - 1 - unit % nqb
            tail[bh // H, bh % H, qb * bq:(qb + 1) * bq] = True
            n_cut += 1
    return torch.as_tensor(tail, device=DEV), n_cut


def _check_vs_plain(o_sp, l_sp, o_pl, l_pl, tail, what):
    """Rows of whole blocks: the plain launch's bits.  Cut rows: one LSE-space
    combine of partials more, and in the online body each piece rounds its
    probabilities to bf16 against its own running max, so O differs at bf16
    rounding level of P (relative 2^-9 per element); row sums and LSE at fp32
    level."""
    whole = ~tail
    ot = tail.permute(0, 2, 1)  # [B, Lq, H]
    assert torch.equal(l_sp[whole], l_pl[whole]), what
    assert torch.equal(o_sp[~ot], o_pl[~ot]), what
    assert torch.equal(torch.isneginf(l_sp), torch.isneginf(l_pl)), what
    fin = torch.isfinite(l_pl) & tail
    dl = (l_sp[fin] - l_pl[fin]).abs()
    assert dl.numel() == 0 or bool((dl <= 1e-5 + 1e-6 * l_pl[fin].abs()).all()), (what, dl.max().item())
    if ot.any():
        err = (o_sp[ot].float() - o_pl[ot].float()).abs()
        assert err.max().item() <= 4e-3 and err.mean().item() <= 3e-4, (what, err.max().item(), err.mean().item())


MASKS = [
    {},
    {"causal": True},
    {"causal": True, "window": 300},
    {"q_valid": 700, "kv_valid": 901},
    {"cu_seqlens_q": [0, 70, 600, 1000, 1100], "cu_seqlens_kv": [0, 70, 600, 1000, 1100], "causal": True},
]


@pytest.mark.parametrize("n_cus", [0, 7, 16, 29])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_balanced_against_oracle_and_plain(mi, D, n_cus):
    # 30 query blocks of an 18-tile walk in XCD shares of 4 or 3, cut in 2:
    # all of them on the device's units (0); none on 7 workgroups (one unit
    # per XCD; the eighth share has no workgroup of its own and is taken over
    # by the others); 2 on 16 (2 units per XCD); 6 on 29 (3 per XCD).
    mask = MASKS[mi]
    B, H, L = 2, 3, 1100
    scale = 1 / math.sqrt(D)
    q, k, v = (_rand((B, L, H, D), 300 + 10 * mi + s) for s in range(3))
    blocks = _blocks(mask, B, L, L, D) if mi % 2 == 0 else None  # run lists and the inline walk
    nbytes, cut, pieces = _plan(B, H, L, L, D, n_cus)
    assert pieces == 2 and cut == {0: 30, 7: 0, 16: 2, 29: 6}[n_cus]
    o, l = bw.bwa_attn_fwd_balanced(q, k, v, mask, blocks=blocks, scale=scale, n_cus=n_cus,
                                    out_dtype=torch.float32)
    o_ref, l_ref = oracle_attention(q, k, v, mask, scale)
    assert_close(o, l, o_ref, l_ref, torch.bfloat16, f"balanced {mask} n_cus={n_cus}")
    o_pl, l_pl = bw.bwa_attn_fwd(q, k, v, mask, blocks=blocks, scale=scale, out_dtype=torch.float32)
    tail, n_cut = _tail_rows(B, H, L, D, n_cus, pieces)
    assert n_cut == cut
    _check_vs_plain(o, l, o_pl, l_pl, tail, f"balanced vs plain {mask} n_cus={n_cus}")
    # bf16 output: the same merged values, rounded once
    ob, lb = bw.bwa_attn_fwd_balanced(q, k, v, mask, blocks=blocks, scale=scale, n_cus=n_cus)
    assert torch.equal(lb, l)
    assert torch.equal(ob, o.to(torch.bfloat16))


def test_balanced_long_causal_determinism():
    # 32 query blocks of 4..64 tiles, all cut in 4 on the device's units.
    B, H, L, D = 1, 2, 4096, 128
    scale = 1 / math.sqrt(D)
    mask = {"causal": True}
    q, k, v = (_rand((B, L, H, D), 400 + s) for s in range(3))
    blocks = _blocks(mask, B, L, L, D, bkv=128)
    nbytes, cut, pieces = _plan(B, H, L, L, D, 0)
    assert cut == 32 and pieces == 4
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    outs = []
    for fill in (0x00, 0xFF, 0x7F):
        ws.fill_(fill)  # the call clears what it reads
        outs.append(bw.bwa_attn_fwd_balanced(q, k, v, mask, blocks=blocks, scale=scale, workspace=ws,
                                             out_dtype=torch.float32))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
    rows = np.r_[0:3, 250:262, 1020:1030, 2047:2050, 3000:3004, 4090:4096]
    o_ref, l_ref = oracle_attention(q, k, v, mask, scale, rows=rows)
    idx = torch.as_tensor(rows, device=DEV)
    assert_close(outs[0][0].index_select(1, idx), outs[0][1].index_select(2, idx), o_ref, l_ref,
                 torch.bfloat16, "long causal sampled rows")
    o_pl, l_pl = bw.bwa_attn_fwd(q, k, v, mask, blocks=blocks, scale=scale, out_dtype=torch.float32)
    tail, n_cut = _tail_rows(B, H, L, D, 0, pieces)
    assert n_cut == cut == 32 and bool(tail.all())
    _check_vs_plain(outs[0][0], outs[0][1], o_pl, l_pl, tail, "long causal vs plain")


@pytest.mark.parametrize("D", [64, 128])
def test_balanced_modes_and_gate(D):
    # 12 query blocks in XCD shares of 2 or 1, cut in 4 by a 33-tile key
    # range that the causal offset mostly hides (pieces without tiles
    # included): all of them on the device's units, the 4 single-block shares
    # on 16 workgroups (2 per XCD).
    B, H, Lq, Lk = 1, 4, 700, 2100
    scale = 1 / math.sqrt(D)
    q = _rand((B, Lq, H, D), 500)
    k = _rand((B, Lk, H, D), 501)
    v = _rand((B, Lk, H, D), 502)
    k[0, 11, 1] *= 50  # head 1 fails the gate
    mask = {"causal": True, "kv_offset": 150}
    blocks = _blocks(mask, B, Lq, Lk, D)
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, [k], scale, 106.5)
    assert gate[0].tolist() == [1, 0, 1, 1]
    o_ref, l_ref = oracle_attention(q, k, v, mask, scale)
    for n_cus in (0, 16):
        _, cut, pieces = _plan(B, H, Lq, Lk, D, n_cus)
        assert pieces == 4 and cut == {0: 12, 16: 4}[n_cus]
        # fixed-m with the gate: the failing head is left untouched
        o = torch.full((B, Lq, H, D), float("nan"), device=DEV)
        l = torch.full((B, H, Lq), float("nan"), device=DEV)
        bw.bwa_attn_fwd_balanced(q, k, v, mask, blocks=blocks, scale=scale, mode=bw.BWA_MODE_FIXED_M, m=m,
                                 gate=gate, n_cus=n_cus, o=o, lse=l)
        assert torch.isnan(o[:, :, 1]).all() and torch.isnan(l[:, 1]).all()
        hs = [0, 2, 3]
        assert_close(o[:, :, hs], l[:, hs], o_ref[:, :, hs], l_ref[:, hs], torch.bfloat16, "fixed-m gated heads")
        # the online call of the pair fills exactly the failing head
        bw.bwa_attn_fwd_balanced(q, k, v, mask, blocks=blocks, scale=scale, mode=bw.BWA_MODE_ONLINE, gate=gate,
                                 n_cus=n_cus, o=o, lse=l)
        assert_close(o, l, o_ref, l_ref, torch.bfloat16, "gated pair")
        # one gated launch: the pair's bits (the same blocks cut the same way)
        og, lg = bw.bwa_attn_fwd_balanced(q, k, v, mask, blocks=blocks, scale=scale, mode=bw.BWA_MODE_GATED,
                                          m=m, gate=gate, n_cus=n_cus, out_dtype=torch.float32)
        assert torch.equal(og, o) and torch.equal(lg, l)
        pl = bw.bwa_attn_fwd(q, k, v, mask, blocks=blocks, scale=scale, mode=bw.BWA_MODE_GATED, m=m, gate=gate,
                             out_dtype=torch.float32)
        tail, n_cut = _tail_rows(B, H, Lq, D, n_cus, pieces)
        assert n_cut == cut
        _check_vs_plain(og, lg, pl[0], pl[1], tail, f"gated vs plain n_cus={n_cus}")


@pytest.mark.parametrize("n_cus", [0, 16])
def test_balanced_blocks_without_tiles(n_cus):
    # Query blocks with no visible key anywhere (padding) and calls where no
    # block has a tile: rows come out 0 / -inf (24 blocks, 24 or 8 cut in 2).
    B, H, L, D = 2, 2, 1300, 128
    scale = 1 / math.sqrt(D)
    q, k, v = (_rand((B, L, H, D), 600 + s) for s in range(3))
    for mask in ({"q_valid": 200, "causal": True}, {"kv_valid": 0}, {"q_valid": 0}):
        blocks = _blocks(mask, B, L, L, D)
        o = torch.full((B, L, H, D), float("nan"), device=DEV)
        l = torch.full((B, H, L), float("nan"), device=DEV)
        bw.bwa_attn_fwd_balanced(q, k, v, mask, blocks=blocks, scale=scale, n_cus=n_cus, o=o, lse=l)
        o_ref, l_ref = oracle_attention(q, k, v, mask, scale)
        assert_close(o, l, o_ref, l_ref, torch.bfloat16, f"tile-less blocks {mask}")


def test_balanced_workspace_reuse_and_sizes():
    # One workspace, sized for the larger call (12 blocks cut in 3), serves a
    # smaller call next (4 blocks of a 6-tile walk: none cut); a workspace one
    # byte short is refused before any launch.
    D, n_cus = 128, 24
    scale = 1 / math.sqrt(D)
    nbytes, cut, pieces = _plan(2, 3, 1500, 1500, D, n_cus)
    assert (cut, pieces) == (12, 3)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    mask = {"causal": True}
    for (B, H, L) in ((2, 3, 1500), (1, 2, 333)):
        q, k, v = (_rand((B, L, H, D), 700 + L + s) for s in range(3))
        need, cut, pieces = _plan(B, H, L, L, D, n_cus)
        assert 0 < need <= nbytes
        blocks = _blocks(mask, B, L, L, D)
        o, l = bw.bwa_attn_fwd_balanced(q, k, v, mask, blocks=blocks, scale=scale, n_cus=n_cus, workspace=ws,
                                        out_dtype=torch.float32)
        o_pl, l_pl = bw.bwa_attn_fwd(q, k, v, mask, blocks=blocks, scale=scale, out_dtype=torch.float32)
        tail, n_cut = _tail_rows(B, H, L, D, n_cus, pieces)
        assert n_cut == cut
        _check_vs_plain(o, l, o_pl, l_pl, tail, f"reuse {B, H, L}")
    assert cut == 0
    with pytest.raises(bw.BwaError) as e:
        bw.bwa_attn_fwd_balanced(q, k, v, mask, blocks=blocks, scale=scale, n_cus=n_cus, workspace=ws[:need - 1])
    assert e.value.status == 7


@pytest.mark.parametrize("mode", ["online", "fixed", "gated"])
def test_balanced_carry_two_chunks(mode):
    # Two key chunks of one causal sequence; hop 1 through the balanced launch
    # merges the fp32 partial of hop 0 (whole blocks in their epilogue, cut
    # blocks in the piece merge).
    B, H, Lq, L0, L1, D = 2, 3, 1100, 400, 1100, 128
    scale = 1 / math.sqrt(D)
    q = _rand((B, Lq, H, D), 800)
    k = _rand((B, L0 + L1, H, D), 801)
    v = _rand((B, L0 + L1, H, D), 802)
    k[1, 5, 2] *= 30  # head 2 of batch 1 fails the gate
    ks, vs = [k[:, :L0], k[:, L0:]], [v[:, :L0], v[:, L0:]]
    masks = [{"causal": True, "kv_offset": 0, "q_valid": 1050}, {"causal": True, "kv_offset": L0, "q_valid": 1050}]
    kmax, mmax, m, gate = bw.bwa_fixed_m_bound(q, ks, scale, 106.5, q_valid=1050)
    args = {"online": dict(mode=bw.BWA_MODE_ONLINE),
            "fixed": dict(mode=bw.BWA_MODE_FIXED_M, m=m),
            "gated": dict(mode=bw.BWA_MODE_GATED, m=m, gate=gate)}[mode]
    o_ref, l_ref = oracle_attention(q, k, v, {"causal": True, "q_valid": 1050}, scale)
    heads = [0, 1, 2] if mode != "fixed" else [0, 1]  # fixed-m is exact only for heads that pass the gate
    o0, l0 = bw.bwa_attn_fwd(q, ks[0], vs[0], masks[0], scale=scale, out_dtype=torch.float32, **args)
    blocks = _blocks(masks[1], B, Lq, L1, D)
    n_cus = 24  # 30 blocks in XCD shares of 4 or 3 on 3 units each: 6 cut in 2, the rest whole
    nbytes, cut, pieces = _plan(B, H, Lq, L1, D, n_cus)
    assert (cut, pieces) == (6, 2)
    ob, lb = bw.bwa_attn_fwd_balanced(q, ks[1], vs[1], masks[1], blocks=blocks, scale=scale, n_cus=n_cus,
                                      o_prev=o0, lse_prev=l0, out_dtype=torch.float32, **args)
    assert_close(ob[:, :, heads], lb[:, heads], o_ref[:, :, heads], l_ref[:, heads], torch.bfloat16,
                 f"balanced carry {mode}")
    op, lp = bw.bwa_attn_fwd_carry(q, ks[1], vs[1], o0, l0, masks[1], blocks=blocks, scale=scale,
                                   out_dtype=torch.float32, **args)
    tail, n_cut = _tail_rows(B, H, Lq, D, n_cus, pieces)
    assert n_cut == cut
    _check_vs_plain(ob, lb, op, lp, tail, f"balanced carry vs plain carry {mode}")
    # in place: the carried partial is overwritten by the merged result
    oi, li = o0.clone(), l0.clone()
    bw.bwa_attn_fwd_balanced(q, ks[1], vs[1], masks[1], blocks=blocks, scale=scale, n_cus=n_cus,
                             o_prev=oi, lse_prev=li, o=oi, lse=li, **args)
    assert torch.equal(oi, ob) and torch.equal(li, lb)
