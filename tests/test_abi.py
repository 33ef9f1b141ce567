"""CPU checks of the C ABI: the library loads, exports every declared entry
point, its struct layouts match the header, and argument errors come back as
status codes before anything touches a GPU (no compute calls here).
"""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bwattn.h")

bw = pytest.importorskip("blockwise_attention_forward_amd")
L = bw._lib


PROBE_HEADER = os.path.join(ROOT, "include", "bwa_probe.h")
PROBE_LIB = os.path.join(ROOT, "blockwise_attention_forward_amd", "libbwa_probe.so")


def _declared(header=HEADER):
    text = open(header).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(bwa_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 9
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    for n in ("bwa_attn_fwd", "bwa_lse_merge", "bwa_fixed_m_bound", "bwa_block_mask_build"):
        assert n in names


def test_every_header_is_covered():
    # each header under include/ belongs to one of the two libraries checked here
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == ["bwa_probe.h", "bwattn.h"]


def test_probe_library_exports_and_rejects_bad_arguments():
    if not os.path.exists(PROBE_LIB):
        pytest.skip("libbwa_probe.so not built")
    lib = ctypes.CDLL(PROBE_LIB)
    names = _declared(PROBE_HEADER)
    assert names == ["bwa_probe_mfma_bf16", "bwa_probe_mfma_lds_bf16", "bwa_probe_mfma_lds_mix", "bwa_probe_stream"]
    h = lib.bwa_probe_mfma_lds_bf16
    h.restype = ctypes.c_int32
    h.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert h(0, 1, ctypes.c_void_p(16), None) == 1 and h(1, 0, ctypes.c_void_p(16), None) == 1
    assert h(1, 1, None, None) == 1
    m = lib.bwa_probe_mfma_lds_mix
    m.restype = ctypes.c_int32
    m.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert m(1, 1, 0, 1, ctypes.c_void_p(16), None) == 1 and m(1, 1, 1, 0, ctypes.c_void_p(16), None) == 1
    assert m(1, 1, 1, 1, None, None) == 1
    assert m(5, 0, 1, 1, ctypes.c_void_p(16), None) == 1  # a mix that is not built
    g = lib.bwa_probe_stream
    g.restype = ctypes.c_int32
    g.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_void_p]
    assert g(None, 16, 1, None, 1, ctypes.c_void_p(16), None) == 1
    assert g(ctypes.c_void_p(16), 0, 1, None, 1, ctypes.c_void_p(16), None) == 1
    assert g(ctypes.c_void_p(16), 16, 0, None, 1, ctypes.c_void_p(16), None) == 1
    assert g(ctypes.c_void_p(16), 16, 1, None, 1, None, None) == 1
    assert g(ctypes.c_void_p(24), 16, 1, ctypes.c_void_p(32), 1, None, None) == 1
    assert all(hasattr(lib, n) for n in names)
    f = lib.bwa_probe_mfma_bf16
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    # argument errors are reported before any launch
    assert f(0, 1, ctypes.c_void_p(16), None, None) == 1
    assert f(1, 0, ctypes.c_void_p(16), None, None) == 1
    assert f(1, 1, None, None, None) == 1


def test_struct_layout_matches_header():
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "bwattn.h"
int main(void) {
  printf("%zu %zu %zu %zu\n", sizeof(bwa_tensor), offsetof(bwa_tensor, B), offsetof(bwa_tensor, sH), sizeof(bwa_mask));
  printf("%zu %zu %zu %zu\n", offsetof(bwa_mask, num_segments), offsetof(bwa_mask, segment_ids_kv), sizeof(bwa_blocks), offsetof(bwa_blocks, row_hi));
  printf("%zu %zu %zu\n", offsetof(bwa_mask, dilation), offsetof(bwa_mask, prefix), offsetof(bwa_mask, documents));
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "t.c"), os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()
    got = list(map(int, out))
    want = [ctypes.sizeof(bw._Tensor), bw._Tensor.B.offset, bw._Tensor.sH.offset, ctypes.sizeof(bw._Mask),
            bw._Mask.num_segments.offset, bw._Mask.segment_ids_kv.offset, ctypes.sizeof(bw._Blocks),
            bw._Blocks.row_hi.offset, bw._Mask.dilation.offset, bw._Mask.prefix.offset,
            bw._Mask.documents.offset]
    assert got == want


def test_version_and_status_strings():
    assert bw.bwa_version() == 3
    for code in range(9):
        assert bw.bwa_status_string(code) != "unknown status"
    assert bw.bwa_status_string(99) == "unknown status"


def _t(ptr=0x10000, dtype=1, B=1, L=256, H=2, D=128, sB=None, sL=None, sH=None):
    sH = D if sH is None else sH
    sL = H * D if sL is None else sL
    sB = L * H * D if sB is None else sB
    return bw._Tensor(ptr, dtype, 0, B, L, H, D, sB, sL, sH)


def _mask(**kw):
    m = bw._Mask(0, 0, 0, -1, -1, 0, 0, None, None, None, None)
    for k, v in kw.items():
        setattr(m, k, v)
    return m


def _attn(q, k, v, o, mask=None, mode=0, m=None, lse=0x20000):
    mask = mask or _mask()
    return L.bwa_attn_fwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(mask), None, 0.1,
                          mode, m, None, ctypes.byref(o), lse, None)


@pytest.mark.parametrize("case,code", [
    (dict(q=dict(D=96), k=dict(D=96), v=dict(D=96), o=dict(D=96)), 6),
    (dict(q=dict(ptr=0x10008)), 3),
    (dict(q=dict(sL=2 * 128 + 4)), 3),
    (dict(q=dict(ptr=0)), 1),
    (dict(k=dict(dtype=0)), 4),
    (dict(k=dict(dtype=7)), 4),
    (dict(o=dict(L=255)), 2),
    (dict(v=dict(L=100)), 2),
    (dict(k=dict(H=3), v=dict(H=3)), 2),       # 3 key heads do not divide 2 query heads
    (dict(k=dict(H=1), v=dict(H=2)), 2),       # k and v heads differ
    (dict(k=dict(sL=0)), 3),                   # keys broadcast along L (an expanded view)
    (dict(v=dict(sL=64)), 3),                  # rows overlap (L stride under D)
    (dict(q=dict(sH=64)), 3),                  # heads overlap
    (dict(o=dict(sH=0)), 3),                   # output heads aliased
    (dict(k=dict(B=2, sB=1024), v=dict(B=2), q=dict(B=2), o=dict(B=2)), 3),  # batch elements overlap
])
def test_attn_fwd_argument_errors(case, code):
    args = {n: _t(**case.get(n, {})) for n in ("q", "k", "v", "o")}
    assert _attn(args["q"], args["k"], args["v"], args["o"]) == code
    assert bw.bwa_last_error() != ""


@pytest.mark.parametrize("mask,code", [
    (dict(causal=2), 5),
    (dict(dilation=2, window=64), 5),         # a dilated band needs causal
    (dict(dilation=2, causal=1), 5),          # ... and a window
    (dict(dilation=-1), 5),
    (dict(prefix=64), 5),                     # a prefix needs causal
    (dict(prefix=64, causal=1, window=32), 5),  # ... and no window
    (dict(prefix=-1, causal=1), 5),
    (dict(documents=1), 5),                   # documents needs segment ids
    (dict(documents=2, segment_ids_q=0x40000), 5),
    (dict(q_valid=300), 5),                   # > Lq
    (dict(kv_valid=300), 5),
    (dict(num_segments=2), 5),                # segments without cu_seqlens
    (dict(cu_seqlens_q=0x30000), 5),          # cu_seqlens without num_segments
    (dict(cu_seqlens_q=0x30000, num_segments=1, segment_ids_q=0x40000), 5),
])
def test_mask_errors(mask, code):
    q = _t()
    assert _attn(q, _t(), _t(), _t(), mask=_mask(**mask)) == code


def test_row_stride_limit():
    # row strides of 2^24 elements or more are refused before anything runs
    # (the tile copies use 32-bit offsets over 64 rows)
    assert _attn(_t(), _t(sL=1 << 24), _t(), _t()) == 3
    assert "row stride" in bw.bwa_last_error()
    assert _attn(_t(), _t(sL=(1 << 24) - 8, sB=(1 << 24) * 256), _t(), _t(), mask=_mask(causal=2)) == 5


def test_non_overlapping_layouts_pass_the_stride_check():
    # head-major [B, H, L, D] views, a padded row pitch and a single row per
    # head with a zero stride are valid layouts: each call gets past the
    # tensor checks and stops at the bad mask (nothing is launched)
    hm = dict(sL=128, sH=256 * 128)
    bad = _mask(causal=2)
    assert _attn(_t(**hm), _t(**hm), _t(**hm), _t(**hm), mask=bad) == 5
    assert _attn(_t(sL=2 * 128 + 64, sB=256 * 320), _t(), _t(), _t(), mask=bad) == 5
    one = dict(L=1, sL=0)
    assert _attn(_t(**one), _t(**one), _t(**one), _t(**one), mask=bad) == 5


def _carry(q, k, v, o, o_prev, lse_prev=0x30000, lse=0x20000):
    return L.bwa_attn_fwd_carry(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(_mask()), None,
                                0.1, 0, None, None, ctypes.byref(o_prev) if o_prev is not None else None,
                                lse_prev, ctypes.byref(o), lse, None)


@pytest.mark.parametrize("o_prev,o,lse_prev,code", [
    (None, {}, 0x30000, 1),                          # o_prev is required
    (dict(dtype=1), {}, 0x30000, 4),                 # carried partial must be fp32
    (dict(dtype=0, L=255), {}, 0x30000, 2),          # not q's shape
    (dict(dtype=0), {}, None, 1),                    # lse_prev missing
    (dict(dtype=0, ptr=0x50000), dict(ptr=0x50000), 0x30000, 3),   # alias with a bf16 output
    (dict(dtype=0, ptr=0x50000, sL=128, sH=256 * 128), dict(ptr=0x50000, dtype=0), 0x30000, 3),  # alias, other strides
])
def test_attn_fwd_carry_argument_errors(o_prev, o, lse_prev, code):
    op = _t(**o_prev) if o_prev is not None else None
    assert _carry(_t(), _t(), _t(), _t(**o), op, lse_prev=lse_prev) == code
    assert bw.bwa_last_error() != ""


def test_gqa_head_checks():
    # 8 query heads on 2 key/value heads pass the shape checks: each call
    # below fails at a later argument check (nothing is launched)
    q, kv = _t(H=8), _t(H=2)
    assert _attn(q, kv, _t(H=2), _t(H=8), mask=_mask(causal=2)) == 5
    assert "causal" in bw.bwa_last_error()
    assert _attn(q, _t(H=3), _t(H=3), _t(H=8)) == 2
    ks = (bw._Tensor * 2)(_t(H=2), _t(H=2, dtype=0))
    assert L.bwa_fixed_m_bound(ctypes.byref(_t(H=8)), ks, 2, None, 0, None, -1, 0.1, 106.5, 0x1000, 0x1000,
                               0x1000, 0x1000, None) == 2
    assert "k_chunks[1]" in bw.bwa_last_error()
    ks3 = (bw._Tensor * 1)(_t(H=3))
    assert L.bwa_fixed_m_bound(ctypes.byref(_t(H=8)), ks3, 1, None, 0, None, -1, 0.1, 106.5, 0x1000, 0x1000,
                               0x1000, 0x1000, None) == 2
    assert "do not divide" in bw.bwa_last_error()


def test_fixed_m_needs_m_and_lse():
    q = _t()
    assert _attn(q, _t(), _t(), _t(), mode=1, m=None) == 1
    assert _attn(q, _t(), _t(), _t(), lse=None) == 1
    assert _attn(q, _t(), _t(), _t(), mode=5) == 2


def test_block_mask_size():
    n, c, b = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    m = _mask(causal=1, window=512)
    st = L.bwa_block_mask_size(ctypes.byref(m), 1, 4096, 4096, 128, 128, ctypes.byref(n), ctypes.byref(c),
                               ctypes.byref(b))
    assert st == 0 and n.value == 32 and c.value == 96 and b.value == 1
    assert L.bwa_block_mask_size(ctypes.byref(m), 1, 4096, 4096, 100, 128, ctypes.byref(n), ctypes.byref(c),
                                 ctypes.byref(b)) == 2
    seg = _mask(cu_seqlens_q=0x30000, num_segments=3)
    assert L.bwa_block_mask_size(ctypes.byref(seg), 1, 33024, 33024, 128, 128, ctypes.byref(n),
                                 ctypes.byref(c), ctypes.byref(b)) == 0
    assert n.value == 258 and c.value == 258 * 130 and b.value == 1
    ids = _mask(segment_ids_q=0x30000)
    assert L.bwa_block_mask_size(ctypes.byref(ids), 4, 512, 512, 128, 128, ctypes.byref(n),
                                 ctypes.byref(c), ctypes.byref(b)) == 0
    assert b.value == 4 and c.value == 4 * 4


def test_block_mask_build_checks_capacity():
    m = _mask(causal=1)
    blk = bw._Blocks(128, 128, 1024, 1024, 1, 8, 23, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    assert L.bwa_block_mask_build(ctypes.byref(m), 1, 1024, 1024, ctypes.byref(blk), None) == 7
    blk.n_qblocks = 9
    assert L.bwa_block_mask_build(ctypes.byref(m), 1, 1024, 1024, ctypes.byref(blk), None) == 2


def test_merge_and_bound_errors():
    parts = (bw._Tensor * 1)(_t(dtype=0))
    lps = (ctypes.c_void_p * 1)(0x20000)
    out = _t()
    assert L.bwa_lse_merge(0, parts, lps, ctypes.byref(out), None, None) == 2
    assert L.bwa_lse_merge(17, parts, lps, ctypes.byref(out), None, None) == 2
    bad = (bw._Tensor * 1)(_t(dtype=1))
    assert L.bwa_lse_merge(1, bad, lps, ctypes.byref(out), None, None) == 4
    q = _t()
    ks = (bw._Tensor * 1)(_t(H=3))
    assert L.bwa_fixed_m_bound(ctypes.byref(q), ks, 1, None, 0, None, -1, 0.1, 106.5, 0x1000, 0x1000,
                               0x1000, 0x1000, None) == 2
    assert L.bwa_fixed_m_bound(ctypes.byref(q), ks, 17, None, 0, None, -1, 0.1, 106.5, 0x1000, 0x1000,
                               0x1000, 0x1000, None) == 2
    ok1 = (bw._Tensor * 1)(_t())
    assert L.bwa_fixed_m_bound(ctypes.byref(q), ok1, 1, None, 2, None, -1, 0.1, 106.5, 0x1000, 0x1000,
                               0x1000, 0x1000, None) == 1


def test_attn_tile():
    assert bw.bwa_attn_tile(1, 128)[1] == 64 and bw.bwa_attn_tile(1, 128)[0] % 128 == 0 and bw.bwa_attn_tile(0, 128) == (128, 64)
    with pytest.raises(bw.BwaError):
        bw.bwa_attn_tile(1, 80)


def test_balanced_workspace_size():
    n, cut, pieces = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    f = L.bwa_attn_fwd_balanced_workspace
    # 8 query blocks of 256 rows, one per XCD share, on 64 workgroups (8 per
    # XCD): each share's block is a partial round, cut in 2 pieces of a
    # 16-tile walk; each piece keeps 256 rows x (D + 1) fp32 after the
    # 256-byte queue counters
    assert f(1, 1, 2, 1000, 1000, 128, 64, ctypes.byref(n), ctypes.byref(cut), ctypes.byref(pieces)) == 0
    assert (cut.value, pieces.value) == (8, 2)
    assert n.value == 256 + 8 * 2 * 256 * 4 + 8 * 2 * 256 * 128 * 4
    # 64 blocks, 8 per share, on 48 workgroups (6 per XCD): 2 per share cut in 4
    assert f(1, 2, 4, 2048, 4096, 64, 48, ctypes.byref(n), ctypes.byref(cut), ctypes.byref(pieces)) == 0
    assert (cut.value, pieces.value) == (16, 4) and n.value == 256 + 16 * 4 * 256 * 4 + 16 * 4 * 256 * 64 * 4
    # whole rounds only (one workgroup per XCD), or keys too short to cut: only the counters
    assert f(1, 1, 2, 1000, 1000, 128, 8, ctypes.byref(n), ctypes.byref(cut), None) == 0
    assert n.value == 256 and cut.value == 0
    assert f(1, 1, 2, 1000, 400, 128, 64, ctypes.byref(n), ctypes.byref(cut), None) == 0
    assert n.value == 256 and cut.value == 0
    assert f(1, 1, 2, 1000, 1000, 128, 7, None, None, None) == 1
    assert f(1, 1, 2, 1000, 1000, 96, 7, ctypes.byref(n), None, None) == 6
    assert f(7, 1, 2, 1000, 1000, 128, 7, ctypes.byref(n), None, None) == 4
    assert f(1, -1, 2, 1000, 1000, 128, 7, ctypes.byref(n), None, None) == 2
    assert f(1, 1, 2, 1000, 1000, 128, (1 << 16) + 1, ctypes.byref(n), None, None) == 6


def _bal_blocks(L=256, bq=256):
    nqb = (L + bq - 1) // bq
    return bw._Blocks(bq, 64, L, L, 1, nqb, 4 * nqb, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)


def _bal(q, k, v, o, blocks, ws=0x100000, ws_bytes=1 << 30, n_cus=4):
    # 2 query blocks on 4 workgroups: the workspace holds the queue counter
    bs = ctypes.byref(blocks) if blocks is not None else None
    return L.bwa_attn_fwd_balanced(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(_mask()), bs,
                                   0.1, 0, None, None, n_cus, ws, ws_bytes, ctypes.byref(o), 0x20000, None)


@pytest.mark.parametrize("kw,code", [
    (dict(ws=None), 1),                         # workspace is required
    (dict(ws=0x100010), 3),                     # 256-byte alignment
    (dict(ws_bytes=100), 7),                    # smaller than the queue counter
    (dict(n_cus=(1 << 16) + 1), 6),
])
def test_balanced_argument_errors(kw, code):
    assert _bal(_t(), _t(), _t(), _t(), _bal_blocks(), **kw) == code
    assert bw.bwa_last_error() != ""


def test_balanced_needs_bf16_inputs():
    f32 = dict(dtype=0)
    assert _bal(_t(**f32), _t(**f32), _t(**f32), _t(**f32), bw._Blocks(128, 64, 256, 256, 1, 2, 8, 0x1000,
                0x1000, 0x1000, 0x1000, 0x1000, 0x1000)) == 6


def test_balanced_carry_needs_o_prev():
    assert L.bwa_attn_fwd_balanced_carry(ctypes.byref(_t()), ctypes.byref(_t()), ctypes.byref(_t()),
                                         ctypes.byref(_mask()), None, 0.1, 0, None, None, None, 0x30000, 4,
                                         0x100000, 1 << 30, ctypes.byref(_t()), 0x20000, None) == 1


# ---------------------------------------------------------------- backward
def test_bwd_workspace_size():
    n, t = ctypes.c_int64(), ctypes.c_int64()
    f = L.bwa_attn_bwd_workspace
    pad = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # delta [B, H, Lq] fp32, row intervals [c, Lq] x 2, query-tile summaries
    # [c, ceil(Lq/64)] x 16 bytes, key-block ranges [c, ceil(Lk/128)] x 2,
    # document-id filters [c, ceil(Lq/64)] and [c, ceil(Lk/64)] x 4 bytes and
    # the tiles' single ids [c, ceil(Lq/64)] and [c, ceil(Lk/64)] x 8 bytes
    m = _mask(causal=1, window=512)
    assert f(ctypes.byref(m), 2, 16, 4096, 8192, ctypes.byref(n), ctypes.byref(t)) == 0
    assert n.value == (pad(2 * 16 * 4096 * 4) + 2 * pad(4096 * 4) + pad(64 * 16) + 2 * pad(64 * 4) + pad(64 * 4)
                       + pad(128 * 4) + pad(64 * 8) + pad(128 * 8))
    assert t.value == 128
    # per-token segment ids: one copy per batch element
    m = _mask(segment_ids_q=0x40000)
    assert f(ctypes.byref(m), 3, 2, 1000, 1000, ctypes.byref(n), None) == 0
    assert n.value == (pad(3 * 2 * 1000 * 4) + 2 * pad(3 * 1000 * 4) + pad(3 * 16 * 16) + 2 * pad(3 * 8 * 4)
                       + pad(3 * 16 * 4) + pad(3 * 16 * 4)
                       + pad(3 * 16 * 8) + pad(3 * 16 * 8))
    assert f(ctypes.byref(m), 3, 2, 1000, 1000, None, None) == 1
    # a dilated band that runs as g strided windows: the larger of the two
    full = lambda B, H, Lq, Lk: (pad(B * H * Lq * 4) + 2 * pad(Lq * 4) + pad(-(-Lq // 64) * 16)  # noqa: E731
                                 + 2 * pad(-(-Lk // 128) * 4) + pad(-(-Lq // 64) * 4) + pad(-(-Lk // 64) * 4)
                                 + pad(-(-Lq // 64) * 8) + pad(-(-Lk // 64) * 8))
    m = _mask(causal=1, window=1024, dilation=4)
    assert f(ctypes.byref(m), 2, 16, 8192, 8192, ctypes.byref(n), None) == 0
    assert n.value == max(full(2, 16, 8192, 8192), pad(16 * 8192 * 4) + full(4, 16, 2048, 2048))
    m = _mask(causal=1, window=1024, dilation=4, kv_offset=2)  # not a multiple of g: the band's own
    assert f(ctypes.byref(m), 2, 16, 8192, 8192, ctypes.byref(n), None) == 0
    assert n.value == full(2, 16, 8192, 8192)
    assert f(ctypes.byref(_mask()), -1, 2, 10, 10, ctypes.byref(n), None) == 2
    assert f(ctypes.byref(_mask(causal=2)), 1, 2, 10, 10, ctypes.byref(n), None) == 5


def _bwd(q=None, k=None, v=None, o=None, lse=0x20000, do=None, order=0, perm=None, ws=0x100000,
         ws_bytes=1 << 30, dq=None, dk=None, dv=None, mask=None):
    t = lambda x, **kw: x if x is not None else _t(**kw)  # noqa: E731
    args = [t(q), t(k), t(v), t(o), t(do), t(dq, dtype=0), t(dk, dtype=0), t(dv, dtype=0)]
    mask = mask or _mask()
    return L.bwa_attn_bwd(*[ctypes.byref(a) for a in args[:4]], lse, ctypes.byref(args[4]), ctypes.byref(mask),
                          0.1, order, perm, ws, ws_bytes, *[ctypes.byref(a) for a in args[5:]], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=_t(dtype=0), k=_t(dtype=0), v=_t(dtype=0)), 6),  # fp32 inputs: bf16 only
    (dict(k=_t(dtype=0)), 4),                    # q, k, v share a dtype
    (dict(do=_t(dtype=0)), 4),                   # dout must be bf16
    (dict(dk=_t(dtype=1)), 4),                   # gradients share a dtype
    (dict(o=_t(L=255)), 2),
    (dict(dq=_t(dtype=0, H=4)), 2),
    (dict(dv=_t(dtype=0, L=100)), 2),
    (dict(k=_t(H=3), v=_t(H=3), dk=_t(dtype=0, H=3), dv=_t(dtype=0, H=3)), 2),
    (dict(order=4), 2),
    (dict(order=3), 1),                          # a custom order needs kv_order
    (dict(lse=None), 1),
    (dict(ws=None), 1),
    (dict(ws=0x100010), 3),
    (dict(ws_bytes=1000), 7),
    (dict(mask=_mask(causal=2)), 5),
    (dict(q=_t(D=96), k=_t(D=96), v=_t(D=96)), 6),
])
def test_bwd_argument_errors(kw, code):
    assert _bwd(**kw) == code
    assert bw.bwa_last_error() != ""


def test_balanced_noalloc_rejects_plans_beyond_the_static_scratch():
    # 37,800 query rows x 20 heads of 256-row blocks on 256 workgroups: 144
    # blocks cut in 4 pieces need ~76 MB of partials, beyond the 64 MiB
    # scratch; refused before anything is enqueued (no device is touched)
    q = _t(L=37800, H=20, sL=20 * 128, sB=37800 * 20 * 128)
    k = _t(L=37800, H=20, sL=20 * 128, sB=37800 * 20 * 128)
    f = L.bwa_attn_fwd_balanced_noalloc
    st = f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), ctypes.byref(_mask()), None, 0.1, 0, None, None, 256,
           ctypes.byref(q), 0x20000, None)
    assert st == 7 and "67108864" in bw.bwa_last_error()
    assert f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), ctypes.byref(_mask()), None, 0.1, 0, None, None,
             (1 << 16) + 1, ctypes.byref(q), 0x20000, None) == 6
