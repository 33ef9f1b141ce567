"""Python binding of libbwattn.so (blockwise attention forward, MI355X / gfx950).

Argument marshalling only: every computation runs in the library's HIP
kernels; torch supplies device memory and the current stream.  The functions
carry the names of the C entry points declared in ``include/bwattn.h``.  If
the library has not been built this module raises on import: there is no
fallback implementation.

Layouts: q, k, v, o are ``[B, L, H, D]`` tensors with a contiguous last
dimension; lse and m are ``[B, H, L]`` fp32; gate is ``[B, H]`` uint8.
"""

import ctypes
import os

import torch

__all__ = [
    "BWA_F32", "BWA_BF16", "BWA_MODE_ONLINE", "BWA_MODE_FIXED_M", "BWA_MODE_GATED",
    "BWA_TILE_SKIP", "BWA_TILE_FULL", "BWA_TILE_PARTIAL", "BwaError", "Mask", "BlockLists",
    "lib_path", "bwa_version", "bwa_status_string", "bwa_last_error", "bwa_attn_tile",
    "bwa_block_mask_size", "bwa_block_mask_build", "bwa_fixed_m_bound", "bwa_attn_fwd",
    "bwa_attn_fwd_carry", "bwa_attn_fwd_balanced", "bwa_attn_fwd_balanced_workspace", "bwa_lse_merge",
    "bwa_attn_fwd_balanced_carry", "BWA_ORDER_ASC", "BWA_ORDER_DESC", "BWA_ORDER_OUTSIDE_IN",
    "BWA_ORDER_CUSTOM", "bwa_attn_bwd", "bwa_attn_bwd_workspace", "bwa_attn_fwd_balanced_noalloc",
]

BWA_F32, BWA_BF16 = 0, 1
BWA_MODE_ONLINE, BWA_MODE_FIXED_M, BWA_MODE_GATED = 0, 1, 2
BWA_TILE_SKIP, BWA_TILE_FULL, BWA_TILE_PARTIAL = 0, 1, 2
BWA_ORDER_ASC, BWA_ORDER_DESC, BWA_ORDER_OUTSIDE_IN, BWA_ORDER_CUSTOM = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libbwattn.so")


class BwaError(RuntimeError):
    def __init__(self, status, fn, detail):
        super().__init__(f"{fn} failed: {bwa_status_string(status)} ({status}): {detail}")
        self.status = status


class _Tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("B", ctypes.c_int64), ("L", ctypes.c_int64), ("H", ctypes.c_int64), ("D", ctypes.c_int64),
                ("sB", ctypes.c_int64), ("sL", ctypes.c_int64), ("sH", ctypes.c_int64)]


class _Mask(ctypes.Structure):
    _fields_ = [("causal", ctypes.c_int32), ("window", ctypes.c_int32), ("kv_offset", ctypes.c_int64),
                ("q_valid", ctypes.c_int64), ("kv_valid", ctypes.c_int64),
                ("num_segments", ctypes.c_int32), ("dilation", ctypes.c_int32),
                ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_kv", ctypes.c_void_p),
                ("segment_ids_q", ctypes.c_void_p), ("segment_ids_kv", ctypes.c_void_p),
                ("prefix", ctypes.c_int64), ("documents", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class _Blocks(ctypes.Structure):
    _fields_ = [("bq", ctypes.c_int32), ("bkv", ctypes.c_int32), ("lq", ctypes.c_int64),
                ("lk", ctypes.c_int64), ("batch", ctypes.c_int64), ("n_qblocks", ctypes.c_int64),
                ("capacity", ctypes.c_int64), ("row_ptr", ctypes.c_void_p), ("run_begin", ctypes.c_void_p),
                ("run_end", ctypes.c_void_p), ("run_kind", ctypes.c_void_p), ("row_lo", ctypes.c_void_p),
                ("row_hi", ctypes.c_void_p)]


def _load():
    if not os.path.exists(lib_path):
        raise ImportError(f"{lib_path} is missing: build it with "
                          "`python -m blockwise_attention_forward_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(lib_path)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    TP, MP, BP = ctypes.POINTER(_Tensor), ctypes.POINTER(_Mask), ctypes.POINTER(_Blocks)
    I64P, I32P = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)
    sig = {
        "bwa_status_string": (ctypes.c_char_p, [I32]),
        "bwa_last_error": (ctypes.c_char_p, []),
        "bwa_version": (I32, []),
        "bwa_attn_tile": (I32, [I32, I64, I32P, I32P]),
        "bwa_block_mask_size": (I32, [MP, I64, I64, I64, I32, I32, I64P, I64P, I64P]),
        "bwa_block_mask_build": (I32, [MP, I64, I64, I64, BP, P]),
        "bwa_fixed_m_bound": (I32, [TP, TP, I32, P, I32, I64P, I64, F32, F32, P, P, P, P, P]),
        "bwa_attn_fwd": (I32, [TP, TP, TP, MP, BP, F32, I32, P, P, TP, P, P]),
        "bwa_attn_fwd_carry": (I32, [TP, TP, TP, MP, BP, F32, I32, P, P, TP, P, TP, P, P]),
        "bwa_attn_fwd_balanced": (I32, [TP, TP, TP, MP, BP, F32, I32, P, P, I32, P, I64, TP, P, P]),
        "bwa_attn_fwd_balanced_carry": (I32, [TP, TP, TP, MP, BP, F32, I32, P, P, TP, P, I32, P, I64, TP, P, P]),
        "bwa_attn_fwd_balanced_workspace": (I32, [I32, I64, I64, I64, I64, I64, I32, I64P, I64P, I32P]),
        "bwa_attn_fwd_balanced_noalloc": (I32, [TP, TP, TP, MP, BP, F32, I32, P, P, I32, TP, P, P]),
        "bwa_lse_merge": (I32, [I32, TP, ctypes.POINTER(ctypes.c_void_p), TP, P, P]),
        "bwa_attn_bwd": (I32, [TP, TP, TP, TP, P, TP, MP, F32, I32, P, P, I64, TP, TP, TP, P]),
        "bwa_attn_bwd_workspace": (I32, [MP, I64, I64, I64, I64, I64P, I64P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


_lib = _load()


def bwa_status_string(status):
    return _lib.bwa_status_string(int(status)).decode()


def bwa_last_error():
    return _lib.bwa_last_error().decode()


def bwa_version():
    return _lib.bwa_version()


def _check(status, fn):
    if status != 0:
        raise BwaError(status, fn, bwa_last_error())


def _dtype_code(t):
    if t.dtype == torch.float32:
        return BWA_F32
    if t.dtype == torch.bfloat16:
        return BWA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _tensor(t):
    if t.dim() != 4:
        raise ValueError("expected a [B, L, H, D] tensor")
    if t.stride(3) != 1 and t.shape[3] > 1:
        raise ValueError("the last dimension must be contiguous")
    B, L, H, D = t.shape
    return _Tensor(t.data_ptr() if t.numel() else None, _dtype_code(t), 0, B, L, H, D,
                   t.stride(0), t.stride(1), t.stride(2))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def bwa_attn_tile(dtype, D):
    """Tile sizes (bq, bkv) the attention kernel needs for run lists."""
    code = dtype if isinstance(dtype, int) else (BWA_BF16 if dtype == torch.bfloat16 else BWA_F32)
    bq, bkv = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.bwa_attn_tile(code, int(D), ctypes.byref(bq), ctypes.byref(bkv)), "bwa_attn_tile")
    return bq.value, bkv.value


class Mask:
    """Mask description (see ``bwa_mask`` in bwattn.h) with its device arrays.

    Keyword names: causal, window, kv_offset, q_valid, kv_valid,
    cu_seqlens_q, cu_seqlens_kv (host sequences or tensors), segment_ids_q,
    segment_ids_kv ([B, L] or [L] host/device integer arrays), prefix,
    dilation, documents.  The device copies are made once here and kept
    alive by this object.
    """

    def __init__(self, device="cuda", causal=False, window=0, kv_offset=0, q_valid=-1, kv_valid=-1,
                 cu_seqlens_q=None, cu_seqlens_kv=None, segment_ids_q=None, segment_ids_kv=None,
                 prefix=0, dilation=0, documents=False):
        def dev(x):
            if x is None:
                return None
            return torch.as_tensor(x).to(device=device, dtype=torch.int32).contiguous()
        self._keep = [dev(cu_seqlens_q), dev(cu_seqlens_kv), dev(segment_ids_q), dev(segment_ids_kv)]
        cq, ck, iq, ik = self._keep
        nseg = 0 if cq is None else int(cq.numel()) - 1
        self.struct = _Mask(int(bool(causal)), int(window), int(kv_offset),
                            -1 if q_valid is None else int(q_valid),
                            -1 if kv_valid is None else int(kv_valid), nseg, int(dilation or 0),
                            _ptr(cq), _ptr(ck), _ptr(iq), _ptr(ik), int(prefix or 0), int(bool(documents)), 0)

    @classmethod
    def of(cls, mask, device="cuda"):
        if isinstance(mask, Mask):
            return mask
        return cls(device=device, **(mask or {}))


class BlockLists:
    """Device buffers of a tile run list (``bwa_blocks``) and its descriptor."""

    def __init__(self, n_qblocks, capacity, batch, bq, bkv, lq, lk, device):
        i64, i32 = torch.int64, torch.int32
        self.row_ptr = torch.empty(batch * (n_qblocks + 1), dtype=i64, device=device)
        self.run_begin = torch.empty(batch * capacity, dtype=i32, device=device)
        self.run_end = torch.empty(batch * capacity, dtype=i32, device=device)
        self.run_kind = torch.empty(batch * capacity, dtype=torch.uint8, device=device)
        self.row_lo = torch.empty(max(1, batch * lq), dtype=i32, device=device)
        self.row_hi = torch.empty(max(1, batch * lq), dtype=i32, device=device)
        self.struct = _Blocks(bq, bkv, lq, lk, batch, n_qblocks, capacity,
                              _ptr(self.row_ptr), _ptr(self.run_begin), _ptr(self.run_end),
                              _ptr(self.run_kind), _ptr(self.row_lo), _ptr(self.row_hi))

    def host(self, copy=0):
        """(row_ptr, begin, end, kind) of one list copy on the host (synchronises)."""
        s = self.struct
        rp = self.row_ptr.view(s.batch, s.n_qblocks + 1)[copy].cpu().numpy()
        n = int(rp[-1])
        sl = slice(copy * s.capacity, copy * s.capacity + n)
        return (rp, self.run_begin[sl].cpu().numpy(), self.run_end[sl].cpu().numpy(),
                self.run_kind[sl].cpu().numpy())


def bwa_block_mask_size(mask, B, lq, lk, bq, bkv, device="cuda"):
    m = Mask.of(mask, device)
    nqb, cap, lb = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.bwa_block_mask_size(ctypes.byref(m.struct), B, lq, lk, bq, bkv, ctypes.byref(nqb),
                                    ctypes.byref(cap), ctypes.byref(lb)), "bwa_block_mask_size")
    return nqb.value, cap.value, lb.value


def bwa_block_mask_build(mask, B, lq, lk, bq=128, bkv=128, device="cuda", out=None):
    """Tile run lists and row intervals for ``mask``.

    The buffers are allocated here with torch unless ``out`` (a BlockLists of
    the right size from an earlier call) is given to be rebuilt in place.
    """
    m = Mask.of(mask, device)
    nqb, cap, lb = bwa_block_mask_size(m, B, lq, lk, bq, bkv, device)
    bl = out if out is not None else BlockLists(nqb, cap, lb, bq, bkv, lq, lk, device)
    bl.mask = m
    _check(_lib.bwa_block_mask_build(ctypes.byref(m.struct), B, lq, lk, ctypes.byref(bl.struct),
                                     _stream(device)), "bwa_block_mask_build")
    return bl


def bwa_fixed_m_bound(q, k_chunks, scale, tau, kmax_in=None, kv_valid=None, q_valid=-1, out=None):
    """Per-row bound m, per-head key max, max bound and gate.  Returns (kmax, mmax, m, gate).

    kmax_in: optional [S, B, H] fp32 device tensor of other shards' max||k||.
    """
    B, Lq, H, _ = q.shape
    if out is None:
        out = (torch.empty(B, H, dtype=torch.float32, device=q.device),
               torch.empty(B, H, dtype=torch.float32, device=q.device),
               torch.empty(B, H, Lq, dtype=torch.float32, device=q.device),
               torch.empty(B, H, dtype=torch.uint8, device=q.device))
    kmax, mmax, m, gate = out
    n = len(k_chunks)
    arr = (_Tensor * max(1, n))(*[_tensor(k) for k in k_chunks])
    kv = None
    if kv_valid is not None:
        kv = (ctypes.c_int64 * n)(*[int(x) for x in kv_valid])
    qt = _tensor(q)
    n_in = 0 if kmax_in is None else int(kmax_in.numel() // max(1, B * H))
    if kmax_in is not None:
        kmax_in = kmax_in.to(torch.float32).contiguous()
    _check(_lib.bwa_fixed_m_bound(ctypes.byref(qt), arr, n, _ptr(kmax_in), n_in, kv, int(q_valid),
                                  float(scale), float(tau), _ptr(kmax), _ptr(mmax), _ptr(m),
                                  _ptr(gate), _stream(q.device)), "bwa_fixed_m_bound")
    return kmax, mmax, m, gate


def bwa_attn_fwd(q, k, v, mask=None, blocks=None, scale=None, mode=BWA_MODE_ONLINE, m=None, gate=None,
                 o=None, lse=None, out_dtype=None):
    """Blockwise attention forward of one key chunk.  Returns (o, lse)."""
    B, Lq, H, D = q.shape
    if scale is None:
        scale = D ** -0.5
    if o is None:
        o = torch.empty(B, Lq, H, D, dtype=out_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(B, H, Lq, dtype=torch.float32, device=q.device)
    mk = Mask.of(mask, q.device)
    qt, kt, vt, ot = _tensor(q), _tensor(k), _tensor(v), _tensor(o)
    bs = ctypes.byref(blocks.struct) if blocks is not None else None
    _check(_lib.bwa_attn_fwd(ctypes.byref(qt), ctypes.byref(kt), ctypes.byref(vt), ctypes.byref(mk.struct),
                             bs, float(scale), int(mode), _ptr(m), _ptr(gate), ctypes.byref(ot),
                             _ptr(lse), _stream(q.device)), "bwa_attn_fwd")
    return o, lse


def bwa_attn_fwd_carry(q, k, v, o_prev, lse_prev, mask=None, blocks=None, scale=None, mode=BWA_MODE_ONLINE,
                       m=None, gate=None, o=None, lse=None, out_dtype=None):
    """bwa_attn_fwd over k/v merged with the carried fp32 partial (o_prev,
    lse_prev) of earlier key chunks.  o may be o_prev itself (fp32) and lse may
    be lse_prev.  Returns (o, lse)."""
    B, Lq, H, D = q.shape
    if scale is None:
        scale = D ** -0.5
    if o is None:
        o = torch.empty(B, Lq, H, D, dtype=out_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(B, H, Lq, dtype=torch.float32, device=q.device)
    mk = Mask.of(mask, q.device)
    qt, kt, vt, ot, pt = _tensor(q), _tensor(k), _tensor(v), _tensor(o), _tensor(o_prev)
    bs = ctypes.byref(blocks.struct) if blocks is not None else None
    _check(_lib.bwa_attn_fwd_carry(ctypes.byref(qt), ctypes.byref(kt), ctypes.byref(vt), ctypes.byref(mk.struct),
                                   bs, float(scale), int(mode), _ptr(m), _ptr(gate), ctypes.byref(pt),
                                   _ptr(lse_prev), ctypes.byref(ot), _ptr(lse), _stream(q.device)),
           "bwa_attn_fwd_carry")
    return o, lse


def bwa_attn_fwd_balanced_workspace(dtype, B, H, Lq, Lk, D, n_cus=0, plan=False):
    """Workspace bytes of bwa_attn_fwd_balanced (dtype: BWA_BF16 or a torch
    dtype); with plan=True, (bytes, cut_blocks, pieces)."""
    if isinstance(dtype, torch.dtype):
        dtype = BWA_BF16 if dtype == torch.bfloat16 else BWA_F32
    n, cut, pieces = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    _check(_lib.bwa_attn_fwd_balanced_workspace(int(dtype), int(B), int(H), int(Lq), int(Lk), int(D), int(n_cus),
                                                ctypes.byref(n), ctypes.byref(cut), ctypes.byref(pieces)),
           "bwa_attn_fwd_balanced_workspace")
    return (n.value, cut.value, pieces.value) if plan else n.value


def bwa_attn_fwd_balanced(q, k, v, mask=None, blocks=None, scale=None, mode=BWA_MODE_ONLINE, m=None, gate=None,
                          n_cus=0, workspace=None, o=None, lse=None, out_dtype=None, o_prev=None, lse_prev=None):
    """bwa_attn_fwd with one workgroup per compute unit taking whole query
    blocks and then pieces of the last ones from a queue (bf16 inputs).
    workspace: a uint8 device tensor of at least
    bwa_attn_fwd_balanced_workspace bytes (allocated here if None).  With
    o_prev / lse_prev, the carried partial is merged as in
    bwa_attn_fwd_carry (bwa_attn_fwd_balanced_carry).  Returns (o, lse)."""
    B, Lq, H, D = q.shape
    if scale is None:
        scale = D ** -0.5
    if o is None:
        o = torch.empty(B, Lq, H, D, dtype=out_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(B, H, Lq, dtype=torch.float32, device=q.device)
    if workspace is None:
        n = bwa_attn_fwd_balanced_workspace(_dtype_code(q), B, H, Lq, k.shape[1], D, n_cus)
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device) if n > 0 else None
    mk = Mask.of(mask, q.device)
    qt, kt, vt, ot = _tensor(q), _tensor(k), _tensor(v), _tensor(o)
    bs = ctypes.byref(blocks.struct) if blocks is not None else None
    nbytes = workspace.numel() if workspace is not None else 0
    if o_prev is not None:
        pt = _tensor(o_prev)
        _check(_lib.bwa_attn_fwd_balanced_carry(ctypes.byref(qt), ctypes.byref(kt), ctypes.byref(vt),
                                                ctypes.byref(mk.struct), bs, float(scale), int(mode), _ptr(m),
                                                _ptr(gate), ctypes.byref(pt), _ptr(lse_prev), int(n_cus),
                                                _ptr(workspace), nbytes, ctypes.byref(ot), _ptr(lse),
                                                _stream(q.device)), "bwa_attn_fwd_balanced_carry")
        return o, lse
    _check(_lib.bwa_attn_fwd_balanced(ctypes.byref(qt), ctypes.byref(kt), ctypes.byref(vt),
                                      ctypes.byref(mk.struct), bs, float(scale), int(mode), _ptr(m), _ptr(gate),
                                      int(n_cus), _ptr(workspace), nbytes, ctypes.byref(ot),
                                      _ptr(lse), _stream(q.device)), "bwa_attn_fwd_balanced")
    return o, lse


def bwa_attn_fwd_balanced_noalloc(q, k, v, mask=None, blocks=None, scale=None, mode=BWA_MODE_ONLINE, m=None,
                                  gate=None, n_cus=0, o=None, lse=None, out_dtype=None):
    """bwa_attn_fwd_balanced with the library's static device scratch in
    place of a caller workspace (the call allocates nothing; o and lse are
    allocated here with torch only when not given).  Returns (o, lse)."""
    B, Lq, H, D = q.shape
    if scale is None:
        scale = D ** -0.5
    if o is None:
        o = torch.empty(B, Lq, H, D, dtype=out_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(B, H, Lq, dtype=torch.float32, device=q.device)
    mk = Mask.of(mask, q.device)
    qt, kt, vt, ot = _tensor(q), _tensor(k), _tensor(v), _tensor(o)
    bs = ctypes.byref(blocks.struct) if blocks is not None else None
    _check(_lib.bwa_attn_fwd_balanced_noalloc(ctypes.byref(qt), ctypes.byref(kt), ctypes.byref(vt),
                                              ctypes.byref(mk.struct), bs, float(scale), int(mode), _ptr(m),
                                              _ptr(gate), int(n_cus), ctypes.byref(ot), _ptr(lse),
                                              _stream(q.device)), "bwa_attn_fwd_balanced_noalloc")
    return o, lse


def bwa_lse_merge(o_parts, lse_parts, o_out=None, lse_out=None, out_dtype=torch.bfloat16):
    """LSE-space merge of fp32 partials over disjoint key chunks.  Returns (o, lse)."""
    n = len(o_parts)
    B, L, H, D = o_parts[0].shape
    dev = o_parts[0].device
    if o_out is None:
        o_out = torch.empty(B, L, H, D, dtype=out_dtype, device=dev)
    if lse_out is None:
        lse_out = torch.empty(B, H, L, dtype=torch.float32, device=dev)
    parts = (_Tensor * n)(*[_tensor(t) for t in o_parts])
    lps = (ctypes.c_void_p * n)(*[t.data_ptr() for t in lse_parts])
    ot = _tensor(o_out)
    _check(_lib.bwa_lse_merge(n, parts, lps, ctypes.byref(ot), _ptr(lse_out), _stream(dev)),
           "bwa_lse_merge")
    return o_out, lse_out


def bwa_attn_bwd_workspace(mask, B, H, Lq, Lk, device="cuda", tiles=False):
    """Workspace bytes of bwa_attn_bwd; with tiles=True, (bytes, 64-key tiles)."""
    mk = Mask.of(mask, device)
    n, t = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.bwa_attn_bwd_workspace(ctypes.byref(mk.struct), int(B), int(H), int(Lq), int(Lk), ctypes.byref(n),
                                       ctypes.byref(t)), "bwa_attn_bwd_workspace")
    return (n.value, t.value) if tiles else n.value


def bwa_attn_bwd(q, k, v, o, lse, dout, mask=None, scale=None, order=BWA_ORDER_ASC, kv_order=None,
                 workspace=None, dq=None, dk=None, dv=None, grad_dtype=torch.float32):
    """Backward pass of bwa_attn_fwd (bf16 q/k/v/dout; o and lse from the
    forward).  kv_order: a device int32 permutation of the 64-key tiles for
    BWA_ORDER_CUSTOM.  workspace: a uint8 device tensor of at least
    bwa_attn_bwd_workspace bytes (allocated here if None).  Returns
    (dq, dk, dv)."""
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    if scale is None:
        scale = D ** -0.5
    if dq is None:
        dq = torch.empty(q.shape, dtype=grad_dtype, device=q.device)
    if dk is None:
        dk = torch.empty(k.shape, dtype=grad_dtype, device=q.device)
    if dv is None:
        dv = torch.empty(v.shape, dtype=grad_dtype, device=q.device)
    mk = Mask.of(mask, q.device)
    if workspace is None:
        n = bwa_attn_bwd_workspace(mk, B, H, Lq, Lk, q.device)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    ts = [_tensor(t) for t in (q, k, v, o, dout, dq, dk, dv)]
    _check(_lib.bwa_attn_bwd(ctypes.byref(ts[0]), ctypes.byref(ts[1]), ctypes.byref(ts[2]), ctypes.byref(ts[3]),
                             _ptr(lse), ctypes.byref(ts[4]), ctypes.byref(mk.struct), float(scale), int(order),
                             _ptr(kv_order), _ptr(workspace), workspace.numel(), ctypes.byref(ts[5]),
                             ctypes.byref(ts[6]), ctypes.byref(ts[7]), _stream(q.device)), "bwa_attn_bwd")
    return dq, dk, dv
