"""Seeded synthetic inputs for blockwise attention forward.

This module only draws inputs.  It holds none of the attention arithmetic and
imports neither the oracle nor the HIP library, so both sides of a parity
check can take their inputs from here.

Every tensor is drawn i.i.d. N(0, 1) in fp32 from a seeded torch generator on
the requested device and rounded once to the workload dtype (round to nearest
even).  Layout is token-major ``[B, L, H, D]`` (packed varlen sequences
concatenate along ``L``).  The workloads stand in for the pages' models,
prompts and training data, which are not available: the shapes, masks and
value structure follow the pages (see each ``make_*``).
"""

import math

import numpy as np
import torch

__all__ = [
    "WORKLOADS", "normal", "make_tiny", "make_varlen", "make_window", "make_page_mask", "PAGE_MASKS",
    "make_dit_share", "make_long_causal", "long_causal_segments",
    "sample_rows", "rope_3axis",
]

# name -> short description (sizes as used by the tests and the benchmark)
WORKLOADS = {
    "tiny": "B=1 H=2 Lq=Lk=256 D=64 fp32, no mask; also split into 2 KV chunks",
    "varlen": "B=1 H=24 D=128 bf16, 33,024 packed tokens, cu_seqlens [0, 33002, 33024], "
              "22 alignment rows zeroed (q_valid 33002)",
    "window": "B=1 H=16 D=128 bf16, causal band W in {512, 1024, 2048}, "
              "Lq x Lk in {4096x4096, 4096x8192, 8192x8192}, bottom-right aligned",
    "dit_share": "B=1 H=20 D=128 bf16, Lq=37,800 vs 2 KV hops of 37,800 (of 75,600 = 21x45x80 "
                 "latent tokens), 3-axis RoPE on q/k, per-head k scale U[0.5, 2], optional sink head",
    "long_causal": "B=1 H=8 D=128 bf16, Lq=Lk=1,048,576 causal; single segment or packed "
                   "segments of U[4096, 131072] tokens",
    "page_masks": "B=1 H=16 D=128 bf16, Lq x Lk in {4096x4096, 4096x8192, 8192x8192}: prefix_lm "
                  "(prefix: the positions of the first Lq/4 queries), dilated_sliding_window (W 1024, dilation 4), document (64-token "
                  "chunks dealt to 8 documents at random), two-sided band (W 1024)",
}

# The flash-attention block-sparse tables ("Add more optimal dk order optional
# arg") time these masks at these shapes without giving their parameters;
# the parameters here are this package's choice.
PAGE_MASKS = ("prefix_lm", "dilated_sliding_window", "document", "two_sided_window")


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, seed, device="cpu", dtype=torch.bfloat16, chunk_elems=1 << 27):
    """i.i.d. N(0,1) drawn in fp32 (in chunks along dim 0/1) and rounded to ``dtype``."""
    g = _gen(seed, device)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        flat[s:e] = torch.randn(e - s, generator=g, device=device, dtype=torch.float32).to(dtype)
    return out


def make_tiny(device="cpu", seed=1000):
    """B=1, H=2, Lq=Lk=256, D=64, fp32 q/k/v ~ N(0,1), scale 1/sqrt(D), no mask."""
    B, L, H, D = 1, 256, 2, 64
    q = normal((B, L, H, D), seed, device, torch.float32)
    k = normal((B, L, H, D), seed + 1, device, torch.float32)
    v = normal((B, L, H, D), seed + 2, device, torch.float32)
    return dict(q=q, k=k, v=v, mask={}, scale=1.0 / math.sqrt(D),
                chunks=[(0, 128), (128, 256)])


def make_varlen(device="cpu", seed=1001, H=24, D=128, total=33024, real=33002):
    """Packed sequence ``cu_seqlens [0, real, total]``, alignment rows past ``real``.

    The H3 request of sglang pull request 47566 (Motivation): a 1280x704
    request packs 33,002 real tokens, padded to a multiple of 64 per Ulysses
    rank (33,024 = 64 * 516).  The 22 alignment rows form their own segment
    and are zeroed (``q_valid = real``).
    """
    q = normal((1, total, H, D), seed, device)
    k = normal((1, total, H, D), seed + 1, device)
    v = normal((1, total, H, D), seed + 2, device)
    mask = dict(cu_seqlens_q=[0, real, total], cu_seqlens_kv=[0, real, total],
                q_valid=real)
    return dict(q=q, k=k, v=v, mask=mask, scale=1.0 / math.sqrt(D))


def make_window(Lq, Lk, window, device="cpu", seed=1002, H=16, D=128):
    """Causal sliding-window band, bottom-right aligned (``kv_offset = Lq - Lk``).

    Shapes and windows of the flash-attention block-sparse timing tables
    ("Add more optimal dk order optional arg", "The numbers").
    """
    q = normal((1, Lq, H, D), seed, device)
    k = normal((1, Lk, H, D), seed + 1, device)
    v = normal((1, Lk, H, D), seed + 2, device)
    mask = dict(causal=True, window=int(window), kv_offset=int(Lq - Lk))
    return dict(q=q, k=k, v=v, mask=mask, scale=1.0 / math.sqrt(D))


def make_page_mask(kind, Lq, Lk, device="cpu", seed=1006, H=16, D=128):
    """One of the named masks of the flash-attention tables at ``Lq x Lk``.

    Causal masks are bottom-right aligned (``kv_offset = Lq - Lk``).
    ``document`` deals 64-token chunks of both sequences to 8 documents at
    random (a document's tokens are not contiguous); the ids are [1, L].
    """
    q = normal((1, Lq, H, D), seed, device)
    k = normal((1, Lk, H, D), seed + 1, device)
    v = normal((1, Lk, H, D), seed + 2, device)
    off = int(Lq - Lk)
    if kind == "prefix_lm":
        mask = dict(causal=True, kv_offset=off, prefix=Lq // 4)  # positions of the first quarter of the queries
    elif kind == "dilated_sliding_window":
        mask = dict(causal=True, kv_offset=off, window=1024, dilation=4)
    elif kind == "document":
        rng = np.random.Generator(np.random.PCG64(seed + 3))
        ids_q = np.repeat(rng.integers(0, 8, size=(Lq + 63) // 64), 64)[:Lq]
        ids_k = np.repeat(rng.integers(0, 8, size=(Lk + 63) // 64), 64)[:Lk]
        mask = dict(segment_ids_q=ids_q[None].astype(np.int32), segment_ids_kv=ids_k[None].astype(np.int32),
                    documents=True)
    elif kind == "two_sided_window":
        mask = dict(window=1024, kv_offset=off)
    else:
        raise ValueError(kind)
    return dict(q=q, k=k, v=v, mask=mask, scale=1.0 / math.sqrt(D))


def rope_3axis(x, positions, base=10000.0, split=(22, 21, 21)):
    """Rotate adjacent pairs of the last dim by 3-axis (t, h, w) RoPE angles.

    ``x`` is ``[B, L, H, D]`` (fp32), ``positions`` is ``[L, 3]``.  The pairs
    ``(2p, 2p+1)`` are split over the axes as ``split``; pair ``k`` of an
    axis with ``n`` pairs turns by ``pos * base**(-k/n)``.  Rotations keep
    every norm, so the fixed-m bound does not depend on these details.
    """
    D = x.shape[-1]
    assert sum(split) * 2 == D
    ang = []
    for a, n in enumerate(split):
        freq = base ** (-torch.arange(n, dtype=torch.float64, device=x.device) / n)
        ang.append(positions[:, a:a + 1].to(torch.float64) * freq[None, :])
    ang = torch.cat(ang, dim=1).to(torch.float32)  # [L, D/2]
    c, s = torch.cos(ang)[None, :, None, :], torch.sin(ang)[None, :, None, :]
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = torch.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def make_dit_share(device="cpu", seed=1003, H=20, D=128, grid=(21, 45, 80), hops=2,
                   sink=True, kscale=True):
    """One rank's share of 2-ring x 2-Ulysses video-DiT self-attention.

    "Fixed-m softmax for 2D-ring x Ulysses attention (WAN 2.2)", Result: 720p
    81-frame T2V on dp2 x (ring2 x uly2).  The latent grid has
    21 x 45 x 80 = 75,600 tokens; this rank holds H = 20 heads (of 40) and the
    query shard of tokens [0, 37,800) and sees the keys as ``hops`` sequential
    KV chunks of 37,800.  q and k are RoPE-rotated from N(0,1) pre-rotation
    values (3-axis t/h/w positions, t-major flattening); k is then scaled per
    head by ``c_h ~ U[0.5, 2]``.  With ``sink`` one seeded head gets one key
    whose norm is multiplied by 50, so that head fails the fixed-m gate.
    Returns the query, the per-hop K/V chunks (each contiguous), the sink
    location and the per-hop ``kv_offset``.
    """
    T, Hh, W = grid
    N = T * Hh * W
    Lq = N // 2
    Lc = N // hops
    tt = torch.arange(T, device=device).repeat_interleave(Hh * W)
    hh = torch.arange(Hh, device=device).repeat_interleave(W).repeat(T)
    ww = torch.arange(W, device=device).repeat(T * Hh)
    pos = torch.stack([tt, hh, ww], dim=1)
    q = rope_3axis(normal((1, Lq, H, D), seed, device, torch.float32), pos[:Lq])
    rng = np.random.Generator(np.random.PCG64(seed))
    cscale = torch.tensor(rng.uniform(0.5, 2.0, size=H) if kscale else np.ones(H),
                          dtype=torch.float32, device=device)
    sink_head = int(rng.integers(0, H)) if sink else None
    sink_key = int(rng.integers(0, N)) if sink else None
    ks, vs = [], []
    for t in range(hops):
        kt = normal((1, Lc, H, D), seed + 10 + t, device, torch.float32)
        kt = rope_3axis(kt, pos[t * Lc:(t + 1) * Lc]) * cscale[None, None, :, None]
        if sink and t * Lc <= sink_key < (t + 1) * Lc:
            kt[0, sink_key - t * Lc, sink_head, :] *= 50.0
        ks.append(kt.to(torch.bfloat16).contiguous())
        vs.append(normal((1, Lc, H, D), seed + 20 + t, device))
    return dict(q=q.to(torch.bfloat16).contiguous(), k_chunks=ks, v_chunks=vs,
                kv_offsets=[t * Lc for t in range(hops)], scale=1.0 / math.sqrt(D),
                sink_head=sink_head, sink_key=sink_key, tau=106.5, mask={})


def long_causal_segments(total=1 << 20, lo=4096, hi=131072, seed=1004):
    """Cumulative lengths of packed segments with lengths U[lo, hi] (inclusive).

    Draws until the total is reached and truncates the last segment to fit.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    cu = [0]
    while cu[-1] < total:
        cu.append(min(total, cu[-1] + int(rng.integers(lo, hi, endpoint=True))))
    return cu


def make_long_causal(device="cpu", seed=1005, L=1 << 20, H=8, D=128, packed=False):
    """Causal attention over ``L`` tokens; ``packed`` adds seeded segments.

    "Let splash attention exceed 524,288 tokens when packing is off": a
    1,048,576-token context, once as one sequence and once packed.
    """
    q = normal((1, L, H, D), seed, device)
    k = normal((1, L, H, D), seed + 1, device)
    v = normal((1, L, H, D), seed + 2, device)
    mask = dict(causal=True)
    if packed:
        cu = long_causal_segments(L)
        mask.update(cu_seqlens_q=cu, cu_seqlens_kv=cu)
    return dict(q=q, k=k, v=v, mask=mask, scale=1.0 / math.sqrt(D))


def sample_rows(Lq, n=512, seed=7, must=()):
    """Seeded sorted sample of ``n`` query rows that always holds ``must``.

    ``must`` lists rows to include (first and last valid rows, rows at
    segment boundaries, an invalid row ...).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    must = sorted({int(r) for r in must if 0 <= int(r) < Lq})
    rest = max(0, min(n, Lq) - len(must))
    pool = np.setdiff1d(np.arange(Lq), must)
    pick = rng.choice(pool, size=min(rest, pool.size), replace=False) if rest else []
    return np.unique(np.concatenate([np.asarray(must, dtype=np.int64),
                                     np.asarray(pick, dtype=np.int64)]))
