"""fp64 dense-softmax attention, LSE merge and the fixed-m bound (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Mask description
----------------
A mask is a plain dict with the keys below (missing keys take the default):

``causal`` (False), ``window`` (0), ``kv_offset`` (0), ``q_valid`` (Lq),
``kv_valid`` (Lk), ``cu_seqlens_q`` / ``cu_seqlens_kv`` (None),
``segment_ids_q`` / ``segment_ids_kv`` (None; 1-D, one batch), ``prefix``
(0), ``dilation`` (0), ``documents`` (False).

Query row ``i`` sits at position ``i``; key ``j`` sits at position
``j + kv_offset``; write ``d = i - (j + kv_offset)``.  Key ``j`` is visible
to row ``i`` iff all of:

1. ``j < kv_valid`` and ``i < q_valid`` -- padding sits only at the end of the
   global sequence and the mask is taken from positions, not tiled per shard
   (maxdiffusion pull request 404, review of the ulysses_ring padding mask);
   rows past ``q_valid`` are the alignment rows that are zeroed (sglang pull
   request 47566, Modifications).
2. same segment: ``seg_q(i) == seg_kv(j)``, where ``seg`` comes from
   ``cu_seqlens`` (segment ``s`` covers ``[cu[s], cu[s+1])``; a position
   covered by no segment sees nothing) or from per-token segment ids
   ("Let splash attention exceed 524,288 tokens when packing is off",
   description; sglang pull request 47566, Motivation).
3. ``causal`` => ``d >= 0``, or, with ``prefix = P > 0``, ``d >= 0`` or
   ``j + kv_offset < P`` (prefix-LM: the first ``P`` positions are seen by
   every row).
4. ``window > 0`` => ``d < window`` when causal (the band holds ``window``
   keys counting the query's own position), ``|d| < window`` when not (a
   two-sided band).
5. ``dilation = g >= 2`` (with causal and a window) => ``d mod g == 0``.

The flash-attention page ("Add more optimal dk order optional arg", the
mask tables) names ``sliding_window:512``, ``prefix_lm``,
``dilated_sliding_window`` and ``document`` masks without defining them;
the terms above are the plainest readings.  With ``documents`` the
per-token ids of term 2 may come in any order (a document's tokens need
not be contiguous); without it they are non-decreasing.

Attention output for a row with at least one visible key is the plain softmax
average ``O_i = sum_j p_ij v_j / sum_j p_ij`` with ``p_ij = exp(s_ij - M_i)``,
``s_ij = scale * q_i . k_j`` and ``M_i = max_visible s_ij``; its log-sum-exp
is ``M_i + ln sum_j p_ij`` (natural log).  A row with no visible key has
``O_i = 0`` and ``LSE_i = -inf`` (the alignment rows of sglang pull request
47566 are zeroed; the same reading covers every row that sees nothing).
"""

import numpy as np


def _get(mask, key, default):
    v = mask.get(key, None) if mask else None
    return default if v is None else v


def _segment_index(pos, cu):
    """Segment of each position under cumulative lengths ``cu``; -1 if none."""
    cu = np.asarray(cu, dtype=np.int64)
    seg = np.searchsorted(cu, pos, side="right") - 1
    covered = (pos >= cu[0]) & (pos < cu[-1])
    return np.where(covered, seg, -1)


def visibility(rows, Lk, mask, Lq=None):
    """Boolean matrix ``[len(rows), Lk]``: key ``j`` visible to query row ``i``.

    This is the predicate in the module docstring, evaluated element by
    element with no blocking.
    """
    rows = np.asarray(rows, dtype=np.int64)
    if Lq is None:
        Lq = int(rows.max()) + 1 if rows.size else 0
    i = rows[:, None]
    j = np.arange(Lk, dtype=np.int64)[None, :]
    q_valid = int(_get(mask, "q_valid", Lq))
    kv_valid = int(_get(mask, "kv_valid", Lk))
    off = int(_get(mask, "kv_offset", 0))
    vis = (j < kv_valid) & (i < q_valid)
    cu_q = _get(mask, "cu_seqlens_q", None)
    ids_q = _get(mask, "segment_ids_q", None)
    if cu_q is not None:
        cu_k = _get(mask, "cu_seqlens_kv", cu_q)
        sq = _segment_index(rows, cu_q)[:, None]
        sk = _segment_index(np.arange(Lk, dtype=np.int64), cu_k)[None, :]
        vis &= (sq == sk) & (sq >= 0)
    elif ids_q is not None:
        ids_k = _get(mask, "segment_ids_kv", ids_q)
        sq = np.asarray(ids_q, dtype=np.int64)[rows][:, None]
        sk = np.asarray(ids_k, dtype=np.int64)[:Lk][None, :]
        vis &= sq == sk
    d = i - (j + off)
    causal = bool(_get(mask, "causal", False))
    if causal:
        prefix = int(_get(mask, "prefix", 0))
        vis &= (d >= 0) | ((j + off) < prefix)
    w = int(_get(mask, "window", 0))
    if w > 0:
        vis &= (d < w) if causal else (np.abs(d) < w)
    g = int(_get(mask, "dilation", 0))
    if g >= 2:
        vis &= (d % g) == 0
    return vis


def contiguous(mask):
    """True when every row's visible keys form one interval (all masks but
    dilated bands and document ids)."""
    return int(_get(mask, "dilation", 0)) < 2 and not _get(mask, "documents", False)


def row_intervals_bruteforce(Lq, Lk, mask):
    """Per-row ``[lo, hi)`` of visible keys read off the element predicate.

    Rows that see nothing get ``(0, 0)``.  Returns int64 arrays ``(lo, hi)``.
    """
    lo = np.zeros(Lq, dtype=np.int64)
    hi = np.zeros(Lq, dtype=np.int64)
    for r0 in range(0, Lq, 256):
        rows = np.arange(r0, min(Lq, r0 + 256))
        vis = visibility(rows, Lk, mask, Lq)
        anyv = vis.any(axis=1)
        first = np.argmax(vis, axis=1)
        last = Lk - 1 - np.argmax(vis[:, ::-1], axis=1)
        lo[rows] = np.where(anyv, first, 0)
        hi[rows] = np.where(anyv, last + 1, 0)
        if contiguous(mask):
            assert np.all(vis.sum(axis=1) == np.where(anyv, last + 1 - first, 0))
    return lo, hi


def row_intervals(Lq, Lk, mask):
    """Per-row ``[lo, hi)`` from the mask terms directly (no element matrix).

    An independent second derivation for sequences too long for the element
    predicate: each term of the mask bounds the visible keys of a row from
    below or above.  Segment ids must be non-decreasing (contiguous
    segments), and the mask contiguous (no dilation, no document ids).  Rows
    that see nothing get ``(0, 0)``.
    """
    assert contiguous(mask), "row_intervals needs a contiguous mask"
    i = np.arange(Lq, dtype=np.int64)
    q_valid = int(_get(mask, "q_valid", Lq))
    kv_valid = int(_get(mask, "kv_valid", Lk))
    off = int(_get(mask, "kv_offset", 0))
    lo = np.zeros(Lq, dtype=np.int64)
    hi = np.full(Lq, min(kv_valid, Lk), dtype=np.int64)
    cu_q = _get(mask, "cu_seqlens_q", None)
    ids_q = _get(mask, "segment_ids_q", None)
    if cu_q is not None:
        cu_k = np.asarray(_get(mask, "cu_seqlens_kv", cu_q), dtype=np.int64)
        s = _segment_index(i, cu_q)
        ok = s >= 0
        ss = np.where(ok, s, 0)
        lo = np.maximum(lo, np.where(ok, cu_k[ss], 0))
        hi = np.minimum(hi, np.where(ok, cu_k[ss + 1], 0))
    elif ids_q is not None:
        ids_k = np.asarray(_get(mask, "segment_ids_kv", ids_q), dtype=np.int64)[:Lk]
        assert np.all(np.diff(ids_k) >= 0), "segment ids must be non-decreasing"
        mine = np.asarray(ids_q, dtype=np.int64)[:Lq]
        lo = np.maximum(lo, np.searchsorted(ids_k, mine, side="left"))
        hi = np.minimum(hi, np.searchsorted(ids_k, mine, side="right"))
    causal = bool(_get(mask, "causal", False))
    if causal:
        # the causal part [0, i - off] and the prefix part [0, P - off) are
        # both prefixes of the key axis: their union ends at the larger end
        prefix = int(_get(mask, "prefix", 0))
        hi = np.minimum(hi, np.maximum(i - off + 1, prefix - off))
    w = int(_get(mask, "window", 0))
    if w > 0:
        lo = np.maximum(lo, i - off - w + 1)
        if not causal:
            hi = np.minimum(hi, i - off + w)
    lo = np.maximum(lo, 0)
    empty = (lo >= hi) | (i >= q_valid)
    return np.where(empty, 0, lo), np.where(empty, 0, hi)


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def softmax_probs(q, k, mask, scale, rows=None):
    """Attention probabilities ``P[rows, Lk]`` (rows that see nothing: 0)."""
    q, k = _as64(q), _as64(k)
    Lq, Lk = q.shape[0], k.shape[0]
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    vis = visibility(rows, Lk, mask, Lq)
    s = scale * (q[rows] @ k.T)
    s = np.where(vis, s, -np.inf)
    anyv = vis.any(axis=1)
    m = np.where(anyv, s.max(axis=1, initial=-np.inf), 0.0)
    p = np.where(vis, np.exp(s - m[:, None]), 0.0)
    l = p.sum(axis=1)
    return np.where(anyv[:, None], p / np.where(anyv, l, 1.0)[:, None], 0.0)


def attention(q, k, v, mask, scale, rows=None):
    """Dense softmax attention for one (batch, head) in fp64.

    ``q`` is ``[Lq, D]``, ``k`` and ``v`` are ``[Lk, D]`` (any float type,
    widened exactly to fp64).  Returns ``(O[rows, D], LSE[rows])``.  Online
    softmax, fixed-m and the LSE merge all reach this result in real
    arithmetic ("Fixed-m softmax for 2D-ring x Ulysses attention (WAN 2.2)":
    the output is exact either way; the merge is invariant to the overshoot).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    Lq, Lk = q.shape[0], k.shape[0]
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    vis = visibility(rows, Lk, mask, Lq)
    s = scale * (q[rows] @ k.T)
    s = np.where(vis, s, -np.inf)
    anyv = vis.any(axis=1)
    m_row = s.max(axis=1, initial=-np.inf)
    m_safe = np.where(anyv, m_row, 0.0)
    p = np.where(vis, np.exp(s - m_safe[:, None]), 0.0)
    l = p.sum(axis=1)
    l_safe = np.where(anyv, l, 1.0)
    o = np.where(anyv[:, None], (p @ v) / l_safe[:, None], 0.0)
    lse = np.where(anyv, m_safe + np.log(l_safe), -np.inf)
    return o, lse


def attention_rows(q, k, v, mask, scale, rows, chunk=64):
    """``attention`` on selected rows, ``chunk`` rows at a time (bounded memory)."""
    rows = np.asarray(rows, dtype=np.int64)
    outs, lses = [], []
    for r0 in range(0, rows.size, chunk):
        o, l = attention(q, k, v, mask, scale, rows=rows[r0:r0 + chunk])
        outs.append(o)
        lses.append(l)
    D = np.asarray(v).shape[1]
    if not outs:
        return np.zeros((0, D)), np.zeros(0)
    return np.concatenate(outs), np.concatenate(lses)


def lse_merge(parts):
    """Merge attention partials over disjoint key chunks in LSE space.

    ``parts`` is a list of ``(O_t[..., D], lse_t[...])``.  Returns
    ``(O, lse)`` with ``lse = ln sum_t exp(lse_t)`` and
    ``O = sum_t exp(lse_t - lse) O_t``; when every ``lse_t`` is ``-inf`` the
    row saw nothing and ``O = 0``, ``lse = -inf`` ("Fixed-m softmax for
    2D-ring x Ulysses attention (WAN 2.2)", Notes: a gate failure falls back
    to an LSE-space merge of the hop partials).
    """
    lses = np.stack([_as64(p[1]) for p in parts])
    outs = np.stack([_as64(p[0]) for p in parts])
    mx = lses.max(axis=0)
    anyv = np.isfinite(mx)
    mx_safe = np.where(anyv, mx, 0.0)
    tot = np.exp(lses - mx_safe).sum(axis=0)
    lse = np.where(anyv, mx_safe + np.log(np.where(anyv, tot, 1.0)), -np.inf)
    w = np.where(anyv, np.exp(lses - np.where(anyv, lse, 0.0)), 0.0)
    o = (w[..., None] * outs).sum(axis=0)
    return o, lse


def fixed_m_safe_max():
    """Largest per-row bound whose fixed-m softmax is provably safe in the
    library's arithmetic (reading of "Fixed-m softmax for 2D-ring x Ulysses
    attention (WAN 2.2)", description: heads whose bound cannot be proven safe
    keep online softmax).

    The fixed-m body forms ``p = 2**32 * exp(s - m_i)`` in fp32 and rounds it
    to bf16 for the value product.  With ``|s| <= m_i`` the largest ``p`` of a
    row is at least ``2**(32 - 2 m_i log2 e)``.  Terms under the fp32/bf16
    normal range may be flushed; for a row of up to ``2**30`` keys their weight
    stays under ``2**-12`` of the row's largest term when that term is at least
    ``2**30 * tiny / 2**-12``.  Solving for ``m_i`` gives ``58 ln 2``.
    """
    tiny_exp = int(np.log2(np.finfo(np.float32).tiny))  # -126
    shift, max_keys_exp, weight_exp = 32, 30, -12
    floor_exp = max_keys_exp + tiny_exp - weight_exp     # the largest term's lowest exponent
    return (shift - floor_exp) / (2.0 * np.log2(np.e))


def fixed_m_bound(q, k_chunks, scale, tau, q_valid=None, kv_valid=None,
                  kmax_in=None):
    """Per-query Cauchy-Schwarz bound and per-head gate for one (batch, head).

    From "Fixed-m softmax for 2D-ring x Ulysses attention (WAN 2.2)"
    (description, Notes, Tests):

    * ``kmax = max ||k_j||_2`` over every chunk's valid keys (the bound is
      global over all K shards, so the pinned ``m`` is the same on every hop);
      a caller-supplied per-chunk ``kmax_in`` is folded in with ``max``
      (the per-shard value is promoted to the global bound).
    * ``m_i = scale * ||q_i||_2 * kmax`` bounds every score of row ``i``.
    * The head passes the gate iff ``max_{i < q_valid} m_i <= tau`` (a tie
      passes) and ``max m_i <= fixed_m_safe_max()`` (the bound must also be
      one the fixed-m arithmetic can prove safe).  The decision is taken in
      fp32, the precision the bound is produced in: the fp64 maximum is
      rounded to fp32 and compared with ``float32(tau)`` and
      ``float32(fixed_m_safe_max())``.

    Padded keys (``j >= kv_valid`` of their chunk) do not enter ``kmax``.
    Returns ``(kmax, m[Lq], mmax, gate)`` with fp64 values and a bool gate.
    """
    q = _as64(q)
    Lq = q.shape[0]
    q_valid = Lq if q_valid is None else int(q_valid)
    kmax = 0.0
    for c, kc in enumerate(k_chunks):
        kc = _as64(kc)
        n = kc.shape[0] if kv_valid is None else int(kv_valid[c])
        if n > 0:
            kmax = max(kmax, float(np.sqrt((kc[:n] ** 2).sum(axis=1)).max()))
    if kmax_in is not None:
        kmax = max(kmax, float(np.max(_as64(kmax_in))))
    m = scale * np.sqrt((q ** 2).sum(axis=1)) * kmax
    mmax = float(m[:q_valid].max()) if q_valid > 0 else 0.0
    gate = bool(np.float32(mmax) <= np.float32(tau) and np.float32(mmax) <= np.float32(fixed_m_safe_max()))
    return kmax, m, mmax, gate


def kv_head(h, H, H_kv):
    """Key/value head read by query head ``h`` when ``H`` query heads share
    ``H_kv`` key/value heads in contiguous groups (grouped-query attention;
    ``H_kv = 1`` is multi-query, ``H_kv = H`` one head each).  The
    flash-attention page's benchmark rows carry a ``kv_mode`` column (``mha``
    in every row); grouping consecutive query heads is the plainest reading
    of the other modes."""
    assert H_kv >= 1 and H % H_kv == 0
    return h // (H // H_kv)
