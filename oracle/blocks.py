"""Tile classification and run lists (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Add more optimal dk order optional arg" (flash-attention pull request 2512),
"Sliding window perf issue": the work of a block-sparse attention kernel is a
list of tiles, each either partial (an element mask is needed), full (every
pair is visible) or not visited at all, and the page walks one kind of list
after the other; "A simplish fix" and the closing comment merge the two into
one ordered list.  The forward analogue built here:

* the query axis is cut into blocks of ``bq`` rows and the key axis into
  blocks of ``bkv`` keys, both clipped to ``[0, Lq) x [0, Lk)`` (positions
  past the end of either axis are not part of any tile);
* a tile is SKIP if no pair in it is visible, FULL if every pair in it is
  visible, PARTIAL otherwise (a tile that holds a row past ``q_valid`` can
  never be FULL, because such a row sees nothing);
* each query block lists its non-SKIP key blocks in ascending order as
  maximal runs ``[begin, end)`` of one kind.

Kind codes: SKIP = 0, FULL = 1, PARTIAL = 2.  Lists are CSR:
``row_ptr[nQb + 1]`` (int64), ``begin``/``end`` (int32), ``kind`` (uint8).
"""

import numpy as np

from .attention import visibility

SKIP, FULL, PARTIAL = 0, 1, 2


def _nblocks(n, b):
    return (n + b - 1) // b


def block_kinds_bruteforce(mask, Lq, Lk, bq, bkv):
    """Kind of every tile, from the element predicate (one query block at a time)."""
    nqb, nkb = _nblocks(Lq, bq), _nblocks(Lk, bkv)
    kinds = np.zeros((nqb, nkb), dtype=np.uint8)
    for qb in range(nqb):
        rows = np.arange(qb * bq, min(Lq, (qb + 1) * bq))
        vis = visibility(rows, Lk, mask, Lq)
        for kb in range(nkb):
            sub = vis[:, kb * bkv:min(Lk, (kb + 1) * bkv)]
            if sub.all():
                kinds[qb, kb] = FULL
            elif sub.any():
                kinds[qb, kb] = PARTIAL
    return kinds


def block_kinds_intervals(lo, hi, Lq, Lk, bq, bkv, qblocks=None):
    """Kind of every tile from per-row visible intervals ``[lo_i, hi_i)``.

    Uses only that each row's visible keys are one contiguous interval (true
    for every mask here but dilated bands and document ids): a tile is visited iff some row interval
    meets its key range, and FULL iff every row interval covers it.
    ``qblocks`` restricts the output to the listed query blocks.
    """
    lo = np.asarray(lo, dtype=np.int64)
    hi = np.asarray(hi, dtype=np.int64)
    nqb, nkb = _nblocks(Lq, bq), _nblocks(Lk, bkv)
    if qblocks is None:
        qblocks = np.arange(nqb)
    j0 = np.arange(nkb, dtype=np.int64) * bkv
    j1 = np.minimum(j0 + bkv, Lk)
    out = np.zeros((len(qblocks), nkb), dtype=np.uint8)
    for n, qb in enumerate(qblocks):
        r = slice(qb * bq, min(Lq, (qb + 1) * bq))
        l, h = lo[r][:, None], hi[r][:, None]
        nonempty = l < h
        meets = nonempty & (l < j1[None, :]) & (h > j0[None, :])
        covers = nonempty & (l <= j0[None, :]) & (h >= j1[None, :])
        out[n] = np.where(covers.all(axis=0), FULL,
                          np.where(meets.any(axis=0), PARTIAL, SKIP))
    return out


def runs_from_kinds(kinds):
    """CSR run lists: maximal same-kind runs of non-SKIP blocks, ascending."""
    row_ptr = [0]
    begin, end, kind = [], [], []
    for row in kinds:
        kb, n = 0, len(row)
        while kb < n:
            k = row[kb]
            if k == SKIP:
                kb += 1
                continue
            e = kb
            while e < n and row[e] == k:
                e += 1
            begin.append(kb)
            end.append(e)
            kind.append(k)
            kb = e
        row_ptr.append(len(begin))
    return (np.asarray(row_ptr, dtype=np.int64), np.asarray(begin, dtype=np.int32),
            np.asarray(end, dtype=np.int32), np.asarray(kind, dtype=np.uint8))


def block_lists(mask, Lq, Lk, bq, bkv):
    """Run lists of one batch element from the element predicate."""
    return runs_from_kinds(block_kinds_bruteforce(mask, Lq, Lk, bq, bkv))


def counted_flops(kinds, Lq, Lk, bq, bkv, D):
    """``4 * D * rows_in_range * cols_in_range`` summed over non-SKIP tiles.

    One (batch, head); 2 FLOP per multiply-add for each of Q K^T and P V.
    """
    nqb, nkb = kinds.shape
    rows = np.minimum((np.arange(nqb) + 1) * bq, Lq) - np.arange(nqb) * bq
    cols = np.minimum((np.arange(nkb) + 1) * bkv, Lk) - np.arange(nkb) * bkv
    area = rows[:, None].astype(np.float64) * cols[None, :]
    return float(4.0 * D * (area * (kinds != SKIP)).sum())
