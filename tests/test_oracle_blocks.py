"""Pins for the oracle's tile classification and run lists.

* closed-form tile counts for causal and causal-window bands;
* the worked example of "Add more optimal dk order optional arg"
  ("Sliding window perf issue"), stored under tests/golden/;
* the element-predicate classification against the independent per-row
  interval classification, on random masks and on downscaled packed
  sequences (segments of 64..1024 tokens in 8192);
* run-list format: ascending, maximal, one kind per run.
"""

import os

import numpy as np
import pytest

import oracle
from oracle import FULL, PARTIAL, SKIP

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kinds(mask, L, Lk=None, b=128):
    Lk = L if Lk is None else Lk
    lo, hi = oracle.row_intervals(L, Lk, mask)
    return oracle.block_kinds_intervals(lo, hi, L, Lk, b, b)


@pytest.mark.parametrize("L", [1024, 1000, 4096])
def test_causal_counts(L):
    n = (L + 127) // 128
    k = oracle.block_kinds_bruteforce({"causal": True}, L, L, 128, 128)
    assert (k != SKIP).sum() == n * (n + 1) // 2
    assert (k == PARTIAL).sum() == n
    assert np.array_equal(np.diag(k), np.full(n, PARTIAL))


@pytest.mark.parametrize("W", [512, 1024, 2048])
@pytest.mark.parametrize("L", [4096, 8192])
def test_causal_window_counts(L, W):
    n, w = L // 128, W // 128
    k = _kinds({"causal": True, "window": W}, L)
    assert (k != SKIP).sum() == w * (w + 1) // 2 + (n - w) * (w + 1)
    # steady state: two partial tiles (diagonal and window edge), w-1 full
    for m in range(w, n):
        row = k[m]
        assert (row == PARTIAL).sum() == 2 and (row == FULL).sum() == w - 1


@pytest.mark.parametrize("W,expect", [(512, 160), (1024, 288), (2048, 544)])
def test_bottom_right_window_counts(W, expect):
    # Lq x Lk = 4096 x 8192, queries are the last 4096 positions
    k = _kinds({"causal": True, "window": W, "kv_offset": 4096 - 8192}, 4096, 8192)
    assert (k != SKIP).sum() == expect


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                key, *vals = line.split()
                out[key] = vals
    return out


def test_dk_order_worked_example():
    g = _read_golden("dk_order_sliding_window_512_column4.txt")
    W = int(g["mask"][1])
    Lq, Lk = map(int, g["shape"])
    bq, bkv = map(int, g["tile"])
    n = int(g["column"][0])
    k = oracle.block_kinds_bruteforce({"causal": True, "window": W}, Lq, Lk, bq, bkv)
    col = k[:, n]
    mirror = lambda ms: sorted(2 * n - int(m) for m in ms)  # noqa: E731
    assert sorted(np.nonzero(col == PARTIAL)[0].tolist()) == mirror(g["partial"])
    assert sorted(np.nonzero(col == FULL)[0].tolist()) == mirror(g["full"])


def _random_masks(n, L, seed):
    r = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(n):
        m = {}
        if r.random() < 0.7:
            m["causal"] = True
            if r.random() < 0.6:
                m["window"] = int(r.integers(1, L))
        if r.random() < 0.4:
            m["kv_offset"] = int(r.integers(-L // 2, L // 2))
        if r.random() < 0.3:
            m["q_valid"] = int(r.integers(0, L + 1))
        if r.random() < 0.3:
            m["kv_valid"] = int(r.integers(0, L + 1))
        if r.random() < 0.5:
            cuts = np.sort(r.choice(np.arange(1, L), size=int(r.integers(1, 12)), replace=False))
            cu = [0] + cuts.tolist() + [L]
            m["cu_seqlens_q"] = cu
            m["cu_seqlens_kv"] = cu
        out.append(m)
    return out


@pytest.mark.parametrize("mask", _random_masks(25, 700, 31))
@pytest.mark.parametrize("tile", [(128, 128), (64, 128), (128, 64)])
def test_bruteforce_equals_intervals(mask, tile):
    L = 700
    bq, bkv = tile
    kb = oracle.block_kinds_bruteforce(mask, L, L, bq, bkv)
    lo, hi = oracle.row_intervals(L, L, mask)
    ki = oracle.block_kinds_intervals(lo, hi, L, L, bq, bkv)
    assert np.array_equal(kb, ki)


@pytest.mark.parametrize("causal", [False, True])
def test_downscaled_packed_sequence(causal):
    # packed sequence of 8192 tokens, segments of U[64, 1024] tokens
    r = np.random.Generator(np.random.PCG64(41))
    cu = [0]
    while cu[-1] < 8192:
        cu.append(min(8192, cu[-1] + int(r.integers(64, 1024, endpoint=True))))
    mask = {"cu_seqlens_q": cu, "cu_seqlens_kv": cu, "causal": causal}
    kb = oracle.block_kinds_bruteforce(mask, 8192, 8192, 128, 128)
    lo, hi = oracle.row_intervals(8192, 8192, mask)
    lo2, hi2 = oracle.row_intervals_bruteforce(8192, 8192, mask)
    assert np.array_equal(lo, lo2) and np.array_equal(hi, hi2)
    assert np.array_equal(kb, oracle.block_kinds_intervals(lo, hi, 8192, 8192, 128, 128))


def test_run_lists_format():
    mask = {"causal": True, "window": 300, "cu_seqlens_q": [0, 200, 450, 900],
            "cu_seqlens_kv": [0, 200, 450, 900]}
    kinds = oracle.block_kinds_bruteforce(mask, 900, 900, 64, 64)
    row_ptr, begin, end, kind = oracle.runs_from_kinds(kinds)
    assert row_ptr[0] == 0 and row_ptr[-1] == len(begin) and np.all(np.diff(row_ptr) >= 0)
    for qb in range(kinds.shape[0]):
        runs = list(zip(begin[row_ptr[qb]:row_ptr[qb + 1]], end[row_ptr[qb]:row_ptr[qb + 1]],
                        kind[row_ptr[qb]:row_ptr[qb + 1]]))
        rebuilt = np.zeros(kinds.shape[1], dtype=np.uint8)
        for i, (b, e, k) in enumerate(runs):
            assert b < e and k in (FULL, PARTIAL)
            rebuilt[b:e] = k
            if i:
                pb, pe, pk = runs[i - 1]
                assert pe <= b and (pe < b or pk != k)  # ascending and maximal
        assert np.array_equal(rebuilt, kinds[qb])


def test_workload_counts():
    # packed H3 request: 258 x 258 tiles, the alignment tiles skipped
    L = 33024
    mask = {"cu_seqlens_q": [0, 33002, 33024], "cu_seqlens_kv": [0, 33002, 33024],
            "q_valid": 33002}
    k = _kinds(mask, L)
    assert (k != SKIP).sum() == 66564 and (k == PARTIAL).sum() == 515
    assert np.isclose(oracle.counted_flops(k, L, L, 128, 128, 128) * 24, 1.340e13, rtol=1e-3)
    # one KV hop of the video-DiT share: every tile full, ragged 40-token tail
    k4 = _kinds({}, 37800)
    assert k4.shape == (296, 296) and np.all(k4 == FULL)
    np.testing.assert_allclose(oracle.counted_flops(k4, 37800, 37800, 128, 128, 128) * 20,
                               4 * 128 * 37800.0 ** 2 * 20)


@pytest.mark.parametrize("g,W,Lq,Lk,off,qv,kvv", [
    (2, 7, 24, 24, 0, 24, 24),
    (3, 10, 24, 36, -12, 21, 33),
    (4, 16, 32, 32, 4, 28, 32),
    (5, 3, 40, 20, 20, 40, 15),
    (4, 1, 16, 16, 0, 16, 16),
])
def test_dilated_band_is_strided_windows(g, W, Lq, Lk, off, qv, kvv):
    # The library computes a dilated band whose sizes are multiples of g as g
    # causal windows of ceil(W / g) keys over the residue classes r: rows
    # r + g a, keys r + g c, kv_offset / g.  The band's visibility must equal
    # the union of those windows' (brute force on the oracle's definition).
    band = {"causal": True, "window": W, "dilation": g, "kv_offset": off, "q_valid": qv, "kv_valid": kvv}
    full = oracle.visibility(np.arange(Lq), Lk, band, Lq)
    sub = {"causal": True, "window": -(-W // g), "kv_offset": off // g, "q_valid": qv // g, "kv_valid": kvv // g}
    win = oracle.visibility(np.arange(Lq // g), Lk // g, sub, Lq // g)
    split = np.zeros_like(full)
    for r in range(g):
        split[r::g, r::g] = win
    assert np.array_equal(full, split)
