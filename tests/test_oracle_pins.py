"""Pins for the fp64 oracle: it is checked against facts other than itself.

Each check is chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign or index, a transposed operand, a mask term with the wrong
direction) fails at least one of them:

* a pure-Python triple loop written here from the definition (every mask kind);
* a hand-computed two-key example (non-square, so a transposed operand fails);
* closed forms (identical keys -> mean of V, window 1 -> own value, causal
  row 0 -> v_0, one key -> v_0);
* invariants stated on the pages (one segment == non-segmented; padded keys
  masked == truncated; alignment rows zero; LSE merge == full attention;
  fixed-m shift invariance and the Cauchy-Schwarz bound).
"""

import math

import numpy as np
import pytest

import oracle

RNG = np.random.Generator(np.random.PCG64(20261203))


def _qkv(Lq, Lk, D, seed=0):
    r = np.random.Generator(np.random.PCG64(seed))
    return r.standard_normal((Lq, D)), r.standard_normal((Lk, D)), r.standard_normal((Lk, D))


# ---------------------------------------------------------------- triple loop
def _seg(pos, cu):
    for s in range(len(cu) - 1):
        if cu[s] <= pos < cu[s + 1]:
            return s
    return None


def _visible_py(i, j, Lq, Lk, m):
    """The visibility rule restated term by term in plain Python."""
    if j >= m.get("kv_valid", Lk) or i >= m.get("q_valid", Lq):
        return False
    if m.get("cu_seqlens_q") is not None:
        a = _seg(i, m["cu_seqlens_q"])
        b = _seg(j, m.get("cu_seqlens_kv") or m["cu_seqlens_q"])
        if a is None or b is None or a != b:
            return False
    if m.get("segment_ids_q") is not None:
        if m["segment_ids_q"][i] != m["segment_ids_kv"][j]:
            return False
    pos_k = j + m.get("kv_offset", 0)
    if m.get("causal") and pos_k > i and not pos_k < m.get("prefix", 0):
        return False
    if m.get("window", 0) > 0:
        if m.get("causal") and i - pos_k >= m["window"]:
            return False
        if not m.get("causal") and abs(i - pos_k) >= m["window"]:
            return False
    if m.get("dilation", 0) >= 2 and (i - pos_k) % m["dilation"] != 0:
        return False
    return True


def _attention_py(q, k, v, m, scale):
    Lq, D = len(q), len(q[0])  # D: width of q and k
    Lk = len(k)
    O, LSE = [], []
    for i in range(Lq):
        scores = []
        for j in range(Lk):
            if _visible_py(i, j, Lq, Lk, m):
                s = 0.0
                for d in range(D):
                    s += q[i][d] * k[j][d]
                scores.append((j, scale * s))
        if not scores:
            O.append([0.0] * len(v[0]))
            LSE.append(-math.inf)
            continue
        mx = max(s for _, s in scores)
        w = [(j, math.exp(s - mx)) for j, s in scores]
        tot = sum(x for _, x in w)
        O.append([sum(x * v[j][d] for j, x in w) / tot for d in range(len(v[0]))])
        LSE.append(mx + math.log(tot))
    return np.array(O), np.array(LSE)


MASKS = [
    {},
    {"causal": True},
    {"causal": True, "window": 5},
    {"causal": True, "window": 1},
    {"causal": True, "kv_offset": -7},
    {"causal": True, "kv_offset": 4, "window": 9},
    {"q_valid": 20, "kv_valid": 17},
    {"cu_seqlens_q": [0, 9, 22, 31], "cu_seqlens_kv": [0, 9, 22, 31]},
    {"cu_seqlens_q": [0, 12, 31], "cu_seqlens_kv": [0, 5, 24], "causal": True},
    {"cu_seqlens_q": [3, 15, 31], "cu_seqlens_kv": [0, 14, 29], "q_valid": 25},
    {"causal": True, "window": 6, "cu_seqlens_q": [0, 10, 31], "cu_seqlens_kv": [0, 10, 31]},
    {"causal": True, "prefix": 6},
    {"causal": True, "prefix": 12, "kv_offset": 3},
    {"causal": True, "prefix": 8, "cu_seqlens_q": [0, 10, 31], "cu_seqlens_kv": [0, 10, 29]},
    {"window": 4},
    {"window": 3, "kv_offset": -5},
    {"causal": True, "window": 9, "dilation": 3},
    {"causal": True, "window": 12, "dilation": 2, "kv_offset": 2},
    {"segment_ids_q": [3, 1, 3, 2, 1, 1, 3, 2, 2, 0, 3, 1, 1, 2, 3, 0, 0, 3, 1, 2, 3, 1, 2, 2, 3, 0, 1, 1, 3, 2, 1],
     "segment_ids_kv": [1, 3, 2, 2, 0, 1, 3, 3, 1, 2, 0, 1, 3, 2, 2, 1, 0, 3, 1, 1, 2, 3, 0, 2, 1, 3, 3, 2, 1],
     "documents": True},
    {"segment_ids_q": [0, 1, 0, 1, 2, 2, 0, 1, 0, 2, 1, 1, 0, 0, 2, 1, 2, 0, 1, 0, 2, 2, 1, 0, 1, 0, 2, 1, 0, 1, 2],
     "segment_ids_kv": [0, 1, 0, 1, 2, 2, 0, 1, 0, 2, 1, 1, 0, 0, 2, 1, 2, 0, 1, 0, 2, 2, 1, 0, 1, 0, 2, 1, 0],
     "documents": True, "causal": True},
]


@pytest.mark.parametrize("mask", MASKS)
def test_triple_loop_agrees(mask):
    Lq, Lk, D = 31, 29, 5
    q, k, v = _qkv(Lq, Lk, D, seed=3)
    v = v[:, :3]  # value width differs from D: a transposed or mixed-up operand fails
    o_ref, lse_ref = _attention_py(q.tolist(), k.tolist(), v.tolist(), mask, 0.37)
    o, lse = oracle.attention(q, k, v, mask, 0.37)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    assert np.array_equal(np.isinf(lse), np.isinf(lse_ref))
    f = np.isfinite(lse_ref)
    np.testing.assert_allclose(lse[f], lse_ref[f], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("chunk", [64, 7, 1])
def test_attention_rows_over_many_chunks(chunk):
    # attention_rows is what every sampled parity check and the CPU baseline
    # run: ~300 unordered rows (repeats, invalid rows, segment edges) must give
    # the rows of the whole call, however they are chunked.
    Lq, Lk, D = 320, 257, 16
    q, k, v = _qkv(Lq, Lk, D, seed=41)
    v = v[:, :11]
    mask = {"cu_seqlens_q": [0, 130, 300, 320], "cu_seqlens_kv": [0, 120, 250, 257], "causal": True,
            "kv_offset": -9, "q_valid": 310}
    rng = np.random.Generator(np.random.PCG64(42))
    rows = np.concatenate([rng.permutation(Lq)[:250], [0, 129, 130, 299, 300, 309, 310, 319, 5, 5]])
    rng.shuffle(rows)
    o_all, lse_all = oracle.attention(q, k, v, mask, 0.3)
    o, lse = oracle.attention_rows(q, k, v, mask, 0.3, rows, chunk=chunk)
    assert o.shape == (rows.size, 11) and lse.shape == (rows.size,)
    np.testing.assert_allclose(o, o_all[rows], rtol=1e-12, atol=1e-13)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_all[rows]))
    f = np.isfinite(lse_all[rows])
    np.testing.assert_allclose(lse[f], lse_all[rows][f], rtol=1e-12, atol=1e-13)
    # and against the triple loop on a slice of the rows
    sub = rows[:70]
    o_py, lse_py = _attention_py(q.tolist(), k.tolist(), v.tolist(), mask, 0.3)
    np.testing.assert_allclose(o[:70], o_py[sub], rtol=1e-12, atol=1e-13)


def test_segment_ids_triple_loop():
    Lq = Lk = 27
    ids = np.array([0] * 5 + [1] * 11 + [2] * 3 + [4] * 8)
    mask = {"segment_ids_q": ids, "segment_ids_kv": ids, "causal": True}
    q, k, v = _qkv(Lq, Lk, 4, seed=5)
    o_ref, lse_ref = _attention_py(q.tolist(), k.tolist(), v.tolist(), mask, 0.5)
    o, lse = oracle.attention(q, k, v, mask, 0.5)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-13)


def test_two_key_worked_example():
    # q = (2, 0, 1), keys along the first two axes; scale 0.5.
    # s = 0.5 * (2, 0) = (1, 0); p = (e, 1) / (e + 1); LSE = ln(e + 1).
    q = np.array([[2.0, 0.0, 1.0]])
    k = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 0.0]])
    v = np.array([[10.0, -1.0], [4.0, 3.0]])
    o, lse = oracle.attention(q, k, v, {}, 0.5)
    e = math.e
    np.testing.assert_allclose(o[0], [(10 * e + 4) / (e + 1), (-e + 3) / (e + 1)], rtol=1e-15)
    np.testing.assert_allclose(lse[0], math.log(e + 1), rtol=1e-15)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("mask", MASKS)
def test_softmax_rows_sum_to_one(mask):
    q, k, _ = _qkv(31, 29, 8, seed=11)
    p = oracle.softmax_probs(q, k, mask, 0.3)
    vis = oracle.visibility(np.arange(31), 29, mask, 31)
    sums = p.sum(axis=1)
    np.testing.assert_allclose(sums[vis.any(axis=1)], 1.0, rtol=0, atol=1e-12)
    assert np.all(sums[~vis.any(axis=1)] == 0)
    assert np.all(p[~vis] == 0)


@pytest.mark.parametrize("mask", MASKS)
def test_identical_keys_give_mean_of_visible_values(mask):
    Lq, Lk, D = 31, 29, 8
    q, _, v = _qkv(Lq, Lk, D, seed=12)
    k = np.tile(RNG.standard_normal(D), (Lk, 1))
    o, _ = oracle.attention(q, k, v, mask, 0.9)
    vis = oracle.visibility(np.arange(Lq), Lk, mask, Lq)
    for i in range(Lq):
        want = v[vis[i]].mean(axis=0) if vis[i].any() else np.zeros(D)
        np.testing.assert_allclose(o[i], want, rtol=0, atol=1e-12)


def test_window_one_returns_own_value():
    q, k, v = _qkv(40, 40, 6, seed=13)
    o, _ = oracle.attention(q, k, v, {"causal": True, "window": 1}, 1.0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-14)


def test_causal_row_zero_and_single_key():
    q, k, v = _qkv(40, 40, 6, seed=14)
    o, lse = oracle.attention(q, k, v, {"causal": True}, 0.2)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0], 0.2 * q[0] @ k[0], rtol=1e-14)
    o1, lse1 = oracle.attention(q, k[:1], v[:1], {}, 0.2)
    np.testing.assert_allclose(o1, np.tile(v[0], (40, 1)), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse1, 0.2 * q @ k[0], rtol=1e-14)


# ---------------------------------------------------------------- invariants
def test_one_segment_equals_non_segmented_exactly():
    # "Let splash attention exceed 524,288 tokens when packing is off": with a
    # single segment the non-segmented kernel produces the same result.
    q, k, v = _qkv(50, 50, 16, seed=15)
    for base in ({}, {"causal": True}, {"causal": True, "window": 7}):
        o0, l0 = oracle.attention(q, k, v, base, 0.25)
        o1, l1 = oracle.attention(q, k, v, dict(base, cu_seqlens_q=[0, 50]), 0.25)
        ids = np.zeros(50, dtype=np.int64)
        o2, l2 = oracle.attention(q, k, v, dict(base, segment_ids_q=ids, segment_ids_kv=ids), 0.25)
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
        assert np.array_equal(o0, o2) and np.array_equal(l0, l2)


def test_padded_keys_masked_equal_truncated():
    q, k, v = _qkv(30, 45, 8, seed=16)
    n = 33
    kg, vg = k.copy(), v.copy()
    kg[n:] = 1e6 * RNG.standard_normal((45 - n, 8))  # garbage past kv_valid
    vg[n:] = -1e6
    for base in ({}, {"causal": True, "kv_offset": -10}):
        o0, l0 = oracle.attention(q, k[:n], v[:n], base, 0.3)
        o1, l1 = oracle.attention(q, kg, vg, dict(base, kv_valid=n), 0.3)
        np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-13)


def test_invalid_and_empty_rows_are_zero():
    # sglang pull request 47566, Modifications: the alignment rows are zeroed.
    q, k, v = _qkv(64, 64, 8, seed=17)
    mask = {"cu_seqlens_q": [0, 42, 64], "cu_seqlens_kv": [0, 42, 64], "q_valid": 42}
    o, lse = oracle.attention(q, k, v, mask, 0.4)
    assert np.all(o[42:] == 0) and np.all(np.isneginf(lse[42:]))
    assert np.all(np.isfinite(lse[:42]))
    # real rows only see real keys: equal to attention on the truncated problem
    o0, l0 = oracle.attention(q[:42], k[:42], v[:42], {}, 0.4)
    np.testing.assert_allclose(o[:42], o0, rtol=0, atol=1e-13)
    # causal with a positive key offset: the first rows see nothing
    o2, l2 = oracle.attention(q, k, v, {"causal": True, "kv_offset": 5}, 0.4)
    assert np.all(o2[:5] == 0) and np.all(np.isneginf(l2[:5]))
    assert np.all(np.isfinite(l2[5:]))


@pytest.mark.parametrize("splits", [[128], [37, 100, 200], [1, 255]])
@pytest.mark.parametrize("mask", [{}, {"causal": True}, {"causal": True, "window": 60},
                                  {"cu_seqlens_q": [0, 90, 256], "cu_seqlens_kv": [0, 90, 256]}])
def test_lse_merge_of_chunks_equals_full(mask, splits):
    L, D = 256, 16
    q, k, v = _qkv(L, L, D, seed=18)
    o_full, l_full = oracle.attention(q, k, v, mask, 0.25)
    edges = [0] + splits + [L]
    parts = []
    for a, b in zip(edges[:-1], edges[1:]):
        m = dict(mask)
        m["kv_offset"] = mask.get("kv_offset", 0) + a
        if "cu_seqlens_kv" in mask:
            # the chunk's keys in local coordinates
            m["cu_seqlens_kv"] = [min(max(c - a, 0), b - a) for c in mask["cu_seqlens_kv"]]
        parts.append(oracle.attention(q, k[a:b], v[a:b], m, 0.25))
    o, l = oracle.lse_merge(parts)
    np.testing.assert_allclose(o, o_full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, l_full, rtol=0, atol=1e-12)


def test_lse_merge_edge_cases():
    D = 4
    o_a = RNG.standard_normal((3, D))
    parts = [(o_a, np.array([-np.inf, 0.5, -np.inf])),
             (np.zeros((3, D)), np.array([-np.inf, -np.inf, -np.inf]))]
    o, l = oracle.lse_merge(parts)
    assert np.all(o[0] == 0) and np.isneginf(l[0]) and np.all(o[2] == 0)
    np.testing.assert_allclose(o[1], o_a[1], rtol=1e-15)
    assert l[1] == 0.5
    # two equal partials: lse grows by ln 2, output unchanged
    o2, l2 = oracle.lse_merge([(o_a, np.ones(3)), (o_a, np.ones(3))])
    np.testing.assert_allclose(o2, o_a, rtol=1e-15)
    np.testing.assert_allclose(l2, 1 + math.log(2), rtol=1e-15)


# ---------------------------------------------------------------- fixed-m
def test_fixed_m_bound_cauchy_schwarz_and_shift_invariance():
    # "Fixed-m softmax for 2D-ring x Ulysses attention (WAN 2.2)": a per-query
    # bound known before streaming replaces the running max; the output is
    # exact either way.
    Lq, Lk, D = 40, 70, 16
    q, k, v = _qkv(Lq, Lk, D, seed=19)
    k[:, :] *= 1.7
    chunks = [k[:30], k[30:]]
    scale = 1 / math.sqrt(D)
    kmax, m, mmax, gate = oracle.fixed_m_bound(q, chunks, scale, 106.5)
    np.testing.assert_allclose(kmax, np.linalg.norm(k, axis=1).max(), rtol=1e-14)
    s = scale * q @ k.T
    assert np.all(s <= m[:, None] * (1 + 1e-12))
    assert np.all(-s <= m[:, None] * (1 + 1e-12))  # two-sided: |s_ij| <= m_i
    # softmax with m_i in place of the row max gives the same output
    p = np.exp(s - m[:, None])
    o_fixed = (p @ v) / p.sum(axis=1)[:, None]
    lse_fixed = m + np.log(p.sum(axis=1))
    o, lse = oracle.attention(q, k, v, {}, scale)
    np.testing.assert_allclose(o_fixed, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_fixed, lse, rtol=0, atol=1e-12)
    assert gate and mmax == pytest.approx(m.max())


def test_fixed_m_gate_sink_padding_and_promotion():
    D = 8
    q, k, _ = _qkv(20, 30, D, seed=20)
    scale = 1 / math.sqrt(D)
    k_sink = k.copy()
    k_sink[7] *= 50.0
    _, _, mmax, gate = oracle.fixed_m_bound(q, [k_sink], scale, 106.5)
    assert not gate and mmax > 106.5
    # the same big key past kv_valid does not enter the bound
    k_pad = k.copy()
    k_pad[25] *= 1e4
    kmax_p, _, _, _ = oracle.fixed_m_bound(q, [k_pad], scale, 106.5, kv_valid=[25])
    np.testing.assert_allclose(kmax_p, np.linalg.norm(k[:25], axis=1).max(), rtol=1e-14)
    # a caller-supplied per-chunk max||k|| is promoted to the global bound
    kmax_g, m_g, _, _ = oracle.fixed_m_bound(q, [k[:10], k[10:]], scale, 106.5,
                                            kmax_in=[100.0, 3.0])
    assert kmax_g == 100.0
    np.testing.assert_allclose(m_g, scale * np.linalg.norm(q, axis=1) * 100.0, rtol=1e-14)
    # rows past q_valid do not enter the gate
    q2 = q.copy()
    q2[-1] *= 1e3
    _, _, mm_all, g_all = oracle.fixed_m_bound(q2, [k], scale, 106.5)
    _, _, mm_v, g_v = oracle.fixed_m_bound(q2, [k], scale, 106.5, q_valid=19)
    assert (not g_all) and g_v and mm_v < mm_all
    # a tie passes
    kmax_t, m_t, mm_t, _ = oracle.fixed_m_bound(q, [k], scale, 106.5)
    assert oracle.fixed_m_bound(q, [k], scale, float(np.float32(mm_t)))[3]


def _bf16_rne(x):
    """fp32 values rounded to bf16 (round to nearest even), returned as fp32."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def _fixed_m_fp32(q, k, v, scale, m, shift):
    """The fixed-m body in fp32 as a GPU computes it: p = 2^(shift) exp(s - m_i)
    by base-2 exponentials whose results under 2^-126 are flushed to zero,
    l summed in fp32, P rounded to bf16 for the value product."""
    f = np.float32
    s = (q.astype(f) @ k.astype(f).T).astype(f)
    e = s * f(scale * math.log2(math.e)) - (m.astype(f) * f(math.log2(math.e)) - f(shift))[:, None]
    p = np.exp2(e.astype(f)).astype(f)
    p[p < np.finfo(f).tiny] = 0.0
    l = p.sum(axis=1, dtype=f)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = (_bf16_rne(p) @ v.astype(f)) / l[:, None]
    return np.nan_to_num(o, nan=0.0)


def test_fixed_m_safe_range_is_what_fp32_supports():
    # Worst rows for a fixed reference: every key points away from the query
    # with the largest norm, so every score sits near -m_i, about 2 m_i below
    # the reference.  Just under the safe maximum the fp32 fixed-m arithmetic
    # stays within the bf16 tolerance of the exact result; at a bound the
    # page's gate (106.5) admits, every term underflows and the row is lost,
    # which is why the gate also requires m_i <= fixed_m_safe_max().
    D, Lk, scale = 16, 4096, 0.25
    rng = np.random.Generator(np.random.PCG64(50))
    qdir = rng.standard_normal(D)
    qdir /= np.linalg.norm(qdir)
    v = rng.standard_normal((Lk, D))
    assert 40.0 < oracle.fixed_m_safe_max() < 40.3
    for m_target, safe in ((0.999 * oracle.fixed_m_safe_max(), True), (103.0, False)):
        a = rng.uniform(0.9, 1.0, Lk)  # key norms; the largest sets kmax
        a[0] = 1.0
        k = -a[:, None] * qdir[None, :]
        qn = m_target / scale  # ||q|| with kmax = 1
        q = qn * qdir[None, :]
        kmax, m, mmax, gate = oracle.fixed_m_bound(q, [k], scale, 106.5)
        assert gate == safe and mmax == pytest.approx(m_target, rel=1e-12)
        s = scale * q @ k.T
        assert s.max() <= -0.89 * m_target  # every key far below the bound
        o_ref, _ = oracle.attention(q, k, v, {}, scale)
        o32 = _fixed_m_fp32(q, k, v, scale, m, shift=32)
        err = np.abs(o32 - o_ref).max()
        assert (err <= 2e-2) == safe, err
    # the gate's boundary: a tie with the safe maximum passes, the next fp32 fails
    edge = float(np.float32(oracle.fixed_m_safe_max()))
    q1 = np.zeros((1, 4))
    k1 = np.zeros((1, 4))
    q1[0, 0], k1[0, 0] = edge, 1.0
    assert oracle.fixed_m_bound(q1, [k1], 1.0, 106.5)[3]
    q1[0, 0] = float(np.nextafter(np.float32(edge), np.float32(100)))
    assert not oracle.fixed_m_bound(q1, [k1], 1.0, 106.5)[3]
    # a caller's tau below the safe maximum still decides
    q1[0, 0] = 30.0
    assert oracle.fixed_m_bound(q1, [k1], 1.0, 106.5)[3] and not oracle.fixed_m_bound(q1, [k1], 1.0, 29.0)[3]


def test_new_masks_reduce_to_known_ones():
    # closed forms of the prefix, two-sided, dilated and document terms
    L, D = 40, 6
    q, k, v = _qkv(L, L, D, seed=31)
    dense = oracle.attention(q, k, v, {}, 0.4)
    causal = oracle.attention(q, k, v, {"causal": True}, 0.4)
    # a prefix covering every key is the dense mask; an empty prefix is causal
    for a, b in ((oracle.attention(q, k, v, {"causal": True, "prefix": L}, 0.4), dense),
                 (oracle.attention(q, k, v, {"causal": True, "prefix": 0}, 0.4), causal),
                 # a two-sided band wider than the sequence is the dense mask
                 (oracle.attention(q, k, v, {"window": L}, 0.4), dense)):
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # the prefix rows: row i < P sees exactly the first P keys (dense on them)
    P = 15
    o_p, l_p = oracle.attention(q, k, v, {"causal": True, "prefix": P}, 0.4)
    o_d, l_d = oracle.attention(q[:P], k[:P], v[:P], {}, 0.4)
    np.testing.assert_allclose(o_p[:P], o_d, rtol=1e-14, atol=1e-15)
    # a band of W <= g keys dilated by g: only d = 0, each row its own value
    o_g, _ = oracle.attention(q, k, v, {"causal": True, "window": 3, "dilation": 3}, 0.4)
    np.testing.assert_allclose(o_g, v, rtol=1e-14, atol=1e-15)
    # dilation g over a band of W: exactly the keys i, i-g, ..., i-g*floor((W-1)/g)
    vis = oracle.visibility(np.arange(L), L, {"causal": True, "window": 10, "dilation": 4}, L)
    for i in range(L):
        assert np.flatnonzero(vis[i]).tolist() == [j for j in (i - 8, i - 4, i) if j >= 0]
    # contiguous non-decreasing ids: the document path equals the segment path
    ids = np.array([0] * 7 + [1] * 13 + [3] * 20)
    for causal_ in (False, True):
        m = {"segment_ids_q": ids, "segment_ids_kv": ids, "causal": causal_}
        a = oracle.attention(q, k, v, m, 0.4)
        b = oracle.attention(q, k, v, dict(m, documents=True), 0.4)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # documents: one permutation of tokens, ids and rows permutes the output
    r = np.random.Generator(np.random.PCG64(32))
    doc = r.integers(0, 4, size=L)
    perm = r.permutation(L)
    o1, l1 = oracle.attention(q, k, v, {"segment_ids_q": doc, "segment_ids_kv": doc, "documents": True}, 0.4)
    o2, l2 = oracle.attention(q[perm], k[perm], v[perm],
                              {"segment_ids_q": doc[perm], "segment_ids_kv": doc[perm], "documents": True}, 0.4)
    np.testing.assert_allclose(o2, o1[perm], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1[perm], rtol=1e-12, atol=1e-13)


def test_kv_head_groups():
    assert [oracle.kv_head(h, 8, 8) for h in range(8)] == list(range(8))
    assert [oracle.kv_head(h, 8, 1) for h in range(8)] == [0] * 8
    assert [oracle.kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [oracle.kv_head(h, 6, 3) for h in range(6)] == [0, 0, 1, 1, 2, 2]
    with pytest.raises(AssertionError):
        oracle.kv_head(0, 6, 4)


# ---------------------------------------------------------------- row intervals
def _random_masks(n, L, seed):
    r = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(n):
        m = {}
        if r.random() < 0.6:
            m["causal"] = True
            u = r.random()
            if u < 0.5:
                m["window"] = int(r.integers(1, L // 2))
            elif u < 0.7:
                m["prefix"] = int(r.integers(1, L))
        elif r.random() < 0.4:
            m["window"] = int(r.integers(1, L // 2))  # two-sided band
        m["kv_offset"] = int(r.integers(-L // 3, L // 3)) if r.random() < 0.4 else 0
        if r.random() < 0.3:
            m["q_valid"] = int(r.integers(0, L + 1))
        if r.random() < 0.3:
            m["kv_valid"] = int(r.integers(0, L + 1))
        u = r.random()
        if u < 0.3:
            cuts = np.sort(r.choice(np.arange(1, L), size=int(r.integers(1, 6)), replace=False))
            cu = [0] + cuts.tolist() + [L]
            m["cu_seqlens_q"] = cu
            m["cu_seqlens_kv"] = cu
        elif u < 0.45:
            ids = np.sort(r.integers(0, 5, size=L))
            m["segment_ids_q"] = ids
            m["segment_ids_kv"] = ids
        out.append(m)
    return out


@pytest.mark.parametrize("mask", _random_masks(40, 300, 21))
def test_row_intervals_two_derivations_agree(mask):
    lo_a, hi_a = oracle.row_intervals_bruteforce(300, 300, mask)
    lo_b, hi_b = oracle.row_intervals(300, 300, mask)
    assert np.array_equal(lo_a, lo_b) and np.array_equal(hi_a, hi_b)
