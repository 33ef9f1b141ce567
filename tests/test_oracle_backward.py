"""Pins for the oracle's attention gradients (``oracle.attention_backward``).

The gradients are checked against facts other than their own formulas:

* central finite differences of the forward oracle (itself pinned by the
  triple loop and the closed forms in ``test_oracle_pins``): every element of
  dQ, dK and dV on a tiny case, and directional derivatives on every mask
  kind of the forward pins;
* closed forms: one visible key (dQ = dK = 0, dV = the sum of the upstream
  gradients of the rows that see it); identical keys (dQ = 0);
* invariants: the scores of a row move together when every key is shifted
  by one vector, so the dK of a head sums to zero over its keys; each row's
  probabilities sum to one, so dV summed over keys is the sum of dO over the
  rows that see something; keys no row sees and rows that see nothing get
  zero gradient;
* grouped-query heads: a shared key/value head collects the gradients of its
  query heads (finite differences on the shared tensor);
* the sampled forms (selected query rows, selected keys) equal the full
  gradients on those rows and keys.

The value width differs from the query/key width in the directional checks,
so a transposed operand fails.
"""

import numpy as np
import pytest

import oracle
from test_oracle_pins import MASKS


def _loss(q, k, v, do, mask, scale):
    o, _ = oracle.attention(q, k, v, mask, scale)
    return float((o * do).sum())


def _inputs(Lq, Lk, D, Dv, seed):
    r = np.random.Generator(np.random.PCG64(seed))
    return (r.standard_normal((Lq, D)), r.standard_normal((Lk, D)), r.standard_normal((Lk, Dv)),
            r.standard_normal((Lq, Dv)))


@pytest.mark.parametrize("mask", [{}, {"causal": True, "window": 3}, {"q_valid": 5, "kv_valid": 4},
                                  {"causal": True, "kv_offset": -2, "prefix": 2}])
def test_every_element_by_finite_differences(mask):
    Lq, Lk, D, Dv, scale = 6, 5, 3, 4, 0.61
    q, k, v, do = _inputs(Lq, Lk, D, Dv, 7)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, mask, scale)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            fd[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], do, mask, scale)
                       - _loss(args_m["q"], args_m["k"], args_m["v"], do, mask, scale)) / (2 * eps)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("mask", MASKS)
def test_directional_derivatives(mask):
    Lq, Lk, D, Dv, scale = 31, 29, 5, 3, 0.37
    q, k, v, do = _inputs(Lq, Lk, D, Dv, 11)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, mask, scale)
    r = np.random.Generator(np.random.PCG64(12))
    eps = 1e-6
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        base = {"q": q, "k": k, "v": v}
        u = r.standard_normal(base[name].shape)
        p, m = dict(base), dict(base)
        p[name] = base[name] + eps * u
        m[name] = base[name] - eps * u
        fd = (_loss(p["q"], p["k"], p["v"], do, mask, scale) - _loss(m["q"], m["k"], m["v"], do, mask, scale)) / (2 * eps)
        an = float((g * u).sum())
        assert abs(an - fd) <= 1e-6 * max(1.0, abs(fd)), (name, an, fd)


def test_single_visible_key():
    # Lk = 1: P = 1 on every row that sees the key, so O_i = v_0 does not move
    # with q or k and dV_0 is the sum of the upstream gradients of those rows.
    Lq, D, Dv = 9, 4, 6
    q, k, v, do = _inputs(Lq, 1, D, Dv, 5)
    mask = {"q_valid": 7}
    dq, dk, dv = oracle.attention_backward(q, k, v, do, mask, 0.5)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    np.testing.assert_allclose(dv[0], do[:7].sum(axis=0), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("mask", [{}, {"causal": True}, {"causal": True, "window": 4}])
def test_identical_keys_give_zero_dq(mask):
    Lq, Lk, D = 12, 10, 5
    q, _, v, do = _inputs(Lq, Lk, D, D, 6)
    k = np.tile(np.random.Generator(np.random.PCG64(1)).standard_normal((1, D)), (Lk, 1))
    dq, _, _ = oracle.attention_backward(q, k, v, do, mask, 0.8)
    assert np.abs(dq).max() < 1e-12


@pytest.mark.parametrize("mask", MASKS)
def test_shift_and_sum_invariants(mask):
    Lq, Lk, D = 31, 29, 5
    q, k, v, do = _inputs(Lq, Lk, D, D, 13)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, mask, 0.45)
    vis = oracle.visibility(np.arange(Lq), Lk, mask, Lq)
    seen_rows = vis.any(axis=1)
    seen_keys = vis.any(axis=0)
    # rows that see nothing pass no gradient; keys no row sees receive none
    assert np.all(dq[~seen_rows] == 0)
    assert np.all(dk[~seen_keys] == 0) and np.all(dv[~seen_keys] == 0)
    if mask.get("cu_seqlens_q") is None and not mask.get("documents"):
        # one softmax group per row over the same key set: shifting every key by
        # one vector moves a row's scores together
        np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-11)
    else:
        # per segment/document the keys of one group shift together
        ids = _groups(mask, Lk)
        for gid in np.unique(ids):
            np.testing.assert_allclose(dk[ids == gid].sum(axis=0), 0.0, atol=1e-11)
    np.testing.assert_allclose(dv.sum(axis=0), do[seen_rows].sum(axis=0), atol=1e-11)


def _groups(mask, Lk):
    if mask.get("cu_seqlens_kv") is not None or mask.get("cu_seqlens_q") is not None:
        cu = mask.get("cu_seqlens_kv") or mask["cu_seqlens_q"]
        j = np.arange(Lk)
        return np.searchsorted(np.asarray(cu), j, side="right")
    return np.asarray(mask["segment_ids_kv"])[:Lk]


def test_grouped_heads_collect_gradients():
    Lq, Lk, H, Hk, D = 11, 9, 4, 2, 3
    r = np.random.Generator(np.random.PCG64(17))
    q = r.standard_normal((Lq, H, D))
    k = r.standard_normal((Lk, Hk, D))
    v = r.standard_normal((Lk, Hk, D))
    do = r.standard_normal((Lq, H, D))
    mask = {"causal": True, "window": 5}
    scale = 0.7
    dq, dk, dv = oracle.attention_backward_heads(q, k, v, do, mask, scale)

    def loss(k_, v_):
        tot = 0.0
        for h in range(H):
            hk = oracle.kv_head(h, H, Hk)
            tot += _loss(q[:, h], k_[:, hk], v_[:, hk], do[:, h], mask, scale)
        return tot

    eps = 1e-6
    for name, x, g in (("k", k, dk), ("v", v, dv)):
        u = r.standard_normal(x.shape)
        a = (x + eps * u, v) if name == "k" else (k, x + eps * u)
        b = (x - eps * u, v) if name == "k" else (k, x - eps * u)
        fd = (loss(*a) - loss(*b)) / (2 * eps)
        assert abs(float((g * u).sum()) - fd) <= 1e-6 * max(1.0, abs(fd))
    # each query head's dQ is that of its own call
    for h in range(H):
        hk = oracle.kv_head(h, H, Hk)
        a, _, _ = oracle.attention_backward(q[:, h], k[:, hk], v[:, hk], do[:, h], mask, scale)
        np.testing.assert_array_equal(dq[:, h], a)


@pytest.mark.parametrize("mask", MASKS)
def test_sampled_rows_and_keys_equal_full(mask):
    Lq, Lk, D = 31, 29, 5
    q, k, v, do = _inputs(Lq, Lk, D, D, 19)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, mask, 0.52)
    rows = np.array([0, 3, 7, 30, 12])
    keys = np.array([28, 0, 5, 13])
    np.testing.assert_allclose(oracle.attention_backward_rows(q, k, v, do, mask, 0.52, rows), dq[rows],
                               rtol=1e-12, atol=1e-13)
    sk, sv = oracle.attention_backward_keys(q, k, v, do, mask, 0.52, keys, chunk=8)
    np.testing.assert_allclose(sk, dk[keys], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sv, dv[keys], rtol=1e-11, atol=1e-12)
