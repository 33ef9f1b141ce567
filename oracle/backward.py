"""fp64 gradients of dense softmax attention (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The flash-attention page "Add more optimal dk order optional arg" (pull
request 2512; description and "Sliding window perf issue") is about the
backward pass of block-sparse attention: a program per key column computes
that column's dK and dV, and the dQ of each query block collects one
contribution per key column that meets it, in an order that the caller may
choose (ascending, descending or any permutation of the columns); a
deterministic order makes dQ repeat bit for bit.  The page does not restate
the gradients themselves.  They are the derivative of the forward definition
(``attention`` in this package), written out with the chain rule:

    P_ij   = softmax_j(s_ij) over the visible keys of row i (0 elsewhere)
    O_i    = sum_j P_ij v_j
    dV_j   = sum_i P_ij dO_i
    dP_ij  = dO_i . v_j
    D_i    = sum_j P_ij dP_ij = dO_i . O_i
    dS_ij  = P_ij (dP_ij - D_i)
    dQ_i   = scale * sum_j dS_ij k_j
    dK_j   = scale * sum_i dS_ij q_i

for the loss ``L = sum_i dO_i . O_i`` (``dO`` is the upstream gradient).
Rows that see no key have ``P = 0``: they pass no gradient and get
``dQ = 0``.  Every sum is a plain fp64 matrix product; the order in which a
GPU adds the key columns into dQ changes its rounding only, so the oracle
has no notion of order.

With grouped-query heads (``kv_head`` in this package), a key/value head's
gradients are the sums over the query heads that read it.
"""

import numpy as np

from .attention import softmax_probs, kv_head, visibility, attention_rows


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def attention_backward(q, k, v, do, mask, scale):
    """``(dQ[Lq, D], dK[Lk, D], dV[Lk, D])`` for one (batch, head) in fp64.

    ``q`` is ``[Lq, D]``; ``k``, ``v`` are ``[Lk, D]``; ``do`` is ``[Lq, D]``;
    ``mask`` and ``scale`` as for ``attention``.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    p = softmax_probs(q, k, mask, scale)
    o = p @ v
    dv = p.T @ do
    dp = do @ v.T
    delta = (do * o).sum(axis=1)
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_backward_heads(q, k, v, do, mask, scale):
    """Gradients of every head of one batch element, grouped-query aware.

    ``q`` and ``do`` are ``[Lq, H, D]``; ``k`` and ``v`` are ``[Lk, H_kv, D]``
    with ``H`` a multiple of ``H_kv``.  Returns ``dQ[Lq, H, D]``,
    ``dK[Lk, H_kv, D]`` and ``dV[Lk, H_kv, D]``: each key/value head sums the
    gradients of the query heads that read it.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    H, Hk = q.shape[1], k.shape[1]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for h in range(H):
        hk = kv_head(h, H, Hk)
        a, b, c = attention_backward(q[:, h], k[:, hk], v[:, hk], do[:, h], mask, scale)
        dq[:, h] = a
        dk[:, hk] += b
        dv[:, hk] += c
    return dq, dk, dv


def attention_backward_rows(q, k, v, do, mask, scale, rows):
    """``dQ[rows]`` of ``attention_backward`` for the selected query rows only.

    Each row's gradient needs only its own probabilities: the same formulas
    restricted to the rows.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    rows = np.asarray(rows, dtype=np.int64)
    p = softmax_probs(q, k, mask, scale, rows=rows)
    o = p @ v
    dp = do[rows] @ v.T
    delta = (do[rows] * o).sum(axis=1)
    ds = p * (dp - delta[:, None])
    return scale * (ds @ k)


def attention_backward_keys(q, k, v, do, mask, scale, keys, chunk=256):
    """``(dK[keys], dV[keys])`` of ``attention_backward`` for selected keys.

    A key's gradients sum over every row that sees it, and each of those
    rows' probabilities needs the row's full log-sum-exp and output: these
    come from ``attention_rows`` over all rows (``chunk`` rows at a time),
    then the formulas run on the selected key columns only.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    keys = np.asarray(keys, dtype=np.int64)
    Lq, Lk = q.shape[0], k.shape[0]
    dk = np.zeros((keys.size, k.shape[1]))
    dv = np.zeros((keys.size, v.shape[1]))
    for r0 in range(0, Lq, chunk):
        rows = np.arange(r0, min(Lq, r0 + chunk))
        o, lse = attention_rows(q, k, v, mask, scale, rows)
        vis = visibility(rows, Lk, mask, Lq)[:, keys]
        s = scale * (q[rows] @ k[keys].T)
        lse_safe = np.where(np.isfinite(lse), lse, 0.0)
        p = np.where(vis, np.exp(np.where(vis, s, 0.0) - lse_safe[:, None]), 0.0)
        dp = do[rows] @ v[keys].T
        delta = (do[rows] * o).sum(axis=1)
        ds = p * (dp - delta[:, None])
        dk += scale * (ds.T @ q[rows])
        dv += p.T @ do[rows]
    return dk, dv
