"""Shared test helpers: oracle runs over [B, L, H, D] tensors and tolerance checks.

Tolerances: bf16 inputs with fp32 accumulation -> output max-abs <= 2e-2 and
mean-abs <= 2e-3; fp32 inputs -> max-abs <= 1e-5.  LSE: 1e-3 + 1e-5 |lse|
(bf16 inputs), 1e-5 + 1e-6 |lse| (fp32 inputs): the LSE carries the rounding
of an fp32 score, so above magnitude 1 its error grows with it (a score of
about 660 times a scale of 1/sqrt(128) gives an LSE near 58, whose fp32 ulp is
3.8e-6).  Rows that see nothing must be exactly 0 with LSE -inf.
"""

import numpy as np
import torch

import oracle

TOL = {
    torch.bfloat16: dict(max=2e-2, mean=2e-3, lse=1e-3, lse_rel=1e-5),
    torch.float32: dict(max=1e-5, mean=1e-5, lse=1e-5, lse_rel=1e-6),
}


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def mask_for_batch(mask, b):
    m = dict(mask or {})
    for key in ("segment_ids_q", "segment_ids_kv"):
        if m.get(key) is not None:
            a = np.asarray(m[key])
            m[key] = a[b] if a.ndim == 2 else a
    return m


def oracle_attention(q, k, v, mask, scale, rows=None, heads=None):
    """Oracle O [B, R, H', D] and LSE [B, H', R] for tensors in [B, L, H, D].

    Converts one (batch, head) at a time to fp64, so long sequences fit.
    """
    B, Lq, H, D = q.shape
    Hk = k.shape[2]  # key/value heads (grouped-query attention when fewer than H)
    heads = list(range(H)) if heads is None else list(heads)
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    O = np.zeros((B, len(rows), len(heads), D))
    L = np.zeros((B, len(heads), len(rows)))
    for b in range(B):
        m = mask_for_batch(mask, b)
        for n, h in enumerate(heads):
            hk = oracle.kv_head(h, H, Hk)
            o, l = oracle.attention_rows(np64(q[b, :, h]), np64(k[b, :, hk]), np64(v[b, :, hk]), m, scale, rows)
            O[b, :, n] = o
            L[b, n] = l
    return O, L


def gpu_rows(o, lse, rows, heads=None):
    """Sampled rows of GPU outputs as fp64: O [B, R, H', D], LSE [B, H', R]."""
    idx = torch.as_tensor(np.asarray(rows), device=o.device, dtype=torch.long)
    os_ = o.index_select(1, idx)
    ls = lse.index_select(2, idx)
    if heads is not None:
        hidx = torch.as_tensor(list(heads), device=o.device, dtype=torch.long)
        os_ = os_.index_select(2, hidx)
        ls = ls.index_select(1, hidx)
    return np64(os_), np64(ls)


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, in_dtype, what=""):
    tol = TOL[in_dtype]
    o = o_gpu if isinstance(o_gpu, np.ndarray) else np64(o_gpu)
    lse = lse_gpu if isinstance(lse_gpu, np.ndarray) else np64(lse_gpu)
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    dead = np.isneginf(lse_ref)  # [B, H, R]
    assert np.array_equal(np.isneginf(lse), dead), f"{what}: -inf LSE rows differ"
    dead_o = np.transpose(dead, (0, 2, 1))[..., None] & np.ones_like(o, dtype=bool)
    assert np.all(o[dead_o] == 0), f"{what}: rows that see nothing must be exactly 0"
    err = np.abs(o - o_ref)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    mx, mean = float(err.max(initial=0)), float(err.mean()) if err.size else 0.0
    assert mx <= tol["max"], f"{what}: max abs err {mx:.3e} > {tol['max']}"
    assert mean <= tol["mean"], f"{what}: mean abs err {mean:.3e} > {tol['mean']}"
    live = ~dead
    if live.any():
        err_l = np.abs(lse[live] - lse_ref[live])
        bound = tol["lse"] + tol["lse_rel"] * np.abs(lse_ref[live])
        worst = int(np.argmax(err_l - bound))
        assert np.all(err_l <= bound), (f"{what}: LSE err {err_l[worst]:.3e} > {bound[worst]:.3e} "
                                        f"at |lse| = {abs(lse_ref[live][worst]):.3g}")
    return mx, mean


# ---------------------------------------------------------------- backward
# Gradient tolerance, derived from the arithmetic (the pages fix none).  The
# kernels round P and dS to bf16 (unit roundoff u = 2^-8) as matrix-core
# operands and accumulate in fp32; delta = dO . O is computed from the
# forward output, which in bf16 carries a relative error u per element.  So
# each gradient element is within u * A of the exact value, where A sums the
# magnitudes of the element's terms:
#   dV[j,d]: A = sum_i P_ij |dO_id|
#   dK[j,d]: A = scale * sum_i (|dS_ij| + P_ij e_i) |q_id|
#   dQ[i,d]: A = scale * sum_j (|dS_ij| + P_ij e_i) |k_jd|
# with e_i = sum_d |dO_id O_id| (the delta error bound over u).  fp32 score,
# exponential and accumulation errors are orders below u; the bound used is
# 2u * A + 1e-6 (a factor 2 of margin), plus u |ref| when the gradient is
# stored in bf16.  Elements whose terms are all zero (keys no row sees, rows
# that see nothing) must be exactly zero.
BWD_U = 2.0 ** -8


def bwd_terms(q, k, v, do, mask, scale, rows, keys, Lq, o_rows=None, lse_rows=None):
    """P, dS and e on rows x keys of one (batch, head), from the oracle's
    visibility and forward (O and LSE of the rows, computed here unless
    given).  q, do: [Lq, D]; k, v: [Lk, D] (fp64)."""
    if o_rows is None:
        o_rows, lse_rows = oracle.attention_rows(q, k, v, mask, scale, rows)
    vis = oracle.visibility(rows, k.shape[0], mask, Lq)[:, keys]
    s = scale * (q[rows] @ k[keys].T)
    lse = np.where(np.isfinite(lse_rows), lse_rows, 0.0)
    p = np.where(vis, np.exp(np.where(vis, s, 0.0) - lse[:, None]), 0.0)
    dp = do[rows] @ v[keys].T
    delta = (do[rows] * o_rows).sum(axis=1)
    ds = p * (dp - delta[:, None])
    e = np.abs(do[rows] * o_rows).sum(axis=1)
    return p, ds, e


def bwd_bounds(q, k, v, do, mask, scale, rows, keys, chunk=512):
    """Error scales A (see above) for dQ[rows] ([R, D]) and dK, dV[keys]
    ([K, D]) of one (batch, head); dK/dV sum over every row in chunks."""
    Lq = q.shape[0]
    rows = np.asarray(rows)
    keys = np.asarray(keys)
    allk = np.arange(k.shape[0])
    p, ds, e = bwd_terms(q, k, v, do, mask, scale, rows, allk, Lq)
    a_dq = scale * ((np.abs(ds) + p * e[:, None]) @ np.abs(k))
    a_dk = np.zeros((keys.size, q.shape[1]))
    a_dv = np.zeros((keys.size, v.shape[1]))
    for r0 in range(0, Lq, chunk):
        rr = np.arange(r0, min(Lq, r0 + chunk))
        p, ds, e = bwd_terms(q, k, v, do, mask, scale, rr, keys, Lq)
        a_dk += scale * ((np.abs(ds) + p * e[:, None]).T @ np.abs(q[rr]))
        a_dv += p.T @ np.abs(do[rr])
    return a_dq, a_dk, a_dv


def assert_grad_close(g, ref, a, bf16_out, what):
    g = g if isinstance(g, np.ndarray) else np64(g)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    zero = a == 0
    assert np.all(g[zero] == 0), f"{what}: elements with no visible term must be exactly 0"
    bound = 2 * BWD_U * a + 1e-6 + (BWD_U * np.abs(ref) if bf16_out else 0.0)
    err = np.abs(g - ref)
    worst = np.unravel_index(int(np.argmax(err - bound)), err.shape) if err.size else None
    assert np.all(err <= bound), (f"{what}: err {err[worst]:.3e} > bound {bound[worst]:.3e} "
                                  f"(ref {ref[worst]:.3e}, A {a[worst]:.3e}) at {worst}")
    return float(err.max(initial=0)), float(err.mean()) if err.size else 0.0
