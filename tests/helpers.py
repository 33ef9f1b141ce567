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
