"""GPU parity of the backward pass (bwa_attn_bwd) against the fp64 oracle.

The gradients follow "Add more optimal dk order optional arg" (flash-attention
pull request 2512, description): dK and dV per key column, dQ per query block
with its key tiles added in a chosen order (ascending, descending,
outside-in, or a caller's permutation), every order deterministic.

Tolerance: the elementwise bound derived in ``helpers`` (2u times the sum of
the magnitudes of each element's terms, u = 2^-8, the bf16 unit roundoff of
the P and dS operands and of a bf16 forward output), exact zeros where no
term is visible.

Inputs: seeded N(0, 1) q, k, v and upstream gradient (bf16); O and LSE come
from the library's own forward pass, as they would in training.  All calls go
through the C ABI.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_grad_close, bwd_bounds, mask_for_batch, np64
from test_gpu_kernels import DILATED_SPLIT, MASKS

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts too
    pytest.skip("needs a GPU", allow_module_level=True)

import blockwise_attention_forward_amd as bw  # noqa: E402

DEV = "cuda"


def _inputs(B, Lq, Lk, H, Hk, D, seed):
    q = synth.normal((B, Lq, H, D), seed, DEV, torch.bfloat16)
    k = synth.normal((B, Lk, Hk, D), seed + 1, DEV, torch.bfloat16)
    v = synth.normal((B, Lk, Hk, D), seed + 2, DEV, torch.bfloat16)
    do = synth.normal((B, Lq, H, D), seed + 3, DEV, torch.bfloat16)
    return q, k, v, do


def _check_full(q, k, v, do, mask, scale, dq, dk, dv, o_bf16, bf16_out, what):
    """Every element of dq, dk, dv against the oracle, per batch element."""
    B, Lq, H, D = q.shape
    Lk, Hk = k.shape[1], k.shape[2]
    stats = []
    for b in range(B):
        m = mask_for_batch(mask, b)
        rq, rk, rv = oracle.attention_backward_heads(np64(q[b]), np64(k[b]), np64(v[b]), np64(do[b]), m, scale)
        a_dk = np.zeros((Lk, Hk, D))
        a_dv = np.zeros((Lk, Hk, D))
        for h in range(H):
            hk = oracle.kv_head(h, H, Hk)
            a_q, a_k, a_v = bwd_bounds(np64(q[b, :, h]), np64(k[b, :, hk]), np64(v[b, :, hk]), np64(do[b, :, h]), m,
                                       scale, np.arange(Lq), np.arange(Lk))
            stats.append(assert_grad_close(dq[b, :, h], rq[:, h], a_q, bf16_out, f"{what} dq b{b} h{h}"))
            a_dk[:, hk] += a_k
            a_dv[:, hk] += a_v
        for hk in range(Hk):
            stats.append(assert_grad_close(dk[b, :, hk], rk[:, hk], a_dk[:, hk], bf16_out, f"{what} dk b{b} h{hk}"))
            stats.append(assert_grad_close(dv[b, :, hk], rv[:, hk], a_dv[:, hk], bf16_out, f"{what} dv b{b} h{hk}"))
    return stats


def _run(q, k, v, do, mask, scale, o_dtype=torch.bfloat16, grad_dtype=torch.float32, **kw):
    if q.shape[1] and k.shape[1]:
        o, lse = bw.bwa_attn_fwd(q, k, v, mask, scale=scale, out_dtype=o_dtype)
    else:  # an empty side: nothing is visible
        o = torch.zeros(q.shape, dtype=o_dtype, device=DEV)
        lse = torch.full((q.shape[0], q.shape[2], q.shape[1]), float("-inf"), device=DEV)
    return bw.bwa_attn_bwd(q, k, v, o, lse, do, mask, scale=scale, grad_dtype=grad_dtype, **kw)


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("D", [64, 128])
def test_masks_against_oracle(mask, D):
    B, L, H, Hk = 2, 333, 2, 2
    q, k, v, do = _inputs(B, L, L, H, Hk, D, 100 + D)
    scale = D ** -0.5
    dq, dk, dv = _run(q, k, v, do, mask, scale)
    torch.cuda.synchronize()
    _check_full(q, k, v, do, mask, scale, dq, dk, dv, True, False, f"D{D} {mask}")


@pytest.mark.parametrize("Hk", [1, 2])
@pytest.mark.parametrize("grad_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("o_dtype", [torch.float32, torch.bfloat16])
def test_grouped_heads_and_dtypes(Hk, grad_dtype, o_dtype):
    B, Lq, Lk, H, D = 1, 200, 260, 4, 128
    q, k, v, do = _inputs(B, Lq, Lk, H, Hk, D, 7)
    mask = {"causal": True, "kv_offset": Lq - Lk, "window": 150}
    dq, dk, dv = _run(q, k, v, do, mask, D ** -0.5, o_dtype=o_dtype, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    _check_full(q, k, v, do, mask, D ** -0.5, dq, dk, dv, o_dtype == torch.bfloat16, grad_dtype == torch.bfloat16,
                f"Hk{Hk}")


def _outside_in(n):
    return [(r >> 1) if r % 2 == 0 else n - 1 - (r >> 1) for r in range(n)]


def test_orders_are_deterministic_and_change_only_dq_rounding():
    B, L, H, D = 1, 700, 2, 128
    q, k, v, do = _inputs(B, L, L, H, H, D, 21)
    mask = {"causal": True, "window": 400}
    scale = D ** -0.5
    o, lse = bw.bwa_attn_fwd(q, k, v, mask, scale=scale, out_dtype=torch.bfloat16)
    n = bw.bwa_attn_bwd_workspace(mask, B, H, L, L, DEV, tiles=True)[1]
    assert n == (L + 63) // 64
    rng = np.random.Generator(np.random.PCG64(5))
    perms = {
        "identity": list(range(n)),
        "reversed": list(range(n))[::-1],
        "outside_in": _outside_in(n),
        "random": rng.permutation(n).tolist(),
    }
    res = {}
    for name, order, perm in [("asc", bw.BWA_ORDER_ASC, None), ("desc", bw.BWA_ORDER_DESC, None),
                              ("outside_in", bw.BWA_ORDER_OUTSIDE_IN, None)] + \
                             [(f"custom_{k_}", bw.BWA_ORDER_CUSTOM, p) for k_, p in perms.items()]:
        kv = torch.tensor(perm, dtype=torch.int32, device=DEV) if perm is not None else None
        first = bw.bwa_attn_bwd(q, k, v, o, lse, do, mask, scale=scale, order=order, kv_order=kv)
        again = bw.bwa_attn_bwd(q, k, v, o, lse, do, mask, scale=scale, order=order, kv_order=kv)
        for x, y in zip(first, again):
            assert torch.equal(x, y), f"{name}: two calls differ"
        res[name] = first
    for name in res:  # dK and dV do not depend on the order
        assert torch.equal(res[name][1], res["asc"][1]) and torch.equal(res[name][2], res["asc"][2]), name
    assert torch.equal(res["custom_identity"][0], res["asc"][0])
    assert torch.equal(res["custom_reversed"][0], res["desc"][0])
    assert torch.equal(res["custom_outside_in"][0], res["outside_in"][0])
    for name, (dq, dk, dv) in res.items():
        _check_full(q, k, v, do, mask, scale, dq, dk, dv, True, False, name)


@pytest.mark.parametrize("Lq,Lk", [(1, 1), (1, 300), (300, 1), (64, 64), (129, 65), (0, 50), (50, 0)])
def test_edge_sizes(Lq, Lk):
    B, H, D = 1, 2, 64
    q, k, v, do = _inputs(B, Lq, Lk, H, H, D, 9)
    for mask in ({}, {"causal": True, "kv_offset": Lq - Lk}):
        dq, dk, dv = _run(q, k, v, do, mask, D ** -0.5)
        torch.cuda.synchronize()
        if Lq and Lk:
            _check_full(q, k, v, do, mask, D ** -0.5, dq, dk, dv, True, False, f"{Lq}x{Lk} {mask}")
        else:
            assert torch.count_nonzero(dq) == 0 and torch.count_nonzero(dk) == 0 and torch.count_nonzero(dv) == 0


def _doc_runs(L, seed, max_run, n_ids):
    """Document ids in runs of 1..max_run tokens, each run's id drawn from
    n_ids values (a document's runs are not contiguous)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ids = []
    while len(ids) < L:
        ids += [int(rng.integers(0, n_ids))] * int(rng.integers(1, max_run + 1))
    return np.array(ids[:L], dtype=np.int32)


@pytest.mark.parametrize("max_run,n_ids", [(100, 12), (40, 1000), (160, 3)])
@pytest.mark.parametrize("D", [64, 128])
def test_document_tile_filters(max_run, n_ids, D):
    # Runs longer and shorter than a 32-row wave, a 64-row tile and a 128-key
    # block, with few or many distinct ids (many: 64-bit filters collide), so
    # that waves, tiles and key blocks skip some tiles and keep the others;
    # q_valid and kv_valid cut the last runs.  Every element against the oracle.
    B, L, H = 2, 700, 2
    q, k, v, do = _inputs(B, L, L, H, H, D, 61 + D + max_run)
    ids = np.stack([_doc_runs(L, 7 + b + max_run, max_run, n_ids) for b in range(B)])
    for extra in ({}, {"causal": True, "q_valid": 650, "kv_valid": 600}):
        mask = {"segment_ids_q": ids, "segment_ids_kv": ids, "documents": True, **extra}
        dq, dk, dv = _run(q, k, v, do, mask, D ** -0.5)
        torch.cuda.synchronize()
        _check_full(q, k, v, do, mask, D ** -0.5, dq, dk, dv, True, False, f"docs {max_run}/{n_ids} {extra}")


def test_document_filters_in_every_order():
    # the filtered key-tile walk of dQ in each order: dK and dV do not depend
    # on it, dQ against the oracle
    B, L, H, D = 1, 900, 2, 64
    q, k, v, do = _inputs(B, L, L, H, H, D, 77)
    ids = _doc_runs(L, 78, 90, 6)[None]
    mask = {"segment_ids_q": ids, "segment_ids_kv": ids, "documents": True}
    n = (L + 63) // 64
    perm = torch.tensor(np.random.Generator(np.random.PCG64(79)).permutation(n), dtype=torch.int32, device=DEV)
    base = _run(q, k, v, do, mask, D ** -0.5)
    for order, kv in ((bw.BWA_ORDER_DESC, None), (bw.BWA_ORDER_OUTSIDE_IN, None), (bw.BWA_ORDER_CUSTOM, perm)):
        dq, dk, dv = _run(q, k, v, do, mask, D ** -0.5, order=order, kv_order=kv)
        torch.cuda.synchronize()
        assert torch.equal(dk, base[1]) and torch.equal(dv, base[2]), order
        _check_full(q, k, v, do, mask, D ** -0.5, dq, dk, dv, True, False, f"docs order {order}")


@pytest.mark.parametrize("ci", range(len(DILATED_SPLIT)))
def test_dilated_band_as_strided_windows(ci):
    # ascending order runs a band whose sizes are multiples of g as g strided
    # windows; descending order walks the band itself: both against the oracle
    g, w, Lq, Lk, off, qv, kvv = DILATED_SPLIT[ci]
    B, H, Hk, D = 2, 4, 2, 64
    q, k, v, do = _inputs(B, Lq, Lk, H, Hk, D, 90 + ci)
    mask = {"causal": True, "window": w, "dilation": g, "kv_offset": off, "q_valid": qv, "kv_valid": kvv}
    for order in (bw.BWA_ORDER_ASC, bw.BWA_ORDER_DESC):
        dq, dk, dv = _run(q, k, v, do, mask, D ** -0.5, order=order)
        torch.cuda.synchronize()
        _check_full(q, k, v, do, mask, D ** -0.5, dq, dk, dv, True, False, f"dilated {DILATED_SPLIT[ci]} {order}")


def test_padding_garbage_does_not_leak():
    # rows past q_valid and keys past kv_valid hold NaN: they must not reach
    # any gradient (they are read as zeros and masked)
    B, L, H, D = 1, 300, 2, 128
    q, k, v, do = _inputs(B, L, L, H, H, D, 31)
    mask = {"causal": True, "q_valid": 250, "kv_valid": 230}
    o, lse = bw.bwa_attn_fwd(q, k, v, mask, scale=D ** -0.5, out_dtype=torch.bfloat16)
    qn, kn, vn, don = q.clone(), k.clone(), v.clone(), do.clone()
    qn[:, 250:] = float("nan")
    don[:, 250:] = float("nan")
    kn[:, 230:] = float("nan")
    vn[:, 230:] = float("nan")
    dq, dk, dv = bw.bwa_attn_bwd(qn, kn, vn, o, lse, don, mask, scale=D ** -0.5)
    torch.cuda.synchronize()
    _check_full(q, k, v, do, mask, D ** -0.5, dq, dk, dv, True, False, "nan padding")


def test_workspace_errors():
    B, L, H, D = 1, 128, 2, 64
    q, k, v, do = _inputs(B, L, L, H, H, D, 3)
    o, lse = bw.bwa_attn_fwd(q, k, v, {}, out_dtype=torch.bfloat16)
    need = bw.bwa_attn_bwd_workspace({}, B, H, L, L, DEV)
    small = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(bw.BwaError) as e:
        bw.bwa_attn_bwd(q, k, v, o, lse, do, {}, workspace=small)
    assert e.value.status == 7  # BWA_ERR_CAPACITY
    with pytest.raises(bw.BwaError) as e:
        bw.bwa_attn_bwd(q.float(), k.float(), v.float(), o, lse, do, {})
    assert e.value.status == 6  # BWA_ERR_UNSUPPORTED


# ---------------------------------------------------------------- page shapes
# The flash-attention page's backward tables: tiles 128 x 128, mha, masks
# sliding_window:512/1024/2048, prefix_lm, dilated_sliding_window, document
# over 4096x4096, 4096x8192 and 8192x8192 (B, H and D are not stated; the
# window workload's B = 1, H = 16, D = 128 is used).  Sampled rows and keys
# of two heads are compared with the oracle.
PAGE = [("sliding_window", 512, 4096, 4096), ("sliding_window", 1024, 4096, 8192),
        ("sliding_window", 2048, 8192, 8192), ("prefix_lm", 0, 4096, 4096),
        ("dilated_sliding_window", 0, 4096, 4096), ("document", 0, 4096, 4096),
        ("two_sided_window", 0, 4096, 4096)]


def _page_mask(kind, W, Lq, Lk):
    if kind == "sliding_window":
        return {"causal": True, "window": W, "kv_offset": Lq - Lk}
    return synth.make_page_mask(kind, Lq, Lk)["mask"]


@pytest.mark.slow
@pytest.mark.parametrize("kind,W,Lq,Lk", PAGE)
def test_page_shapes_sampled(kind, W, Lq, Lk):
    B, H, D = 1, 16, 128
    q, k, v, do = _inputs(B, Lq, Lk, H, H, D, 77)
    mask = _page_mask(kind, W, Lq, Lk)
    scale = D ** -0.5
    dq, dk, dv = _run(q, k, v, do, mask, scale)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(Lq + Lk + W))
    rows = np.sort(np.concatenate([rng.choice(Lq, 60, replace=False), [0, Lq - 1]]))
    keys = np.sort(np.concatenate([rng.choice(Lk, 60, replace=False), [0, Lk - 1]]))
    m = mask_for_batch(mask, 0)
    for h in (0, H - 1):
        qh, kh, vh, gh = np64(q[0, :, h]), np64(k[0, :, h]), np64(v[0, :, h]), np64(do[0, :, h])
        ref_q = oracle.attention_backward_rows(qh, kh, vh, gh, m, scale, rows)
        ref_k, ref_v = oracle.attention_backward_keys(qh, kh, vh, gh, m, scale, keys)
        a_q, a_k, a_v = bwd_bounds(qh, kh, vh, gh, m, scale, rows, keys)
        assert_grad_close(np64(dq[0, rows, h]), ref_q, a_q, False, f"{kind} dq h{h}")
        assert_grad_close(np64(dk[0, keys, h]), ref_k, a_k, False, f"{kind} dk h{h}")
        assert_grad_close(np64(dv[0, keys, h]), ref_v, a_v, False, f"{kind} dv h{h}")
