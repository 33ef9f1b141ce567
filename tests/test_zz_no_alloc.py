"""The allocation-free balanced launch against the balanced launch with a
caller workspace: same plan, same kernels, so the same bits, on two calls in
a row (the second smaller, on the scratch the first left behind), and within
the bf16 tolerance of the oracle on sampled rows."""

import math

import numpy as np
import pytest
import torch

import synth
from helpers import assert_close, oracle_attention

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts too
    pytest.skip("needs a GPU", allow_module_level=True)

import blockwise_attention_forward_amd as bw  # noqa: E402

DEV = "cuda"


def _case(B, H, L, D, seed, mask, n_cus, mode):
    q = synth.normal((B, L, H, D), seed, DEV)
    k = synth.normal((B, L, H, D), seed + 1, DEV)
    v = synth.normal((B, L, H, D), seed + 2, DEV)
    scale = 1 / math.sqrt(D)
    m = gate = None
    if mode != bw.BWA_MODE_ONLINE:
        _, _, m, gate = bw.bwa_fixed_m_bound(q, [k], scale, 106.5)
    nbytes, cut, pieces = bw.bwa_attn_fwd_balanced_workspace(q.dtype, B, H, L, L, D, n_cus, plan=True)
    assert cut > 0 and pieces > 1  # the plan cuts blocks, so the scratch holds partials
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    ref = bw.bwa_attn_fwd_balanced(q, k, v, mask, scale=scale, mode=mode, m=m, gate=gate, n_cus=n_cus,
                                   workspace=ws, out_dtype=torch.float32)
    got = bw.bwa_attn_fwd_balanced_noalloc(q, k, v, mask, scale=scale, mode=mode, m=m, gate=gate, n_cus=n_cus,
                                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    rows = synth.sample_rows(L, 96, seed=seed, must=[0, L - 1])
    o_ref, l_ref = oracle_attention(q, k, v, mask, scale, rows=rows)
    idx = torch.as_tensor(rows, device=DEV)
    assert_close(got[0].index_select(1, idx), got[1].index_select(2, idx), o_ref, l_ref, torch.bfloat16,
                 f"noalloc {B}x{H}x{L} {mask}")


def test_noalloc_matches_the_workspace_launch_twice_shrinking():
    _case(2, 4, 3000, 128, 70, {}, 40, bw.BWA_MODE_GATED)
    _case(1, 2, 1100, 64, 80, {"causal": True}, 16, bw.BWA_MODE_ONLINE)
