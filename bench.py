"""Benchmark of the blockwise attention forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dit_share]
                    [--launch auto|plain|balanced] [--pass fwd|bwd]

Prints ONE JSON line.  A step is one pass of the whole hot path over one
batch of synthetic input already resident in HBM.  The default workload is
one rank's share of 2-ring x 2-Ulysses video-DiT self-attention (720p
81-frame latent grid 21x45x80 = 75,600 tokens; this rank: 20 heads, the
query shard of 37,800 tokens, keys as 2 sequential hops of 37,800), and a
step runs: tile run lists for each hop, the fixed-m bound and gate over both
key chunks, per hop one gated attention launch (fixed-m loop for the heads
that pass the gate, online loop for the rest: one sink head), and the LSE
merge of the two hop partials into the bf16 output.

value      = counted attention FLOPs per step / step time (TFLOP/s), FLOPs
             counted on a 128x128 tile grid over non-skipped tiles, 4*D per
             visible (row, key) pair of those tiles.  (A dilated band whose
             sizes are multiples of its dilation g runs as g strided causal
             windows; it is counted on their grids.)
roofline   = the dominant kernel (the gated attention launch of one hop):
             algorithmic FLOPs per launch / its mean launch time (HIP events on
             the launch stream), against the bf16 dense matrix-core peak.
launch     = plain (one workgroup per query block) or balanced (one
             workgroup per compute unit over per-XCD queues, the last
             partial round of blocks cut along the keys and merged by a
             second kernel); auto takes balanced from 4 rounds of blocks up.
cpu_baseline = the fp64 oracle timed on the host on a bounded sample of the
             same workload (rank 0, N = 1 only).
--pass bwd  = (single-call workloads) time the backward pass instead: a step
             is one bwa_attn_bwd call (dK/dV and dQ kernels plus their plan
             and delta passes) on O and LSE from one forward call made before
             the timed region; FLOPs are counted as 10*D per visible pair of
             the same tiles (five matrix products: scores, dP, dV, dK, dQ).
measured_ceilings = what this device sustains, beside the published peaks: a
             bf16 matrix-core probe (register operands only; libbwa_probe.so)
             and a plain 1 GiB elementwise copy.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def _counted_flops(blocks, D, heads, lq, lk):
    """FLOPs on the 128x128 counting grid from a run list built at 128x128."""
    import numpy as np
    s = blocks.struct
    assert s.bq == 128 and s.bkv == 128
    total = 0.0
    for copy in range(s.batch):
        rp, b, e, _ = blocks.host(copy)
        for qb in range(s.n_qblocks):
            rows = min(lq, (qb + 1) * 128) - qb * 128
            for r in range(rp[qb], rp[qb + 1]):
                c0, c1 = int(b[r]) * 128, min(lk, int(e[r]) * 128)
                total += rows * (c1 - c0)
    return 4.0 * D * heads * total


class Timer:
    """HIP events recorded on the current (launch) stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def start(self, key):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return (key, e)

    def stop(self, tok):
        key, s = tok
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.setdefault(key, []).append((s, e))

    def mean_ms(self, key):
        ps = self.pairs.get(key, [])
        return sum(s.elapsed_time(e) for s, e in ps) / len(ps) if ps else float("nan")

    def reset(self):
        self.pairs = {}


def _source_sha(fname="attn_fwd.hip"):
    """Hash of a kernel source file and the shared device header it includes,
    without comments and blank lines."""
    code = []
    for f in (fname, "internal.h"):
        p = os.path.join(ROOT, "blockwise_attention_forward_amd", "csrc", f)
        for line in open(p, encoding="utf-8"):
            line = line.split("//", 1)[0].rstrip()
            if line:
                code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def _traffic(kernel_key, fname="attn_fwd.hip"):
    """HBM bytes per launch (or per call) from committed rocprofv3 counter runs, if still current."""
    p = os.path.join(ROOT, "profiles", "attn_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    rec = d.get(kernel_key)
    if not rec or rec.get("source_sha") != _source_sha(fname):
        return None
    return rec.get("bytes_per_launch")


def _warm_up(torch, step, args):
    """Untimed steps before the timed ones.  Unless --warmup fixes the count,
    run at least 3 and keep going until 300 ms have passed: the device's
    clocks take that long to settle under sustained load, and a call of a
    fraction of a millisecond would otherwise be timed on a cold device.
    Unless --steps fixes it, the timed count is then at least 20 steps and
    enough for about 200 ms.  Sets args.warmup and args.steps to the counts
    used."""
    t = time.perf_counter()
    n = 0
    while (n < args.warmup) if args.warmup is not None else (n < 3 or time.perf_counter() - t < 0.3):
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t) * 1e3 / max(n, 1)
    args.warmup = n
    if args.steps is None:
        args.steps = int(min(5000, max(20, math.ceil(200.0 / max(ms, 1e-3)))))


def _launcher(torch, bw, launch, q, lk, units):
    """The attention entry point for this workload: plain or balanced (with
    its workspace allocated once), and a description for the JSON line."""
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    if launch == "auto":
        launch = "balanced" if units >= 4 * n_cus else "plain"
    if launch == "plain":
        def carry(q, k, v, o_prev, lse_prev, mask=None, blocks=None, **kw):
            return bw.bwa_attn_fwd_carry(q, k, v, o_prev, lse_prev, mask, blocks=blocks, **kw)
        return bw.bwa_attn_fwd, carry, {"launch": "plain", "units": units}
    B, Lq, H, D = q.shape
    nbytes, cut, pieces = bw.bwa_attn_fwd_balanced_workspace(q.dtype, B, H, Lq, lk, D, plan=True)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)

    def call(q, k, v, mask=None, blocks=None, **kw):
        return bw.bwa_attn_fwd_balanced(q, k, v, mask, blocks=blocks, workspace=ws, **kw)

    def carry(q, k, v, o_prev, lse_prev, mask=None, blocks=None, **kw):
        return bw.bwa_attn_fwd_balanced(q, k, v, mask, blocks=blocks, workspace=ws, o_prev=o_prev,
                                        lse_prev=lse_prev, **kw)
    return call, carry, {"launch": "balanced", "units": units, "workgroups": n_cus, "cut_units": cut,
                         "pieces": pieces}


def setup_dit_share(torch, bw, synth, launch="auto"):
    d = synth.make_dit_share("cuda")
    q, ks, vs = d["q"], d["k_chunks"], d["v_chunks"]
    B, Lq, H, D = q.shape
    Lc = ks[0].shape[1]
    scale, tau = d["scale"], d["tau"]
    masks = [bw.Mask("cuda", kv_offset=off) for off in d["kv_offsets"]]
    bq, _ = bw.bwa_attn_tile(q.dtype, D)
    blocks = [bw.bwa_block_mask_build(m, B, Lq, Lc, bq, 128) for m in masks]
    count_lists = bw.bwa_block_mask_build(masks[0], B, Lq, Lc, 128, 128)
    bound_out = (torch.empty(B, H, device="cuda"), torch.empty(B, H, device="cuda"),
                 torch.empty(B, H, Lq, device="cuda"), torch.empty(B, H, dtype=torch.uint8, device="cuda"))
    o_parts = [torch.empty(B, Lq, H, D, device="cuda") for _ in ks]
    l_parts = [torch.empty(B, H, Lq, device="cuda") for _ in ks]
    o_out = torch.empty(B, Lq, H, D, dtype=torch.bfloat16, device="cuda")
    l_out = torch.empty(B, H, Lq, device="cuda")
    torch.cuda.synchronize()
    flops_hop = _counted_flops(count_lists, D, H, Lq, Lc)
    gate_host = None
    attn, attn_carry, launch_info = _launcher(torch, bw, launch, q, Lc, B * H * ((Lq + bq - 1) // bq))

    def step(timer=None):
        for t, m in enumerate(masks):
            bw.bwa_block_mask_build(m, B, Lq, Lc, bq, 128, out=blocks[t])
        tb = timer.start("bound") if timer else None
        kmax, mmax, mm, gate = bw.bwa_fixed_m_bound(q, ks, scale, tau, out=bound_out)
        if timer:
            timer.stop(tb)
        for t in range(len(ks)):
            tok = timer.start("hop") if timer else None
            attn(q, ks[t], vs[t], m=mm, mask=masks[t], blocks=blocks[t], scale=scale,
                 mode=bw.BWA_MODE_GATED, gate=gate, o=o_parts[t], lse=l_parts[t])
            if timer:
                timer.stop(tok)
        tm = timer.start("merge") if timer else None
        bw.bwa_lse_merge(o_parts, l_parts, o_out, l_out)
        if timer:
            timer.stop(tm)

    def step_carry(timer=None):
        """The same step with the hops chained by the carried partial: hop 0
        writes an fp32 partial, hop 1 merges into it in its epilogue and writes
        the bf16 result, so there is no separate merge launch."""
        for t, m in enumerate(masks):
            bw.bwa_block_mask_build(m, B, Lq, Lc, bq, 128, out=blocks[t])
        kmax, mmax, mm, gate = bw.bwa_fixed_m_bound(q, ks, scale, tau, out=bound_out)
        tok = timer.start("hop0") if timer else None
        attn(q, ks[0], vs[0], m=mm, mask=masks[0], blocks=blocks[0], scale=scale,
             mode=bw.BWA_MODE_GATED, gate=gate, o=o_parts[0], lse=l_parts[0])
        if timer:
            timer.stop(tok)
        for t in range(1, len(ks)):
            last = t == len(ks) - 1
            tok = timer.start("hop_carry") if timer else None
            attn_carry(q, ks[t], vs[t], o_parts[0], l_parts[0], m=mm, mask=masks[t], blocks=blocks[t],
                       scale=scale, mode=bw.BWA_MODE_GATED, gate=gate,
                       o=o_out if last else o_parts[0], lse=l_out if last else l_parts[0])
            if timer:
                timer.stop(tok)

    def online_hop(timer):
        tok = timer.start("online_hop")
        attn(q, ks[0], vs[0], mask=masks[0], blocks=blocks[0], scale=scale,
             mode=bw.BWA_MODE_ONLINE, o=o_parts[0], lse=l_parts[0])
        timer.stop(tok)
        # every head through the branch-free fixed-m body (timing only: the
        # sink head's output from this launch is not used)
        tok = timer.start("fixed_hop")
        attn(q, ks[0], vs[0], mask=masks[0], blocks=blocks[0], scale=scale, m=bound_out[2],
             mode=bw.BWA_MODE_FIXED_M, o=o_parts[0], lse=l_parts[0])
        timer.stop(tok)

    step()
    torch.cuda.synchronize()
    gate_host = bound_out[3].cpu()
    n_fixed = int(gate_host.sum())
    info = dict(
        workload="dit_share: one rank's share of ring2 x uly2 video-DiT self-attention "
                 "(21x45x80 latent tokens), B=1 H=20 D=128 bf16, Lq=37800 vs 2 KV hops of 37800, "
                 "fixed-m (gate 106.5) with one sink head on online fallback in one gated launch per hop, "
                 "LSE merge to bf16",
        B=B, H=H, D=D, Lq=Lq, Lk_per_hop=Lc, hops=len(ks), heads_fixed_m=n_fixed,
        sink_head=d["sink_head"], **launch_info)
    flops_step = flops_hop * len(ks)
    bytes_merge = (len(ks) * (B * Lq * H * D * 4 + B * H * Lq * 4) + B * Lq * H * D * 2 + B * H * Lq * 4)
    bytes_bound = (B * Lq * H * D * 2 + sum(B * k.shape[1] * H * D * 2 for k in ks) + B * H * Lq * 4 * 3)

    def sample_oracle():
        """fp64 oracle on a bounded sample: rows of one head against all 75,600 keys."""
        import numpy as np
        import oracle
        h = 0
        rows = synth.sample_rows(Lq, 32768, seed=11, must=[0, Lq - 1])
        qh = q[0, :, h].double().cpu().numpy()
        kh = torch.cat([k[0, :, h] for k in ks]).double().cpu().numpy()
        vh = torch.cat([v[0, :, h] for v in vs]).double().cpu().numpy()
        t0 = time.perf_counter()
        oracle.attention_rows(qh, kh, vh, {}, scale, rows)
        dt = time.perf_counter() - t0
        fl = 4.0 * D * len(rows) * kh.shape[0]
        return fl, dt, f"head 0, {len(rows)} seeded query rows x all {kh.shape[0]} keys (both hops), fp64"

    return dict(step=step, step_carry=step_carry, online_hop=online_hop, flops_step=flops_step, flops_dominant=flops_hop,
                dominant="hop", info=info, bytes_merge=bytes_merge, bytes_bound=bytes_bound,
                sample_oracle=sample_oracle, hops=len(ks), launch=launch_info["launch"])


def setup_single(torch, bw, synth, name, launch="auto", mode="online"):
    """One attention call of a masked workload (run lists + attention).

    mode "gated": the bound and gate of "Fixed-m softmax for 2D-ring x Ulysses
    attention (WAN 2.2)" (description) are computed in the step, and the call
    runs fixed-m on the heads that pass the gate, online on the rest."""
    if name == "varlen":
        d = synth.make_varlen("cuda")
        desc = ("varlen: H3 packed request, B=1 H=24 D=128 bf16, 33,024 tokens, cu_seqlens [0, 33002, 33024], "
                "22 alignment rows zeroed")
    elif name == "window":
        d = synth.make_window(8192, 8192, 2048, "cuda")
        desc = "window: causal sliding window W=2048, B=1 H=16 D=128 bf16, Lq=Lk=8192"
    elif name in ("long_causal", "long_causal_packed"):
        d = synth.make_long_causal("cuda", packed=name.endswith("packed"))
        desc = ("long_causal: B=1 H=8 D=128 bf16, Lq=Lk=1,048,576 causal"
                + (", packed segments of U[4096, 131072] tokens" if name.endswith("packed") else ""))
    elif name in synth.PAGE_MASKS:
        d = synth.make_page_mask(name, 8192, 8192, "cuda")
        desc = f"{name}: B=1 H=16 D=128 bf16, Lq=Lk=8192 ({synth.WORKLOADS['page_masks']})"
    else:
        raise ValueError(name)
    q, k, v, scale = d["q"], d["k"], d["v"], d["scale"]
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    mask = bw.Mask.of(d["mask"], "cuda")
    bq, _ = bw.bwa_attn_tile(q.dtype, D)
    blocks = bw.bwa_block_mask_build(mask, B, Lq, Lk, bq, 128)
    m = d["mask"]
    g = int(m.get("dilation", 0) or 0)
    off, qv, kvv = int(m.get("kv_offset", 0)), int(m.get("q_valid", Lq)), int(m.get("kv_valid", Lk))
    if g > 1 and all(x % g == 0 for x in (Lq, Lk, off, qv, kvv)):
        # A dilated band of this shape runs as g strided causal windows (one
        # per residue class): count the unmasked blocks of those windows, the
        # work the call does, not the blocks of the band (which would count
        # the g - 1 keys in g that the band hides).
        sub = dict(causal=True, window=-(-int(m["window"]) // g), kv_offset=off // g, q_valid=qv // g,
                   kv_valid=kvv // g)
        count_lists = bw.bwa_block_mask_build(sub, B, Lq // g, Lk // g, 128, 128)
        torch.cuda.synchronize()
        flops = g * _counted_flops(count_lists, D, H, Lq // g, Lk // g)
    else:
        count_lists = bw.bwa_block_mask_build(mask, B, Lq, Lk, 128, 128)
        torch.cuda.synchronize()
        flops = _counted_flops(count_lists, D, H, Lq, Lk)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, Lq, device="cuda")
    attn, _, launch_info = _launcher(torch, bw, launch, q, Lk, B * H * ((Lq + bq - 1) // bq))

    gated = mode == "gated"
    if gated:
        tau = 106.5
        bound_out = (torch.empty(B, H, device="cuda"), torch.empty(B, H, device="cuda"),
                     torch.empty(B, H, Lq, device="cuda"), torch.empty(B, H, dtype=torch.uint8, device="cuda"))

    def step(timer=None):
        bw.bwa_block_mask_build(mask, B, Lq, Lk, bq, 128, out=blocks)
        if gated:
            tb = timer.start("bound") if timer else None
            _, _, mm, gate = bw.bwa_fixed_m_bound(q, [k], scale, tau, kv_valid=[kvv], q_valid=qv, out=bound_out)
            if timer:
                timer.stop(tb)
            tok = timer.start("hop") if timer else None
            attn(q, k, v, mask, blocks=blocks, scale=scale, mode=bw.BWA_MODE_GATED, m=mm, gate=gate, o=o, lse=lse)
        else:
            tok = timer.start("hop") if timer else None
            attn(q, k, v, mask, blocks=blocks, scale=scale, o=o, lse=lse)
        if timer:
            timer.stop(tok)

    def sample_oracle():
        import oracle
        rows = synth.sample_rows(Lq, 64, seed=11, must=[0, Lq - 1])
        m = dict(d["mask"])
        for key in ("segment_ids_q", "segment_ids_kv"):  # batch element 0
            if m.get(key) is not None and getattr(m[key], "ndim", 1) == 2:
                m[key] = m[key][0]
        qh, kh, vh = (x[0, :, 0].double().cpu().numpy() for x in (q, k, v))
        t0 = time.perf_counter()
        oracle.attention_rows(qh, kh, vh, m, scale, rows)
        dt = time.perf_counter() - t0
        visible = sum(int(oracle.visibility([r], Lk, m, Lq).sum()) for r in rows)
        fl = 4.0 * D * float(visible)
        return fl, dt, f"head 0, {len(rows)} seeded query rows against their visible keys, fp64"

    info = dict(workload=desc, B=B, H=H, D=D, Lq=Lq, Lk=Lk, **launch_info)
    if gated:
        step()
        torch.cuda.synchronize()
        info.update(mode=f"gated: fixed-m (gate {tau}) on heads that pass, online on the rest; bound in the step",
                    heads_fixed_m=int(bound_out[3].sum().item()))
    else:
        info.update(mode="online")
    return dict(step=step, flops_step=flops, flops_dominant=flops, dominant="hop", info=info,
                sample_oracle=sample_oracle, data=d)


def _measured_ceilings(torch):
    """What this device sustains: bf16 matrix-core throughput (probe library)
    and the bandwidth of a plain elementwise copy (read N bytes, write N)."""
    import ctypes
    out = {}
    probe = os.path.join(ROOT, "blockwise_attention_forward_amd", "libbwa_probe.so")
    if os.path.exists(probe):
        lib = ctypes.CDLL(probe)
        f = lib.bwa_probe_mfma_bf16
        f.restype = ctypes.c_int32
        f.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        iters = 20000
        sink = torch.empty(256 * 4 * 256, device="cuda")
        clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        best = (0.0, float("nan"))
        for blocks in (256 * 2, 256 * 4):  # two or four wavefronts per SIMD: the better one counts
            assert f(iters // 10, blocks, sink.data_ptr(), clocks.data_ptr(), stream) == 0
            rates, ghz = [], []
            for _ in range(3):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                assert f(iters, blocks, sink.data_ptr(), clocks.data_ptr(), stream) == 0
                b.record()
                torch.cuda.synchronize()
                ms = a.elapsed_time(b)
                rates.append(blocks * 4 * iters * 4 * 32768.0 / (ms * 1e-3) / 1e12)
                cyc, ticks = (int(x) for x in clocks.cpu())
                ghz.append(cyc / (ticks / 100e6) / 1e9 if ticks else float("nan"))
            r = sum(rates) / len(rates)
            if r > best[0]:
                best = (r, sum(ghz) / len(ghz))
        out["mfma_bf16_TFLOPs"] = round(best[0], 1)
        out["mfma_probe_clock_GHz"] = round(best[1], 3)
        # the same products with one operand read from LDS per product (the
        # attention kernel's inner loop without softmax, copies and barriers)
        h = lib.bwa_probe_mfma_lds_bf16
        h.restype = ctypes.c_int32
        h.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        lsink = torch.empty(256 * 512, device="cuda")
        assert h(iters // 10, 256, lsink.data_ptr(), stream) == 0
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(3):
            assert h(iters, 256, lsink.data_ptr(), stream) == 0
        b.record()
        torch.cuda.synchronize()
        out["mfma_lds_bf16_TFLOPs"] = round(256 * 8 * iters * 8 * 32768.0 * 3 / (a.elapsed_time(b) * 1e-3) / 1e12, 1)
        # LDS operand bytes per product against matrix-core rate: the share of
        # the nominal peak with n 16-byte reads and m pairs of transposing
        # 8-byte reads per two products (the forward reads (1, 1), dK/dV (2, 1))
        m = lib.bwa_probe_mfma_lds_mix
        m.restype = ctypes.c_int32
        m.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        mix = {}
        mi = iters // 10
        for nb, nt in ((2, 0), (0, 2), (1, 1), (2, 1), (4, 0), (3, 1), (6, 0)):
            assert m(nb, nt, mi // 10, 256, lsink.data_ptr(), stream) == 0
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            assert m(nb, nt, mi, 256, lsink.data_ptr(), stream) == 0
            b.record()
            torch.cuda.synchronize()
            tf = 256 * 8 * mi * 8 * 32768.0 / (a.elapsed_time(b) * 1e-3) / 1e12
            mix[f"{(nb + nt) / 2:g}KB_per_product_b128x{nb}_trpair_x{nt}"] = round(100.0 * tf / PEAK_BF16_TFLOPS, 1)
        out["mfma_lds_mix_pct_of_peak"] = mix
        # streaming probes: the merge's mix (4 bytes read per byte written)
        # and a read-only pass (the bound's mix), 1 GiB of reads each
        g = lib.bwa_probe_stream
        g.restype = ctypes.c_int32
        g.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                      ctypes.c_void_p, ctypes.c_void_p]
        n16 = (1 << 30) // 16
        src = torch.empty(n16 * 4, dtype=torch.int32, device="cuda").fill_(1)
        dst = torch.empty(n16 // 4 * 4, dtype=torch.int32, device="cuda")
        ssink = torch.empty(4096 * 256, device="cuda")
        for key, ratio, chunks, dptr, moved in (("stream_read4_write1_GBps", 4, n16 // 4, dst.data_ptr(), n16 * 20),
                                                 ("stream_read_GBps", 1, n16, None, n16 * 16)):
            rates = []
            for blocks in (1024, 2048, 4096):
                assert g(src.data_ptr(), chunks, ratio, dptr, blocks, ssink.data_ptr(), stream) == 0
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(5):
                    assert g(src.data_ptr(), chunks, ratio, dptr, blocks, ssink.data_ptr(), stream) == 0
                b.record()
                torch.cuda.synchronize()
                rates.append(moved * 5 / (a.elapsed_time(b) * 1e-3) / 1e9)
            out[key] = round(max(rates), 1)
        del src, dst, ssink
    n = (1 << 30) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        torch.neg(src, out=dst)
    b.record()
    torch.cuda.synchronize()
    out["copy_GBps"] = round(2.0 * n * 4 * 5 / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
    del src, dst
    return out


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return len(os.sched_getaffinity(0))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: at least 20, and enough for about 200 ms)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: at least 3, and until 300 ms have passed)")
    ap.add_argument("--workload", default="dit_share",
                    choices=["dit_share", "varlen", "window", "long_causal", "long_causal_packed",
                             "prefix_lm", "dilated_sliding_window", "document", "two_sided_window"],
                    help="dit_share (default) is the measured configuration; the others time one masked call")
    ap.add_argument("--launch", default="auto", choices=["auto", "plain", "balanced"],
                    help="attention launch; auto: balanced from 4 rounds of query blocks per compute unit up")
    ap.add_argument("--pass", dest="which", default="fwd", choices=["fwd", "bwd"],
                    help="bwd: time the backward pass of a single-call workload")
    ap.add_argument("--mode", default="online", choices=["online", "gated"],
                    help="single-call workloads: online softmax, or the fixed-m bound and gate with online fallback")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run 3 plain elementwise copies of MIB MiB (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.which == "bwd" and args.mode == "gated":
        print("--mode gated applies to the forward pass", file=sys.stderr)
        sys.exit(2)
    if args.workload == "dit_share" and args.mode == "gated":
        print("the dit_share step is gated already (--mode applies to the single-call workloads)", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share only (one MI355X); multi-GPU runs are not part of "
              "this build: run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import blockwise_attention_forward_amd as bw
    import synth

    torch.cuda.set_device(0)
    if args.copy_calibration > 0:
        # A plain elementwise kernel of known traffic (reads and writes MIB MiB
        # each): the scale between HBM byte counters and bytes moved.
        n = (args.copy_calibration << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if args.workload != "dit_share":
        return run_single(args, torch, bw, synth)
    if args.which == "bwd":
        print("--pass bwd times a single-call workload (window, varlen, a page mask, long_causal)", file=sys.stderr)
        sys.exit(2)
    W = setup_dit_share(torch, bw, synth, args.launch)
    timer = Timer(torch)
    _warm_up(torch, W["step"], args)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for _ in range(args.steps):
        W["step"](timer)
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    value = W["flops_step"] / (ms_step * 1e-3) / 1e12
    ms_hop = timer.mean_ms("hop")
    ms_fixed = timer.mean_ms(W["dominant"])
    ms_merge = timer.mean_ms("merge")
    ms_bound = timer.mean_ms("bound")
    achieved = W["flops_dominant"] / (ms_fixed * 1e-3) / 1e12

    t2 = Timer(torch)
    for _ in range(5):
        W["online_hop"](t2)
    torch.cuda.synchronize()
    ms_online_hop = t2.mean_ms("online_hop")
    ms_fixed_hop = t2.mean_ms("fixed_hop")

    # the step with the hops chained by the carried partial (no merge launch)
    t3 = Timer(torch)
    for _ in range(min(args.warmup, 3)):  # the device is warm by now
        W["step_carry"]()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record()
    for _ in range(args.steps):
        W["step_carry"](t3)
    c1.record()
    torch.cuda.synchronize()
    ms_step_carry = c0.elapsed_time(c1) / args.steps

    meas = _measured_ceilings(torch)
    if "mfma_bf16_TFLOPs" in meas:
        meas["attn_pct_of_measured_mfma"] = round(100.0 * achieved / meas["mfma_bf16_TFLOPs"], 1)
    merge_gbps = W["bytes_merge"] / (ms_merge * 1e-3) / 1e9
    bound_gbps = W["bytes_bound"] / (ms_bound * 1e-3) / 1e9
    meas["merge_pct_of_copy"] = round(100.0 * merge_gbps / meas["copy_GBps"], 1)
    meas["bound_pct_of_copy"] = round(100.0 * bound_gbps / meas["copy_GBps"], 1)
    if "stream_read4_write1_GBps" in meas:
        meas["merge_pct_of_stream_read4_write1"] = round(100.0 * merge_gbps / meas["stream_read4_write1_GBps"], 1)
        meas["bound_pct_of_stream_read"] = round(100.0 * bound_gbps / meas["stream_read_GBps"], 1)

    cpu = None
    if not args.no_cpu_baseline:
        fl, dt, what = W["sample_oracle"]()
        cpu = {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
               "sample": what, "seconds": round(dt, 3),
               "host_cores_available": len(os.sched_getaffinity(0))}

    out = {
        "metric": "attention fwd TFLOP/s and % of bf16 MFMA peak; ms per KV hop",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": W["info"],
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "ms_per_kv_hop": round(ms_hop, 4),
        "online_only_ms_per_kv_hop": round(ms_online_hop, 4),
        "fixed_m_all_heads_ms_per_kv_hop": round(ms_fixed_hop, 4),
        "carried_hops": {"launch": W["launch"], "ms_per_step": round(ms_step_carry, 4),
                         "TFLOPs": round(W["flops_step"] / (ms_step_carry * 1e-3) / 1e12, 2),
                         "ms_hop0": round(t3.mean_ms("hop0"), 4),
                         "ms_carry_hop": round(t3.mean_ms("hop_carry"), 4)},
        "merge_ms": round(ms_merge, 4),
        "merge_GBps": round(merge_gbps, 1),
        "merge_pct_of_hbm_peak": round(100.0 * merge_gbps / PEAK_HBM_GBS, 1),
        "bound_ms": round(ms_bound, 4),
        "bound_GBps": round(bound_gbps, 1),
        "bound_pct_of_hbm_peak": round(100.0 * bound_gbps / PEAK_HBM_GBS, 1),
        "measured_ceilings": meas,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": _traffic("attn_fwd_bf16_bal_gated" if W["launch"] == "balanced"
                                         else "attn_fwd_bf16_gated")},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def setup_backward(torch, bw, synth, W):
    """The backward pass of a single-call workload: O and LSE from one forward
    call, then a step is one bwa_attn_bwd call (bf16 gradients)."""
    d = W["data"]
    q, k, v, scale = d["q"], d["k"], d["v"], d["scale"]
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    mask = bw.Mask.of(d["mask"], "cuda")
    o, lse = bw.bwa_attn_fwd(q, k, v, mask, scale=scale, out_dtype=torch.bfloat16)
    do = synth.normal(tuple(q.shape), 404, "cuda", torch.bfloat16)
    ws = torch.empty(max(bw.bwa_attn_bwd_workspace(mask, B, H, Lq, Lk, "cuda"), 1), dtype=torch.uint8, device="cuda")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    torch.cuda.synchronize()
    flops = 2.5 * W["flops_step"]

    def step(timer=None):
        tok = timer.start("hop") if timer else None
        bw.bwa_attn_bwd(q, k, v, o, lse, do, mask, scale=scale, workspace=ws, dq=dq, dk=dk, dv=dv)
        if timer:
            timer.stop(tok)

    def sample_oracle():
        import oracle
        rows = synth.sample_rows(Lq, 512, seed=11, must=[0, Lq - 1])
        m = dict(d["mask"])
        for key in ("segment_ids_q", "segment_ids_kv"):  # batch element 0
            if m.get(key) is not None and getattr(m[key], "ndim", 1) == 2:
                m[key] = m[key][0]
        qh, kh, vh, gh = (x[0, :, 0].double().cpu().numpy() for x in (q, k, v, do))
        t0 = time.perf_counter()
        oracle.attention_backward_rows(qh, kh, vh, gh, m, scale, rows)
        dt = time.perf_counter() - t0
        visible = sum(int(oracle.visibility([r], Lk, m, Lq).sum()) for r in rows)
        fl = 8.0 * D * float(visible)
        return fl, dt, (f"dQ of head 0, {len(rows)} seeded query rows against their visible keys, fp64; "
                        "8*D FLOP per visible pair (scores, O, dP and dQ products)")

    info = {key: W["info"][key] for key in ("workload", "B", "H", "D", "Lq", "Lk")}
    info["workload"] = "backward of " + info["workload"] + "; bf16 gradients, O and LSE from one forward call"
    return dict(step=step, flops_step=flops, flops_dominant=flops, dominant="hop", info=info,
                sample_oracle=sample_oracle)


def run_single(args, torch, bw, synth):
    """A masked workload: one attention call per step (bf16 in and out)."""
    W = setup_single(torch, bw, synth, args.workload, args.launch, args.mode)
    if args.which == "bwd":
        W = setup_backward(torch, bw, synth, W)
    timer = Timer(torch)
    _warm_up(torch, W["step"], args)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        W["step"](timer)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    ms_hop = timer.mean_ms("hop")
    value = W["flops_step"] / (ms_step * 1e-3) / 1e12
    achieved = W["flops_dominant"] / (ms_hop * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        fl, dt, what = W["sample_oracle"]()
        cpu = {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
               "sample": what, "seconds": round(dt, 3), "host_cores_available": len(os.sched_getaffinity(0))}
    bwd = args.which == "bwd"
    out = {
        "metric": ("attention bwd TFLOP/s and % of bf16 MFMA peak; ms per call" if bwd else
                   "attention fwd TFLOP/s and % of bf16 MFMA peak; ms per call"),
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic", "config": W["info"],
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        ("ms_backward" if bwd else "ms_attention"): round(ms_hop, 4),
        **({"ms_bound": round(timer.mean_ms("bound"), 4)} if args.mode == "gated" and not bwd else {}),
        "counted_TFLOP": round(W["flops_step"] / 1e12, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": _traffic("attn_bwd_window", "attn_bwd.hip") if bwd and args.workload == "window"
                     else None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
