"""Throughput of the CSA forward on one MI355X (tokens/s), with the sparse-MLA
kernel's roofline fraction and the CPU oracle as a reported baseline.

    python bench.py [--steps K] [--warmup W] [--workload pack16k] [--seed 0] [--no-cpu-baseline]
                    [--no-backward] [--bwd-steps K] [--no-kl] [--no-learned]

A step is one whole forward over the 16384-token THD pack with every input
already resident in HBM: segment indices, compression of the latent KV and of
the indexer keys, lightning indexer + top-k, sparse MLA.  Prints one JSON line.
After the timed forward steps, a "backward" object times the sparse-MLA backward and
an "indexer_kl" object the indexer's KL-loss gradient, and a "learned_compressor"
object the learned gated compressor (hidden size 4096) for the latent and the indexer
keys, all on the same pack and outside the forward's timed region.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA fwd tokens/s (indexer+top-k+sparse MLA), 16k THD pack; % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
# sources of the sparse-MLA forward kernel (the traffic figure is tied to their hash)
MLA_SRCS = [os.path.join(ROOT, "sparse_attention_thd_amd", "csrc", f) for f in ("csa_mla.hip", "csa_tile.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sparse_mla_pack16k.txt")

WORKLOAD_TEXT = {
    "pack16k": "16384-token THD pack (12 segments, lognormal(7,1) lengths, none a multiple of 4), 64 heads x "
               "d512 shared latent KV (K=V), cmp_ratio 4, window 128, indexer 64x128, top-512, per-head sinks",
    "single4k": "one 4096-token segment, 64 heads x d512 latent KV, cmp_ratio 4, window 128, indexer 64x128, top-512",
    "hca32k": "32768-token THD pack (8 segments), cmp_ratio 128 compressor-only, window 128, 64 heads x d512",
    "cp32k": "context-parallel share: local rows [65536,98304) of a 131072-token pack, prefix KV 98304 rows, "
             "cmp_ratio 4, indexer 64x128, top-512, 64 heads x d512",
}


def _sha(paths):
    h = hashlib.sha256()
    for path in paths:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def _dev(a):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def algorithmic_work(plan, pack):
    """Attended rows (window + kept compressed rows) and indexer pairs that need scores."""
    import torch
    q_pos = plan.q_pos.long()
    wl, wr = pack.ori_win_left, pack.ori_win_right
    seg = plan.q_seg.long()
    cu = plan.L.cu_seqlens_kv.long()
    t = torch.arange(pack.Tq, device=q_pos.device) + pack.global_start
    lo = torch.maximum(cu[seg], t - wl)
    hi = torch.minimum(cu[seg + 1] - 1, t + wr)
    nwin = (hi - lo + 1).sum().item()
    nvis = plan.q_cmp_nvis.long()
    if plan.topk_idx is not None:
        ncmp = (plan.topk_idx >= 0).sum().item()
        need = nvis[nvis > pack.topk].sum().item()
    elif plan.cmp_kv is not None:
        ncmp = nvis.sum().item()
        need = 0
    else:
        ncmp = need = 0
    return int(nwin), int(ncmp), int(need)


def cpu_baseline(pack, budget_s=15.0):
    """The oracle, as it stands, on a bounded sample: full layout + compression, then
    indexer + attention for contiguous query chunks until the time budget is spent;
    the per-query rate is extrapolated to the whole pack."""
    import oracle
    from synth import bf16_bits_to_f32

    class Rows:
        def __init__(self, a):
            self.a, self.shape = a, a.shape

        def __len__(self):
            return self.a.shape[0]

        def __getitem__(self, k):
            v = self.a[k]
            return bf16_bits_to_f32(v) if v.dtype == np.uint16 else v

    V = {k: (Rows(getattr(pack, k)) if getattr(pack, k) is not None else None)
         for k in ("q", "ori_kv", "q_I", "k_I", "w")}
    t0 = time.perf_counter()
    tabs = oracle.build_indices(pack.cu_seqlens_q, pack.cu_seqlens_kv, pack.global_start, pack.Tq, pack.cmp_ratio,
                                pack.ori_win_left, pack.ori_win_right)
    mode = oracle.layer_compress_mode(pack.cmp_ratio, int(tabs["cu_seqlens_cmp"][-1]))
    cmp_kv = kI = None
    if mode != oracle.NO_COMPRESS:
        cmp_kv = oracle.round_to(oracle.compress(V["ori_kv"], pack.cu_seqlens_kv, pack.cmp_ratio), pack.dtype)
    if mode == oracle.INDEXER:
        kI = oracle.round_to(oracle.compress(V["k_I"], pack.cu_seqlens_kv, pack.cmp_ratio), pack.dtype)
    t_fixed = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    done, t_q = 0, 0.0
    chunk = 64
    starts = rng.permutation(np.arange(0, pack.Tq, chunk))
    for a in starts:
        if t_q >= budget_s:
            break
        qs = list(range(int(a), min(int(a) + chunk, pack.Tq)))
        t1 = time.perf_counter()
        cmp_idx = None
        if mode == oracle.INDEXER:
            idx, _ = oracle.indexer_topk(V["q_I"], V["w"], kI, tabs, pack.topk, queries=qs)
            cmp_idx = {i: idx[n] for n, i in enumerate(qs)}
        oracle.sparse_mla_fwd(V["q"], V["ori_kv"], cmp_kv, cmp_idx, tabs, pack.sinks, pack.softmax_scale,
                              pack.ori_win_left, pack.ori_win_right, pack.cu_seqlens_kv, pack.global_start,
                              queries=qs, attend_all_visible=(mode == oracle.COMPRESSOR_ONLY))
        t_q += time.perf_counter() - t1
        done += len(qs)
    total = t_fixed + t_q * pack.Tq / done
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    return {"value": pack.Tq / total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"layout + compression of the whole pack ({t_fixed:.1f} s), then indexer + attention for "
                      f"{done} of {pack.Tq} queries in distinct random 64-query chunks ({t_q:.1f} s), "
                      f"extrapolated per query to the whole pack"}


def gather_phases(plan, pack, ms):
    """Indices + the two compressions as HBM traffic: algorithmic bytes are the index
    tables written (q_seg, q_pos, q_cmp_lo, q_cmp_nvis: 16 B and the window slots 4 W B per
    query, 4 B per compressed row) and, per compressed row, r rows read and one written
    for the latent (d) and for the indexer keys (d_I)."""
    Tc = int(plan.cu_seqlens_cmp[-1].item())
    W = plan.wl + plan.wr + 1
    idx_bytes = pack.Tq * (16 + 4 * W) + 4 * Tc
    cmp_bytes = Tc * (plan.r + 1) * 2 * (pack.d + (pack.d_I if plan.k_I_cmp is not None else 0))
    total = idx_bytes + cmp_bytes
    gbs = total / (ms / 1e3) / 1e9
    return {"calls": "csa_build_indices + csa_compress (latent, indexer keys)", "avg_ms": ms,
            "algorithmic_bytes": total, "achieved_GBps": gbs, "frac_of_hbm": gbs / PEAK_HBM_GBS}


def backward_bench(plan, pack, inputs, nwin, ncmp, steps, warmup, deterministic=False):
    """csa_sparse_mla_bwd on the forward's output and lse with a seeded bf16 dout.

    Algorithmic work: five products of 64 heads x 512 dims per attended (query, key)
    pair (S and dP recomputed, dq, and the two row-gradient terms), 10 H d flops."""
    import torch
    from sparse_attention_thd_amd import _lib
    L = plan.L
    cmp_idx = plan.topk_idx
    topk = plan.topk if cmp_idx is not None else 0
    lse = torch.empty((pack.Tq, pack.H), dtype=torch.float32, device="cuda")
    _lib.csa_sparse_mla_fwd(inputs["q"], inputs["ori_kv"], plan.cmp_kv, cmp_idx, topk, _lib.CSA_IDX_TOPK, L.Tq, L.Tkv,
                            plan.Tc_cap if plan.cmp_kv is not None else 0, plan.H, plan.d, L.cu_seqlens_q,
                            L.cu_seqlens_kv, plan.cu_seqlens_cmp, plan.cmp_residual, L.B, L.global_start, plan.r,
                            plan.wl, plan.wr, inputs["sinks"], plan.scale, plan.out, lse)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    dout = torch.randn(plan.out.shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    Tc = plan.cmp_kv.shape[0] if plan.cmp_kv is not None else 0
    W = plan.wl + plan.wr + 1
    if cmp_idx is not None:
        slots = topk
    else:
        slots = max(1, L.max_seqlen_kv // plan.r) if plan.cmp_kv is not None else 0
    nbytes = _lib.csa_sparse_mla_bwd_workspace_bytes(L.Tq, plan.wl, plan.wr, plan.cmp_kv, cmp_idx, topk,
                                                     L.max_seqlen_kv, plan.r)
    torch.cuda.synchronize()
    base_alloc = torch.cuda.memory_allocated()
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    dq = torch.empty_like(plan.out)
    d_ori = torch.empty((L.Tkv, plan.d), dtype=torch.float32, device="cuda")
    d_cmp = torch.empty((Tc, plan.d), dtype=torch.float32, device="cuda") if Tc else None
    d_sinks = torch.empty(plan.H, dtype=torch.float32, device="cuda")
    ori_l1 = torch.empty((L.Tq, W), dtype=torch.float32, device="cuda")
    cmp_l1 = torch.empty((L.Tq, slots), dtype=torch.float32, device="cuda") if slots else None

    def bwd():
        _lib.csa_sparse_mla_bwd(inputs["q"], inputs["ori_kv"], plan.cmp_kv, cmp_idx, topk, L.Tq, L.Tkv, Tc, plan.H,
                                plan.d, L.cu_seqlens_q, L.cu_seqlens_kv, plan.cu_seqlens_cmp, L.B, L.global_start,
                                plan.r, plan.wl, plan.wr, L.max_seqlen_kv, inputs["sinks"], plan.scale, plan.out, lse,
                                dout, dq, d_ori, d_cmp, d_sinks, ori_l1, cmp_l1, slots, ws)

    torch.cuda.synchronize()
    call_alloc = torch.cuda.memory_allocated() - base_alloc  # workspace + every output of the call
    torch.cuda.reset_peak_memory_stats()
    for _ in range(warmup):
        bwd()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        e0.record(); bwd(); e1.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    flops = 10.0 * pack.H * pack.d * (nwin + ncmp)
    peak = torch.cuda.max_memory_allocated()  # of the atomic call, before the deterministic one
    res_det = None
    if deterministic:
        # the same call with bit-reproducible row gradients (per-item tiles + an ordered reduce)
        dbytes = _lib.csa_sparse_mla_bwd_deterministic_workspace_bytes(L.Tq, L.B, plan.wl, plan.wr, plan.cmp_kv,
                                                                       cmp_idx, topk, L.max_seqlen_kv, plan.r)
        dws = torch.empty(max(dbytes, 1), dtype=torch.uint8, device="cuda")

        def bwd_det():
            _lib.csa_sparse_mla_bwd_deterministic(
                inputs["q"], inputs["ori_kv"], plan.cmp_kv, cmp_idx, topk, L.Tq, L.Tkv, Tc, plan.H, plan.d,
                L.cu_seqlens_q, L.cu_seqlens_kv, plan.cu_seqlens_cmp, L.B, L.global_start, plan.r, plan.wl, plan.wr,
                L.max_seqlen_kv, inputs["sinks"], plan.scale, plan.out, lse, dout, dq, d_ori, d_cmp, d_sinks, ori_l1,
                cmp_l1, slots, dws)
        for _ in range(warmup):
            bwd_det()
        torch.cuda.synchronize()
        evd = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e0, e1 in evd:
            e0.record(); bwd_det(); e1.record()
        torch.cuda.synchronize()
        res_det = {"avg_call_ms": float(np.mean([a.elapsed_time(b) for a, b in evd])), "workspace_bytes": dbytes}
        del dws
    # The library allocates nothing here: the call's memory is the caller's workspace and
    # outputs; the peak is everything torch holds on the device while the calls run
    # (inputs, forward outputs, workspace, gradients).
    return {"call": "csa_sparse_mla_bwd (dq, d_ori_kv, d_cmp_kv, d_sinks, ori/cmp softmax_l1_norm)",
            "steps": steps, "avg_call_ms": ms, "tokens_per_s": pack.Tq / (ms / 1e3),
            "algorithmic_flops_per_call": flops, "achieved_tflops": flops / (ms / 1e3) / 1e12,
            "frac_of_bf16_peak": flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, "workspace_bytes": nbytes,
            "workspace_bytes_per_token": nbytes / max(pack.Tq, 1), "call_buffers_bytes": call_alloc,
            "peak_device_bytes": peak, "deterministic": res_det}


def kl_bench(plan, pack, inputs, ncmp, steps, warmup):
    """csa_indexer_kl_grad on the forward's top-k lists with seeded targets at the kept slots.

    Algorithmic work: three products of 64 heads x 128 dims per kept (query, row) pair
    (the scores u, d_q and d_k), 6 H_I d_I flops; the kernels recompute u twice more."""
    import torch
    from sparse_attention_thd_amd import _lib
    L = plan.L
    idx = plan.topk_idx
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4321)
    p = torch.rand(idx.shape, generator=gen, device="cuda") * (idx >= 0)
    Tc = plan.k_I_cmp.shape[0]
    nbytes = _lib.csa_indexer_kl_grad_workspace_bytes(L.Tq, plan.topk, L.max_seqlen_kv, plan.r)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    d_q = torch.empty_like(inputs["q_I"])
    d_w = torch.empty((L.Tq, plan.H_I), dtype=torch.float32, device="cuda")
    d_k = torch.empty((Tc, plan.d_I), dtype=torch.float32, device="cuda")
    loss = torch.empty(L.Tq, dtype=torch.float32, device="cuda")

    def kl():
        _lib.csa_indexer_kl_grad(inputs["q_I"], inputs["w"], plan.k_I_cmp, idx, p, plan.topk, L.Tq, Tc, plan.H_I,
                                 plan.d_I, L.cu_seqlens_q, L.cu_seqlens_kv, plan.cu_seqlens_cmp, L.B, L.global_start,
                                 plan.r, L.max_seqlen_kv, 1.0 / L.Tq, d_q, d_w, d_k, loss, ws)

    for _ in range(warmup):
        kl()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        e0.record(); kl(); e1.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    flops = 6.0 * plan.H_I * plan.d_I * ncmp
    return {"call": "csa_indexer_kl_grad (d_q_I, d_w, d_k_I_cmp, per-query KL loss)", "steps": steps,
            "avg_call_ms": ms, "tokens_per_s": pack.Tq / (ms / 1e3), "kept_pairs": ncmp,
            "algorithmic_flops_per_call": flops, "achieved_tflops": flops / (ms / 1e3) / 1e12,
            "frac_of_bf16_peak": flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, "workspace_bytes": nbytes}


def learned_bench(plan, pack, steps, warmup, D=4096):
    """csa_compress_learned on the pack's layout with seeded hidden rows and weights.

    Algorithmic work: the two projections of every grouped row (Tc * r rows, 2 C
    columns, C = 2 hd with overlap, hidden size D), 2 * rows * 2C * D flops; the
    pooling epilogue is O(rows * C)."""
    import torch
    from synth import compressor_inputs
    from sparse_attention_thd_amd import _lib
    L = plan.L
    Tc = int(plan.cu_seqlens_cmp[-1].item())
    res = {}
    for name, hd in (("latent_hd512", 512), ("indexer_hd128", 128)):
        ci = compressor_inputs(L.Tkv, D=D, hd=hd, overlap=True, seed=21)
        x, wkv, wgate, ape = _dev(ci.x), _dev(ci.wkv), _dev(ci.wgate), _dev(ci.ape)
        out = torch.empty((plan.Tc_cap, hd), dtype=torch.bfloat16, device="cuda")

        def run():
            _lib.csa_compress_learned(x, L.Tkv, D, wkv, wgate, ape, hd, True, L.cu_seqlens_kv, plan.cu_seqlens_cmp,
                                      L.B, plan.r, out, plan.Tc_cap)

        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e0, e1 in ev:
            e0.record(); run(); e1.record()
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        flops = 2.0 * (Tc * plan.r) * (2 * 2 * hd) * D
        res[name] = {"avg_call_ms": ms, "algorithmic_flops_per_call": flops,
                     "achieved_tflops": flops / (ms / 1e3) / 1e12,
                     "frac_of_bf16_peak": flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS}
        del x, wkv, wgate, ape, out
    res["call"] = f"csa_compress_learned (hidden {D}, cmp_ratio {plan.r}, overlap), bf16 out"
    res["steps"] = steps
    return res


def time_forward(plan, inputs, steps, warmup):
    """W untimed and K timed forward steps; per-phase HIP-event times (ms) on the launch
    stream: the index build + both compressions, the indexer + top-k, the sparse MLA."""
    import torch
    from sparse_attention_thd_amd import _lib
    L = plan.L

    def front():
        _lib.csa_build_indices(L.cu_seqlens_q, L.cu_seqlens_kv, L.B, L.Tq, L.Tkv, L.global_start, plan.r, plan.wl,
                               plan.wr, plan.q_seg, plan.q_pos, plan.win_idx, plan.cu_seqlens_cmp, plan.cmp_residual,
                               plan.q_cmp_lo, plan.q_cmp_nvis, plan.cmp_group, plan.Tc_cap)
        if plan.cmp_kv is not None:
            _lib.csa_compress(inputs["ori_kv"], L.Tkv, plan.d, L.cu_seqlens_kv, plan.cu_seqlens_cmp, L.B, plan.r,
                              plan.cmp_kv, plan.Tc_cap)
        if plan.topk_idx is not None:
            _lib.csa_compress(inputs["k_I"], L.Tkv, plan.d_I, L.cu_seqlens_kv, plan.cu_seqlens_cmp, L.B, plan.r,
                              plan.k_I_cmp, plan.Tc_cap)

    def indexer():
        if plan.topk_idx is not None:
            _lib.csa_indexer_topk(inputs["q_I"], inputs["w"], plan.k_I_cmp, L.Tq, plan.Tc_cap, plan.H_I, plan.d_I,
                                  L.cu_seqlens_q, L.cu_seqlens_kv, plan.cu_seqlens_cmp, plan.cmp_residual, L.B,
                                  L.global_start, plan.r, L.max_seqlen_kv, plan.topk, plan.topk_idx, None,
                                  plan.indexer_ws)

    def mla():
        cmp_idx = plan.topk_idx
        _lib.csa_sparse_mla_fwd(inputs["q"], inputs["ori_kv"], plan.cmp_kv, cmp_idx,
                                plan.topk if cmp_idx is not None else 0, _lib.CSA_IDX_TOPK, L.Tq, L.Tkv,
                                plan.Tc_cap if plan.cmp_kv is not None else 0, plan.H, plan.d, L.cu_seqlens_q,
                                L.cu_seqlens_kv, plan.cu_seqlens_cmp, plan.cmp_residual, L.B, L.global_start, plan.r,
                                plan.wl, plan.wr, inputs["sinks"], plan.scale, plan.out, None)

    for _ in range(warmup):
        front(); indexer(); mla()
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)
    ev = [(E(), E(), E(), E()) for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e0, e1, e2, e3 in ev:
        e0.record(); front(); e1.record(); indexer(); e2.record(); mla(); e3.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    return {"front": np.array([a.elapsed_time(b) for a, b, _, _ in ev]),
            "indexer": np.array([b.elapsed_time(c) for _, b, c, _ in ev]),
            "mla": np.array([c.elapsed_time(d) for _, _, c, d in ev]),
            "step": np.array([a.elapsed_time(d) for a, _, _, d in ev]), "wall": wall}


def workload_bench(name, seed, steps, warmup, backward=True):
    """Throughput of the whole forward on another workload's layout, inputs drawn on the
    device (same scales as the synthetic packs; the work counts depend only on the
    layout).  The sparse MLA is reported against the bf16 MFMA peak and, by its
    compulsory bytes (q and out of every query, every latent and compressed row once),
    against HBM: with few attended rows per query (the ratio-128 pack) it is HBM-bound."""
    import torch
    from synth import workload_layout
    from sparse_attention_thd_amd import CsaPlan, ThdLayout
    lay = workload_layout(name, seed)
    layout = ThdLayout.from_host(lay.cu_seqlens_q, lay.cu_seqlens_kv, lay.global_start)
    plan = CsaPlan(layout, H=lay.H, d=lay.d, H_I=lay.H_I, d_I=lay.d_I, cmp_ratio=lay.cmp_ratio,
                   ori_win_left=lay.ori_win_left, ori_win_right=lay.ori_win_right, topk=lay.topk,
                   softmax_scale=lay.softmax_scale, dtype=torch.bfloat16)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1000 + seed)
    rnd = lambda shape, sc: (torch.randn(shape, generator=gen, device="cuda") * sc).to(torch.bfloat16)
    inputs = dict(q=rnd((lay.Tq, lay.H, lay.d), lay.q_scale), ori_kv=rnd((lay.Tkv, lay.d), lay.kv_scale),
                  sinks=torch.randn(lay.H, generator=gen, device="cuda"))
    if lay.indexer:
        inputs.update(q_I=rnd((lay.Tq, lay.H_I, lay.d_I), 1.0), k_I=rnd((lay.Tkv, lay.d_I), 1.0),
                      w=rnd((lay.Tq, lay.H_I), lay.w_scale))
    torch.cuda.synchronize()
    t = time_forward(plan, inputs, steps, warmup)

    class P:  # the fields algorithmic_work reads
        Tq, global_start, ori_win_left, ori_win_right, topk = lay.Tq, lay.global_start, lay.ori_win_left, \
            lay.ori_win_right, lay.topk
    nwin, ncmp, need = algorithmic_work(plan, P)
    ms_step, mla_ms, idx_ms = float(t["step"].mean()), float(t["mla"].mean()), float(t["indexer"].mean())
    mla_flops = 4.0 * lay.H * lay.d * (nwin + ncmp)
    Tc = int(plan.cu_seqlens_cmp[-1].item())
    hbm_bytes = lay.Tq * lay.H * lay.d * 2 * 2 + (lay.Tkv + Tc) * lay.d * 2
    res = {"workload": f"{name}: {WORKLOAD_TEXT[name]}", "tokens": lay.Tq, "segments": lay.B, "steps": steps,
           "warmup": warmup, "ms_per_step": ms_step, "tokens_per_s": lay.Tq / (ms_step / 1e3),
           "phases_ms": {"indices+compress": float(t["front"].mean()), "indexer_topk": idx_ms, "sparse_mla": mla_ms},
           "sparse_mla": {"attended_rows": nwin + ncmp, "rows_per_query": (nwin + ncmp) / max(lay.Tq, 1),
                          "algorithmic_flops": mla_flops,
                          "frac_of_bf16_peak": mla_flops / (mla_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                          "compulsory_hbm_bytes": hbm_bytes,
                          "frac_of_hbm": hbm_bytes / (mla_ms / 1e3) / 1e9 / PEAK_HBM_GBS}}
    if plan.topk_idx is not None:
        idx_flops = 2.0 * lay.H_I * lay.d_I * need
        res["indexer"] = {"needed_score_flops": idx_flops,
                          "frac_of_bf16_peak": idx_flops / (idx_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS}
    if backward:
        class PB:  # the fields backward_bench reads
            H, d, Tq = lay.H, lay.d, lay.Tq
        res["backward"] = backward_bench(plan, PB, inputs, nwin, ncmp, max(2, steps // 4), 1)
    del inputs, plan
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="pack16k", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-backward", action="store_true", help="skip the sparse-MLA backward measurement")
    ap.add_argument("--bwd-steps", type=int, default=10)
    ap.add_argument("--no-kl", action="store_true", help="skip the indexer KL-loss gradient measurement")
    ap.add_argument("--no-learned", action="store_true", help="skip the learned compressor measurement")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the forward on the other workloads (single4k, hca32k, cp32k)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library runs one GPU's share "
              f"(a context-parallel slice is an input layout); sharding across GPUs is not implemented",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": src.numel() * 2, "copy_calibration_bytes_written":
                          dst.numel() * 2, "steps": max(args.steps, 1)}), flush=True)
        return
    from synth import make_pack
    from sparse_attention_thd_amd import CsaPlan, ThdLayout

    pack = make_pack(args.workload, args.seed)
    layout = ThdLayout.from_host(pack.cu_seqlens_q, pack.cu_seqlens_kv, pack.global_start)
    plan = CsaPlan(layout, H=pack.H, d=pack.d, H_I=pack.H_I, d_I=pack.d_I, cmp_ratio=pack.cmp_ratio,
                   ori_win_left=pack.ori_win_left, ori_win_right=pack.ori_win_right, topk=pack.topk,
                   softmax_scale=pack.softmax_scale, dtype=torch.bfloat16)
    inputs = dict(q=_dev(pack.q), ori_kv=_dev(pack.ori_kv), sinks=_dev(pack.sinks), q_I=_dev(pack.q_I),
                  k_I=_dev(pack.k_I), w=_dev(pack.w))
    torch.cuda.synchronize()

    t = time_forward(plan, inputs, args.steps, args.warmup)
    t_front, t_idx, t_mla, t_step, wall = t["front"], t["indexer"], t["mla"], t["step"], t["wall"]
    ms_step = float(t_step.mean())
    tokens_s = pack.Tq / (ms_step / 1e3)

    nwin, ncmp, need = algorithmic_work(plan, pack)
    mla_flops = 4.0 * pack.H * pack.d * (nwin + ncmp)
    mla_ms = float(t_mla.mean())
    mla_tflops = mla_flops / (mla_ms / 1e3) / 1e12
    idx_flops = 2.0 * pack.H_I * pack.d_I * need
    idx_ms = float(t_idx.mean())
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        # "key: value" lines written from the rocprofv3 FETCH_SIZE / WRITE_SIZE passes; the
        # figure only counts while the kernel source is the one it was measured on
        tr = dict(line.split(":", 1) for line in open(TRAFFIC_FILE) if ":" in line and not line.startswith("#"))
        tr = {k.strip(): v.strip() for k, v in tr.items()}
        if tr.get("kernel_source_sha256_16") == _sha(MLA_SRCS) and tr.get("workload") == args.workload:
            traffic = float(tr["hbm_bytes_per_launch"])
    result = {
        "metric": METRIC,
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {WORKLOAD_TEXT[args.workload]}", "seed": args.seed,
                   "tokens": pack.Tq, "segments": pack.B, "parallelism": "single GPU"},
        "roofline": {"kernel": "csa_sparse_mla_fwd", "bound": "mfma", "achieved": mla_tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": mla_tflops / PEAK_BF16_TFLOPS,
                     "traffic": traffic,
                     "algorithmic_flops_per_launch": mla_flops, "attended_rows": nwin + ncmp,
                     "avg_launch_ms": mla_ms},
        "phases_ms": {"indices+compress": float(t_front.mean()), "indexer_topk": idx_ms, "sparse_mla": mla_ms,
                      "step_p10": float(np.percentile(t_step, 10)), "step_p90": float(np.percentile(t_step, 90))},
        "gather_phases": gather_phases(plan, pack, float(t_front.mean())),
        "indexer": {"needed_score_flops": idx_flops,
                    "mfma_frac": (idx_flops / (idx_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS) if idx_ms > 0 else None},
        "host_wall_s": wall,
    }
    if not args.no_backward and pack.H == 64 and pack.d == 512:
        result["backward"] = backward_bench(plan, pack, inputs, nwin, ncmp, args.bwd_steps, 2, deterministic=True)
    if not args.no_kl and plan.topk_idx is not None and pack.H_I == 64 and pack.d_I == 128:
        result["indexer_kl"] = kl_bench(plan, pack, inputs, ncmp, args.bwd_steps, 2)
    if not args.no_learned and plan.r == 4 and plan.Tc_cap > 0:
        result["learned_compressor"] = learned_bench(plan, pack, args.bwd_steps, 2)
    if not args.no_workloads:
        del inputs, plan
        torch.cuda.empty_cache()
        result["workloads"] = {}
        for name in ("single4k", "hca32k", "cp32k"):
            if name != args.workload:
                result["workloads"][name] = workload_bench(name, args.seed, args.steps, args.warmup,
                                                           backward=not args.no_backward)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(pack, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
