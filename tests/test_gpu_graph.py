"""GPU check that the forward path and the deterministic backward replay inside a HIP graph.

Every compute call only enqueues kernels on the caller's stream (no synchronisation, no
allocation, no memset: buffers are cleared by kernels), so a caller can capture a whole
step once and replay it.  The test captures the forward (index build, both compressions,
indexer + top-k, sparse MLA) and then csa_sparse_mla_bwd_deterministic with torch's
graph capture, overwrites every output with garbage between replays (eager kernels), and
requires each replay to reproduce the eager run's results bit for bit (the forward and
the deterministic backward are bit-reproducible).
"""
from __future__ import annotations

import numpy as np
import pytest

from gpu_support import cpu, to_device
from synth import pack_from_lengths

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _forward_inputs(pack):
    return dict(q=to_device(pack.q), ori_kv=to_device(pack.ori_kv), sinks=to_device(pack.sinks),
                q_I=to_device(pack.q_I), k_I=to_device(pack.k_I), w=to_device(pack.w))


def _plan(pack):
    from sparse_attention_thd_amd import CsaPlan, ThdLayout
    layout = ThdLayout.from_host(pack.cu_seqlens_q, pack.cu_seqlens_kv, pack.global_start)
    return CsaPlan(layout, H=pack.H, d=pack.d, H_I=pack.H_I, d_I=pack.d_I, cmp_ratio=pack.cmp_ratio,
                   ori_win_left=pack.ori_win_left, ori_win_right=pack.ori_win_right, topk=pack.topk,
                   softmax_scale=pack.softmax_scale, dtype=torch.bfloat16, return_lse=True,
                   return_topk_score=True)


def _snapshot(tensors):
    return {k: cpu(v).copy() for k, v in tensors.items() if v is not None}


def _scribble(tensors):
    for v in tensors.values():
        if v is None:
            continue
        if v.dtype.is_floating_point:
            v.fill_(float("nan"))
        else:
            v.fill_(-7)


def test_forward_and_deterministic_backward_replay_in_a_graph():
    import sparse_attention_thd_amd as s
    pack = pack_from_lengths("graph", [900, 1300, 37, 2600], seed=41, topk=64)
    print(f"[case] graph: Tq={pack.Tq} B={pack.B} topk={pack.topk} -> eager forward + backward", flush=True)
    plan = _plan(pack)
    x = _forward_inputs(pack)
    L = plan.L
    T, H, d = pack.Tq, pack.H, pack.d
    Tc = plan.cmp_kv.shape[0]
    W = pack.ori_win_left + pack.ori_win_right + 1
    rng = np.random.default_rng(7)
    dout = torch.from_numpy(rng.standard_normal((T, H, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    nbytes = s.csa_sparse_mla_bwd_deterministic_workspace_bytes(T, L.B, pack.ori_win_left, pack.ori_win_right,
                                                                plan.cmp_kv, plan.topk_idx, pack.topk,
                                                                pack.max_seqlen_kv, pack.cmp_ratio)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    grads = dict(dq=torch.empty_like(plan.out), d_ori=torch.empty((L.Tkv, d), dtype=torch.float32, device="cuda"),
                 d_cmp=torch.empty((Tc, d), dtype=torch.float32, device="cuda"),
                 d_sinks=torch.empty(H, dtype=torch.float32, device="cuda"),
                 ori_l1=torch.empty((T, W), dtype=torch.float32, device="cuda"),
                 cmp_l1=torch.empty((T, pack.topk), dtype=torch.float32, device="cuda"))

    def step():
        plan.run(x["q"], x["ori_kv"], sinks=x["sinks"], q_I=x["q_I"], k_I=x["k_I"], w=x["w"])
        s.csa_sparse_mla_bwd_deterministic(
            x["q"], x["ori_kv"], plan.cmp_kv, plan.topk_idx, pack.topk, T, L.Tkv, Tc, H, d, L.cu_seqlens_q,
            L.cu_seqlens_kv, plan.cu_seqlens_cmp, L.B, L.global_start, pack.cmp_ratio, pack.ori_win_left,
            pack.ori_win_right, pack.max_seqlen_kv, x["sinks"], pack.softmax_scale, plan.out, plan.lse, dout,
            grads["dq"], grads["d_ori"], grads["d_cmp"], grads["d_sinks"], grads["ori_l1"], grads["cmp_l1"],
            pack.topk, ws)

    step()
    torch.cuda.synchronize()
    # compressed rows past the true count are never written (the plan keeps them zero)
    tc = int(cpu(plan.cu_seqlens_cmp)[-1])
    outputs = dict(out=plan.out, lse=plan.lse, topk_idx=plan.topk_idx, topk_score=plan.topk_score,
                   cmp_kv=plan.cmp_kv[:tc], k_I_cmp=plan.k_I_cmp[:tc], cu_seqlens_cmp=plan.cu_seqlens_cmp,
                   q_cmp_nvis=plan.q_cmp_nvis, win_idx=plan.win_idx, **grads)
    ref = _snapshot(outputs)

    # capture on a side stream (torch's graph capture needs a non-default stream)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        _scribble(outputs)  # eager kernels between the replays
        torch.cuda.synchronize()
        print(f"[case] graph: replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(outputs)
        for k, v in ref.items():
            assert np.array_equal(got[k], v, equal_nan=True), f"replay {rep}: {k} differs from the eager run"
