"""csa_indexer_kl_grad_noalloc (the entry point that allocates nothing: its workspace
is a device array the library holds) against csa_indexer_kl_grad with a caller
workspace, on two calls in a row, the second with a smaller input.

Both run the same kernels, so d_q, d_w and the loss must be bit-identical; d_k takes
float atomics in either call, so it must agree within the reordering of float32
additions (the bound the backward's determinism test uses).
"""
from __future__ import annotations

import numpy as np
import pytest

from gpu_support import cpu, run_pack, to_device
from synth import pack_from_lengths

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _inputs(pack, seed):
    plan = run_pack(pack, return_topk_score=False)
    rng = np.random.default_rng(seed)
    idx = cpu(plan.topk_idx)
    p = torch.from_numpy((rng.random(idx.shape).astype(np.float32) * (idx >= 0)).astype(np.float32)).cuda()
    return plan, p


def _outputs(pack, plan):
    T, Tc = pack.Tq, plan.k_I_cmp.shape[0]
    return dict(d_q=torch.full((T, pack.H_I, pack.d_I), float("nan"), dtype=torch.bfloat16, device="cuda"),
                d_w=torch.full((T, pack.H_I), float("nan"), dtype=torch.float32, device="cuda"),
                d_k=torch.full((Tc, pack.d_I), float("nan"), dtype=torch.float32, device="cuda"),
                loss=torch.full((T,), float("nan"), dtype=torch.float32, device="cuda"))


def _call(pack, plan, p, out, noalloc):
    import sparse_attention_thd_amd as s
    L = plan.L
    args = (to_device(pack.q_I), to_device(pack.w), plan.k_I_cmp, plan.topk_idx, p, pack.topk, pack.Tq,
            plan.k_I_cmp.shape[0], pack.H_I, pack.d_I, L.cu_seqlens_q, L.cu_seqlens_kv, plan.cu_seqlens_cmp, L.B,
            L.global_start, pack.cmp_ratio, pack.max_seqlen_kv, 1.0 / pack.Tq, out["d_q"], out["d_w"], out["d_k"],
            out["loss"])
    if noalloc:
        s.csa_indexer_kl_grad_noalloc(*args)
    else:
        nb = s.csa_indexer_kl_grad_workspace_bytes(pack.Tq, pack.topk, pack.max_seqlen_kv, pack.cmp_ratio)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        s.csa_indexer_kl_grad(*args, workspace=ws)
    torch.cuda.synchronize()


def test_noalloc_matches_workspace_call_twice_second_smaller():
    packs = [pack_from_lengths("long", [2500, 37], seed=5, topk=64),            # 2537 queries, lists to 634 rows
             pack_from_lengths("select16", [600, 300, 1201], seed=4, topk=16)]  # fewer queries and slots
    for n, pack in enumerate(packs):
        print(f"[case] noalloc call {n + 1}: {pack.name} Tq={pack.Tq} topk={pack.topk} -> "
              f"csa_indexer_kl_grad_noalloc vs csa_indexer_kl_grad", flush=True)
        plan, p = _inputs(pack, 50 + n)
        ref, got = _outputs(pack, plan), _outputs(pack, plan)
        _call(pack, plan, p, ref, noalloc=False)
        _call(pack, plan, p, got, noalloc=True)
        for k in ("d_q", "d_w", "loss"):
            assert torch.equal(got[k], ref[k]), k
        assert not torch.isnan(got["d_k"]).any()
        torch.testing.assert_close(got["d_k"], ref["d_k"], rtol=1e-4, atol=1e-6)


def test_noalloc_refuses_a_call_beyond_its_scratch():
    """Tq * (4 topk + 2 nvis_cap) above 64 MiB fails on the host before any launch."""
    import sparse_attention_thd_amd as s
    pack = pack_from_lengths("select16", [600, 300, 1201], seed=4, topk=16)
    plan, p = _inputs(pack, 60)
    out = _outputs(pack, plan)
    L = plan.L
    huge_len = 1 << 30  # a max_seqlen_kv that makes the visible-row map alone exceed the scratch
    with pytest.raises(s.CsaError, match="scratch"):
        s.csa_indexer_kl_grad_noalloc(to_device(pack.q_I), to_device(pack.w), plan.k_I_cmp, plan.topk_idx, p,
                                      pack.topk, pack.Tq, plan.k_I_cmp.shape[0], pack.H_I, pack.d_I, L.cu_seqlens_q,
                                      L.cu_seqlens_kv, plan.cu_seqlens_cmp, L.B, L.global_start, pack.cmp_ratio,
                                      huge_len, 1.0, out["d_q"], out["d_w"], out["d_k"], out["loss"])
    assert torch.isnan(out["d_w"]).all(), "a refused call writes nothing"
