"""GPU checks of the index-row precondition check and of the CSA_DEBUG build.

csa_validate_topk_rows accepts the rows csa_indexer_topk emits and names the first
query whose row holds a compressed row it cannot see (past its visible count, or in
another segment) or a repeated entry.  The CSA_DEBUG build (libcsa_debug.so) runs that
check inside the backward, the KL gradient and the top-k-kind forward: with the
indexer's rows it gives the product library's results bit for bit, with a corrupted
row it refuses the call before launching anything.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

from gpu_support import cpu, run_pack, to_device
from synth import pack_from_lengths

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _pack():
    return pack_from_lengths("validate", [600, 300, 1201, 45], seed=31, topk=16)


def _check(plan, pack, rows):
    import sparse_attention_thd_amd as s
    L = plan.L
    s.csa_validate_topk_rows(rows, pack.topk, L.Tq, plan.Tc_cap, L.cu_seqlens_q, L.cu_seqlens_kv,
                             plan.cu_seqlens_cmp, L.B, L.global_start, plan.r)


def _corrupt(plan, pack, how):
    """A copy of the indexer's rows with one entry of one selecting query broken; returns
    (rows, the broken query)."""
    idx = cpu(plan.topk_idx).copy()
    lo, nv = cpu(plan.q_cmp_lo), cpu(plan.q_cmp_nvis)
    cu_cmp = cpu(plan.cu_seqlens_cmp)
    sel = np.nonzero(nv > pack.topk)[0]
    i = int(sel[len(sel) // 2])
    if how == "past_visible":
        idx[i, 3] = int(lo[i] + nv[i])             # the next compressed row: not complete yet
    elif how == "other_segment":
        b = int(np.searchsorted(cu_cmp, lo[i], side="right")) - 1
        idx[i, 3] = int(cu_cmp[b + 1])            # the next segment's first compressed row
    elif how == "repeat":
        idx[i, 5] = idx[i, 4]
    else:
        raise KeyError(how)
    return torch.from_numpy(idx).cuda(), i


def test_validate_accepts_the_indexer_rows():
    pack = _pack()
    print("[case] validate: indexer rows", flush=True)
    plan = run_pack(pack, return_topk_score=False)
    _check(plan, pack, plan.topk_idx)


@pytest.mark.parametrize("how,msg", [("past_visible", "not a compressed row visible"),
                                     ("other_segment", "not a compressed row visible"),
                                     ("repeat", "repeats an earlier entry")])
def test_validate_names_the_first_bad_query(how, msg):
    import sparse_attention_thd_amd as s
    pack = _pack()
    print(f"[case] validate: {how}", flush=True)
    plan = run_pack(pack, return_topk_score=False)
    rows, i = _corrupt(plan, pack, how)
    with pytest.raises(s.CsaError, match=msg) as err:
        _check(plan, pack, rows)
    assert f"query {i}," in str(err.value)


def _bwd(plan, pack, rows, out):
    """csa_sparse_mla_bwd with the given rows (plan's forward out / lse); returns d_cmp_kv and dq."""
    import sparse_attention_thd_amd as s
    L = plan.L
    T, H, d = pack.Tq, pack.H, pack.d
    rng = np.random.default_rng(5)
    dout = torch.from_numpy(rng.standard_normal((T, H, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    Tc = plan.cmp_kv.shape[0]
    nbytes = s.csa_sparse_mla_bwd_workspace_bytes(T, pack.ori_win_left, pack.ori_win_right, plan.cmp_kv, rows,
                                                  pack.topk, pack.max_seqlen_kv, pack.cmp_ratio)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dq = torch.empty_like(plan.out)
    d_ori = torch.empty((L.Tkv, d), dtype=torch.float32, device="cuda")
    d_cmp = torch.empty((Tc, d), dtype=torch.float32, device="cuda")
    d_sinks = torch.empty(H, dtype=torch.float32, device="cuda")
    s.csa_sparse_mla_bwd(to_device(pack.q), to_device(pack.ori_kv), plan.cmp_kv, rows, pack.topk, T, L.Tkv, Tc, H, d,
                         L.cu_seqlens_q, L.cu_seqlens_kv, plan.cu_seqlens_cmp, L.B, L.global_start, pack.cmp_ratio,
                         pack.ori_win_left, pack.ori_win_right, pack.max_seqlen_kv, to_device(pack.sinks),
                         pack.softmax_scale, out, plan.lse, dout, dq, d_ori, d_cmp, d_sinks, None, None, 0, ws)
    torch.cuda.synchronize()
    return cpu(dq), cpu(d_sinks)


def test_debug_build_checks_the_rows_of_the_backward(monkeypatch):
    import sparse_attention_thd_amd as s
    from sparse_attention_thd_amd import _lib
    if not os.path.exists(_lib.DEBUG_LIB_PATH):
        pytest.skip("libcsa_debug.so not built")
    pack = _pack()
    print("[case] debug build: backward with the indexer's rows, then with a corrupted row", flush=True)
    plan = run_pack(pack)
    ref = _bwd(plan, pack, plan.topk_idx, plan.out)
    dbg = _lib.load(_lib.DEBUG_LIB_PATH)
    monkeypatch.setattr(_lib, "LIB", dbg)
    assert s.csa_version().endswith("+debug")
    got = _bwd(plan, pack, plan.topk_idx, plan.out)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)
    rows, i = _corrupt(plan, pack, "repeat")
    with pytest.raises(s.CsaError, match=f"csa_sparse_mla_bwd: query {i},"):
        _bwd(plan, pack, rows, plan.out)
