"""GPU parity of the HIP library against the CPU oracle, through the C ABI.

Index tensors and compressed rows must be bit-exact.  Top-k sets must agree
outside the 1e-3 score-tie band.  Attention outputs must meet the stated
absolute bounds and the scale-aware relative bounds.  Every query of every
workload is compared, the full-size ones included (the oracle computes them one by
one, in chunks that print their progress).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_support import (OutClose, assert_out_close, check_topk_row, cpu, host_view, oracle_attention,
                         oracle_tables, run_pack, to_device, LSE_ABS)
from synth import make_pack, pack_from_lengths

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _small(name):
    if name == "edges":        # lengths 1, r-1, r, r+1 and multi-tile segments
        return pack_from_lengths("edges", [1, 3, 4, 5, 130, 257, 700], seed=3)
    if name == "select16":     # selection active in most queries
        return pack_from_lengths("select16", [600, 300, 1201], seed=4, topk=16)
    if name == "long":         # more than 512 candidates
        return pack_from_lengths("long", [2500, 37], seed=5)
    if name == "short_only":   # every segment shorter than the ratio: no compressed rows
        return pack_from_lengths("short_only", [1, 2, 3, 1], seed=6)
    if name == "hca_small":
        return pack_from_lengths("hca_small", [300, 701, 130], seed=7, cmp_ratio=128, indexer=False)
    if name == "cp_small":     # a context-parallel share whose cuts fall inside segments
        return pack_from_lengths("cp_small", [700, 1500, 900, 400], seed=8, q_rows=(1000, 2600), kv_rows=2600)
    if name == "win_right":
        return pack_from_lengths("win_right", [300, 411], seed=9, ori_win_left=20, ori_win_right=5, topk=32)
    if name == "ratio3":       # ratios that are not powers of two: the mean's one rounding of sum / r
        return pack_from_lengths("ratio3", [301, 700, 2, 130], seed=27, cmp_ratio=3, indexer=False)
    if name == "ratio5":
        return pack_from_lengths("ratio5", [17, 999, 4, 260], seed=28, cmp_ratio=5, indexer=False)
    if name == "no_compress":
        return pack_from_lengths("no_compress", [200, 333], seed=10, cmp_ratio=1, indexer=False)
    if name == "many_segs":    # more than 64 segments (segment search and bounds past one wavefront)
        return pack_from_lengths("many_segs", [5 + (37 * k) % 120 for k in range(80)], seed=13, topk=32)
    if name == "segs1100":     # more segments than the layout kernel stages in LDS (1024)
        return pack_from_lengths("segs1100", [1 + (7 * k) % 13 for k in range(1100)], seed=29, topk=2)
    if name == "pair_long":    # candidate lists of 2048+: queries scored in pairs; odd count, pairs across segments
        return pack_from_lengths("pair_long", [8301, 5, 2, 777], seed=24)
    if name == "topk1024":     # top-k above 512: the larger kernel instances, ~500 selecting queries
        return pack_from_lengths("topk1024", [4600, 300], seed=22, topk=1024)
    if name == "max_limits":   # the largest candidate list (32768 = 131072 / r) and top-k (2048) the calls accept
        return pack_from_lengths("max_limits", [131072], seed=25, topk=2048, q_rows=(131072 - 48, 131072))
    if name == "wide_window":  # 1024 window slots per query (32 window tiles)
        return pack_from_lengths("wide_window", [3000, 700], seed=26, ori_win_left=1023, topk=64)
    if name == "generic_f32":
        return pack_from_lengths("generic_f32", [5, 77, 140], seed=11, dtype="f32", H=4, d=64, H_I=2, d_I=32,
                                 ori_win_left=15, topk=8, q_scale=1.0, kv_scale=1.0, w_scale=2 ** -0.5,
                                 softmax_scale=0.125)
    if name == "generic_bf16":
        return pack_from_lengths("generic_bf16", [9, 120, 64], seed=12, H=8, d=128, H_I=4, d_I=32,
                                 ori_win_left=31, topk=8)
    raise KeyError(name)


FULL = ["tiny", "single4k", "pack16k", "hca32k", "cp32k", "stress"]
SMALL = ["edges", "select16", "long", "short_only", "hca_small", "ratio3", "ratio5", "cp_small", "win_right",
         "no_compress",
         "many_segs", "segs1100", "topk1024", "pair_long", "max_limits", "wide_window", "generic_f32", "generic_bf16"]
ALL = SMALL + FULL

_cache = {}


def result(name):
    """Run a workload once per session; keep host copies of everything."""
    if name in _cache:
        return _cache[name]
    print(f"\n[case] {name}: generating", flush=True)
    pack = make_pack(name) if name in FULL else _small(name)
    print(f"[case] {name}: Tq={pack.Tq} Tkv={pack.Tkv} B={pack.B} H={pack.H} d={pack.d} r={pack.cmp_ratio} "
          f"topk={pack.topk} dtype={pack.dtype} -> csa_forward on GPU", flush=True)
    plan = run_pack(pack)
    res = dict(pack=pack, plan=plan)
    for k in ("q_seg", "q_pos", "win_idx", "cu_seqlens_cmp", "cmp_residual", "q_cmp_lo", "q_cmp_nvis", "cmp_group",
              "cmp_kv", "k_I_cmp", "topk_idx", "topk_score", "out", "lse"):
        res[k] = cpu(getattr(plan, k))
    del plan
    res.pop("plan")
    torch.cuda.empty_cache()
    print(f"[case] {name}: oracle tables", flush=True)
    res["tabs"] = oracle_tables(pack)
    _cache[name] = res
    return res


CHUNK = 4096


def _queries(res):
    return list(range(res["pack"].Tq))


def _chunks(qs, name, what):
    for a in range(0, len(qs), CHUNK):
        if len(qs) > CHUNK:
            print(f"[case] {name}: {what} queries {a}..{min(a + CHUNK, len(qs))} of {len(qs)}", flush=True)
        yield qs[a:a + CHUNK]


@pytest.mark.parametrize("name", ALL)
def test_indices_bitexact(name):
    res = result(name)
    tabs = res["tabs"]
    Tc = int(tabs["cu_seqlens_cmp"][-1])
    for k in ("q_seg", "q_pos", "win_idx", "q_cmp_lo", "q_cmp_nvis", "cu_seqlens_cmp", "cmp_residual"):
        np.testing.assert_array_equal(res[k], tabs[k], err_msg=k)
    np.testing.assert_array_equal(res["cmp_group"][:Tc], tabs["cmp_group"], err_msg="cmp_group")
    assert (res["cmp_group"][Tc:] == -1).all(), "rows past the compressed count must stay untouched"


def _oracle_cmp(res, name):
    pack = res["pack"]
    key = "oracle_" + name
    if key not in res:
        src = host_view(pack, name)
        res[key] = oracle.round_to(oracle.compress(src, pack.cu_seqlens_kv, pack.cmp_ratio), pack.dtype)
    return res[key]


@pytest.mark.parametrize("name", [n for n in ALL if n != "no_compress"])
def test_compress_bitexact(name):
    res = result(name)
    pack = res["pack"]
    Tc = int(res["tabs"]["cu_seqlens_cmp"][-1])
    ref = _oracle_cmp(res, "ori_kv")
    np.testing.assert_array_equal(res["cmp_kv"][:Tc].astype(np.float64), ref)
    assert (res["cmp_kv"][Tc:] == 0).all()
    if pack.has_indexer and pack.cmp_ratio == 4:
        np.testing.assert_array_equal(res["k_I_cmp"][:Tc].astype(np.float64), _oracle_cmp(res, "k_I"))


INDEXER_CASES = [n for n in ALL if n not in ("hca32k", "hca_small", "ratio3", "ratio5", "no_compress")]


@pytest.mark.parametrize("name", INDEXER_CASES)
def test_indexer_topk_sets(name):
    res = result(name)
    pack, tabs = res["pack"], res["tabs"]
    kc = _oracle_cmp(res, "k_I")
    qI, w = host_view(pack, "q_I"), host_view(pack, "w")
    flips = nsel = 0
    for part in _chunks(_queries(res), name, "top-k sets,"):
        for i in part:
            lo, nv = int(tabs["q_cmp_lo"][i]), int(tabs["q_cmp_nvis"][i])
            s = oracle.indexer_scores(qI[i], w[i], kc[lo:lo + nv]) if nv else np.zeros(0)
            gsc = res["topk_score"][i] if nv > pack.topk else None
            flips += check_topk_row(res["topk_idx"][i], lo, nv, s, pack.topk, gpu_scores=gsc)
            nsel += nv > pack.topk
            if nv and nv <= pack.topk:
                np.testing.assert_allclose(res["topk_score"][i][:nv], s, rtol=1e-3, atol=1e-3)
    print(f"[case] {name}: {nsel} selecting queries checked, {flips} in-band swaps vs oracle order")


@pytest.mark.parametrize("name", ALL)
def test_attention_matches_oracle(name):
    res = result(name)
    pack, tabs = res["pack"], res["tabs"]
    qs = _queries(res)
    mode = oracle.layer_compress_mode(pack.cmp_ratio, int(tabs["cu_seqlens_cmp"][-1]))
    cmp_kv = _oracle_cmp(res, "ori_kv") if mode != oracle.NO_COMPRESS else None
    acc, lse_err = OutClose(), 0.0
    for part in _chunks(qs, name, "attention,"):
        rows = res["topk_idx"][part] if mode == oracle.INDEXER else None
        o, l = oracle_attention(pack, tabs, part, cmp_kv, rows, mode)
        acc.add(res["out"][part], o)
        lse_err = max(lse_err, float(np.abs(res["lse"][part] - l).max()))
    msg = acc.check(fp32=(pack.dtype == "f32"))
    print(f"[case] {name}: {len(qs)} queries; {msg}; max|lse diff|={lse_err:.3e}")
    assert lse_err <= LSE_ABS


@pytest.mark.parametrize("name", ["no_compress", "edges", "generic_bf16"])
def test_window_only_call_without_compressed_arrays(name):
    """Window branch alone through the C ABI, with cmp_kv, cmp_idx and cu_seqlens_cmp all NULL."""
    import sparse_attention_thd_amd as s
    res = result(name)
    pack, tabs = res["pack"], res["tabs"]
    print(f"[case] {name}: window-only csa_sparse_mla_fwd, NULL compressed arrays", flush=True)
    dt = torch.bfloat16 if pack.dtype == "bf16" else torch.float32
    out = torch.empty((pack.Tq, pack.H, pack.d), dtype=dt, device="cuda")
    lse = torch.empty((pack.Tq, pack.H), dtype=torch.float32, device="cuda")
    s.csa_sparse_mla_fwd(to_device(pack.q), to_device(pack.ori_kv), None, None, 0, s.CSA_IDX_ANY, pack.Tq, pack.Tkv,
                         0, pack.H, pack.d,
                         torch.as_tensor(np.asarray(pack.cu_seqlens_q), dtype=torch.int32, device="cuda"),
                         torch.as_tensor(np.asarray(pack.cu_seqlens_kv), dtype=torch.int32, device="cuda"), None, None,
                         pack.B, pack.global_start, pack.cmp_ratio, pack.ori_win_left, pack.ori_win_right,
                         to_device(pack.sinks), pack.softmax_scale, out, lse)
    torch.cuda.synchronize()
    qs = _queries(res)
    ref, ref_lse = oracle_attention(pack, tabs, qs, None, None, oracle.NO_COMPRESS)
    msg = assert_out_close(cpu(out)[qs], ref, fp32=(pack.dtype == "f32"))
    print(f"[case] {name}: {len(qs)} queries; {msg}")
    assert np.abs(cpu(lse)[qs] - ref_lse).max() <= LSE_ABS


def test_end_to_end_equals_oracle_selection_on_small_pack():
    """Whole forward vs the oracle's own forward (its own top-k) where no score ties exist."""
    res = result("select16")
    pack = res["pack"]
    ref = oracle.csa_forward(q=host_view(pack, "q"), ori_kv=host_view(pack, "ori_kv"), q_I=host_view(pack, "q_I"),
                             k_I=host_view(pack, "k_I"), w=host_view(pack, "w"), sinks=pack.sinks,
                             cu_seqlens_q=pack.cu_seqlens_q, cu_seqlens_kv=pack.cu_seqlens_kv, global_start=0,
                             cmp_ratio=4, ori_win_left=pack.ori_win_left, ori_win_right=0, topk=pack.topk,
                             softmax_scale=pack.softmax_scale, dtype="bf16")
    same = (res["topk_idx"] == ref["topk_idx"]).all(axis=1)
    assert same.mean() > 0.99
    assert_out_close(res["out"][same], ref["out"][same])


def test_repeat_runs_are_bit_identical():
    pack = make_pack("pack16k")
    print("[case] pack16k twice -> csa_forward", flush=True)
    a = run_pack(pack)
    out_a, idx_a = a.out.clone(), a.topk_idx.clone()
    del a
    b = run_pack(pack)
    assert torch.equal(out_a, b.out) and torch.equal(idx_a, b.topk_idx)


def test_packing_equals_separate_segments():
    pack = _small("edges")
    print("[case] edges packed vs per segment -> csa_forward", flush=True)
    full = run_pack(pack)
    cu = [int(v) for v in pack.cu_seqlens_kv]
    cu_cmp = full.cu_seqlens_cmp.cpu().numpy()
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        one = pack_from_lengths("one", [e - s], seed=0)
        for k in ("q", "ori_kv", "q_I", "k_I", "w"):
            setattr(one, k, getattr(pack, k)[s:e])
        one.sinks = pack.sinks
        sep = run_pack(one)
        assert torch.equal(full.out[s:e], sep.out), f"segment {b}"
        fi = full.topk_idx[s:e]
        rebased = torch.where(fi >= 0, fi - int(cu_cmp[b]), fi)
        assert torch.equal(rebased, sep.topk_idx), f"segment {b}"


def test_cp_share_equals_rows_of_full_prefix_run():
    """The 32768-row context-parallel share equals rows [65536, 98304) of the
    98304-row prefix run (same KV, queries before the cut filled at random)."""
    pack = make_pack("cp32k")
    print("[case] cp32k local share -> csa_forward", flush=True)
    part = run_pack(pack, return_topk_score=False)
    out_p, idx_p, win_p = part.out.clone(), part.topk_idx.clone(), part.win_idx.clone()
    del part
    torch.cuda.empty_cache()
    from sparse_attention_thd_amd import CsaPlan, ThdLayout
    a = pack.global_start
    g = torch.Generator(device="cuda").manual_seed(0)
    pre = lambda shape, s: (torch.randn(shape, generator=g, device="cuda") * s).to(torch.bfloat16)
    q = torch.cat([pre((a, 64, 512), 512 ** -0.5), to_device(pack.q)])
    q_I = torch.cat([pre((a, 64, 128), 1.0), to_device(pack.q_I)])
    w = torch.cat([pre((a, 64), 0.125), to_device(pack.w)])
    layout = ThdLayout.from_host(pack.cu_seqlens_kv, pack.cu_seqlens_kv, 0)
    plan = CsaPlan(layout, H=64, d=512, H_I=64, d_I=128, cmp_ratio=4, topk=512, softmax_scale=pack.softmax_scale)
    print("[case] cp32k full 98304-row prefix -> csa_forward", flush=True)
    plan.run(q, to_device(pack.ori_kv), sinks=to_device(pack.sinks), q_I=q_I, k_I=to_device(pack.k_I), w=w)
    torch.cuda.synchronize()
    assert torch.equal(plan.win_idx[a:], win_p)
    assert torch.equal(plan.topk_idx[a:], idx_p)
    assert torch.equal(plan.out[a:], out_p)


def test_empty_query_slice_is_a_no_op():
    from sparse_attention_thd_amd import CsaPlan, ThdLayout
    print("[case] Tq = 0 -> csa_forward", flush=True)
    layout = ThdLayout.from_host([0, 0], [0, 64], global_start=64)
    plan = CsaPlan(layout, H=64, d=512, H_I=64, d_I=128)
    kv = torch.zeros((64, 512), dtype=torch.bfloat16, device="cuda")
    kI = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda")
    out = plan.run(torch.zeros((0, 64, 512), dtype=torch.bfloat16, device="cuda"), kv,
                   q_I=torch.zeros((0, 64, 128), dtype=torch.bfloat16, device="cuda"), k_I=kI,
                   w=torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert out.shape == (0, 64, 512)
    assert plan.cu_seqlens_cmp.tolist() == [0, 16]


def test_validate_layout_on_device():
    import sparse_attention_thd_amd as s
    p = make_pack("cp32k") if "cp32k" not in _cache else _cache["cp32k"]["pack"]
    cq = torch.as_tensor(p.cu_seqlens_q, device="cuda")
    ck = torch.as_tensor(p.cu_seqlens_kv, device="cuda")
    s.csa_validate_layout(cq, ck, p.B, p.Tq, p.Tkv, p.global_start, p.max_seqlen_kv)
    with pytest.raises(s.CsaError):
        s.csa_validate_layout(cq, ck, p.B, p.Tq, p.Tkv, p.global_start + 1, p.max_seqlen_kv)
    with pytest.raises(s.CsaError):
        s.csa_validate_layout(cq, ck, p.B, p.Tq, p.Tkv, p.global_start, p.max_seqlen_kv - 1)


def test_binding_refuses_short_tensors():
    """A tensor holding fewer elements than the call's sizes give it is refused by the
    binding before anything is launched."""
    import sparse_attention_thd_amd as s
    print("[case] short tensors -> ValueError before any launch", flush=True)
    bf, i32 = torch.bfloat16, torch.int32
    cu = torch.tensor([0, 64], dtype=i32, device="cuda")
    Tq, H, d = 64, 64, 512
    q = torch.zeros((Tq, H, d), dtype=bf, device="cuda")
    kv = torch.zeros((Tq, d), dtype=bf, device="cuda")
    out = torch.zeros((Tq, H, d), dtype=bf, device="cuda")
    A = s.CSA_IDX_ANY
    with pytest.raises(ValueError, match="q holds"):
        s.csa_sparse_mla_fwd(q.view(-1)[:-1], kv, None, None, 0, A, Tq, Tq, 0, H, d, cu, cu, None, None, 1, 0, 4, 127,
                             0, None, 0.04, out)
    with pytest.raises(ValueError, match="out holds"):
        s.csa_sparse_mla_fwd(q, kv, None, None, 0, A, Tq, Tq, 0, H, d, cu, cu, None, None, 1, 0, 4, 127, 0, None, 0.04,
                             out.view(-1)[: Tq * H * d - d])
    with pytest.raises(ValueError, match="cu_seqlens_kv holds"):
        s.csa_sparse_mla_fwd(q, kv, None, None, 0, A, Tq, Tq, 0, H, d, cu, cu[:1], None, None, 1, 0, 4, 127, 0, None,
                             0.04, out)
    cu_cmp = torch.tensor([0, 16], dtype=i32, device="cuda")
    ckv = torch.zeros((16, d), dtype=bf, device="cuda")
    with pytest.raises(ValueError, match="cmp_kv holds"):  # fewer rows than the Tc the call names
        s.csa_sparse_mla_fwd(q, kv, ckv[:15], None, 0, A, Tq, Tq, 16, H, d, cu, cu, cu_cmp, None, 1, 0, 4, 127, 0,
                             None, 0.04, out)
    with pytest.raises(ValueError, match="cmp_residual holds"):
        s.csa_sparse_mla_fwd(q, kv, ckv, None, 0, A, Tq, Tq, 16, H, d, cu, cu, cu_cmp, cu_cmp[:0], 1, 0, 4, 127, 0,
                             None, 0.04, out)
    qI = torch.zeros((Tq, 64, 128), dtype=bf, device="cuda")
    w = torch.zeros((Tq, 64), dtype=bf, device="cuda")
    kI = torch.zeros((16, 128), dtype=bf, device="cuda")
    idx = torch.zeros((Tq, 8), dtype=i32, device="cuda")
    ws = torch.empty(s.csa_indexer_topk_workspace_bytes(Tq, 64, 4), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="topk_idx holds"):
        s.csa_indexer_topk(qI, w, kI, Tq, 16, 64, 128, cu, cu, cu_cmp, None, 1, 0, 4, 64, 16, idx, workspace=ws)
    with pytest.raises(ValueError, match="k_I_cmp holds"):
        s.csa_indexer_topk(qI, w, kI[:15], Tq, 16, 64, 128, cu, cu, cu_cmp, None, 1, 0, 4, 64, 8, idx, workspace=ws)
    with pytest.raises(s.CsaError, match="workspace"):  # a workspace one byte short: refused on the host
        s.csa_indexer_topk(qI, w, kI, Tq, 16, 64, 128, cu, cu, cu_cmp, None, 1, 0, 4, 64, 8, idx,
                           workspace=ws[:-1])
    torch.cuda.synchronize()
