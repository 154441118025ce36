"""GPU checks of the forward call's index-row kinds and of the cmp_residual argument.

* CSA_IDX_TOPK (the plan's default: the rows come from csa_indexer_topk for the same
  layout) skips the index row of queries with at most topk visible rows and reads
  the others without compaction; it must give bit-identical out and lse to
  CSA_IDX_ANY, which compacts every row, on the same top-k rows.
* CSA_IDX_ANY accepts rows in any order with holes and out-of-range entries; the
  valid entries define the set (one fixed case, and seeded random layouts whose rows
  hold random sets of distinct compressed rows, 1 to 2048 entries wide).
* A caller-held cmp_residual equal to len mod r changes nothing; one that disagrees
  poisons exactly the queries of that segment (NaN out / lse, an all -1 top-k row),
  and csa_validate_layout names it.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_support import LSE_ABS, assert_out_close, cpu, host_view, oracle_attention, oracle_tables, run_pack, \
    to_device
from synth import make_pack, pack_from_lengths

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _mla(plan, pack, cmp_idx, kind, residual=None):
    import sparse_attention_thd_amd as s
    L = plan.L
    out = torch.empty_like(plan.out)
    lse = torch.empty((L.Tq, plan.H), dtype=torch.float32, device="cuda")
    topk = cmp_idx.shape[1] if cmp_idx is not None else 0
    s.csa_sparse_mla_fwd(to_device(pack.q), to_device(pack.ori_kv), plan.cmp_kv, cmp_idx, topk, kind, L.Tq, L.Tkv,
                         plan.Tc_cap if plan.cmp_kv is not None else 0, plan.H, plan.d, L.cu_seqlens_q,
                         L.cu_seqlens_kv, plan.cu_seqlens_cmp, residual, L.B, L.global_start, plan.r, plan.wl, plan.wr,
                         to_device(pack.sinks), plan.scale, out, lse)
    torch.cuda.synchronize()
    return out, lse


PACKS = {
    "edges": lambda: pack_from_lengths("edges", [1, 3, 4, 5, 130, 257, 700], seed=3),
    "select16": lambda: pack_from_lengths("select16", [600, 300, 1201], seed=4, topk=16),
    "long": lambda: pack_from_lengths("long", [2500, 37], seed=5),
    "topk1024": lambda: pack_from_lengths("topk1024", [4600, 300], seed=22, topk=1024),
    "many_segs": lambda: pack_from_lengths("many_segs", [5 + (37 * k) % 120 for k in range(80)], seed=13, topk=32),
    "cp_small": lambda: pack_from_lengths("cp_small", [700, 1500, 900, 400], seed=8, q_rows=(1000, 2600),
                                          kv_rows=2600),
    "pack16k": lambda: make_pack("pack16k"),
}


@pytest.mark.parametrize("name", sorted(PACKS))
def test_topk_rows_kind_is_bit_identical_to_any_kind(name):
    import sparse_attention_thd_amd as s
    pack = PACKS[name]()
    print(f"[case] {name}: Tq={pack.Tq} topk={pack.topk} -> forward with CSA_IDX_TOPK and CSA_IDX_ANY", flush=True)
    plan = run_pack(pack, return_topk_score=False)
    assert plan.topk_idx is not None
    out_any, lse_any = _mla(plan, pack, plan.topk_idx, s.CSA_IDX_ANY)
    out_top, lse_top = _mla(plan, pack, plan.topk_idx, s.CSA_IDX_TOPK)
    assert torch.equal(out_top, plan.out)       # the plan runs the TOPK kind
    assert torch.equal(out_any, out_top)
    assert torch.equal(lse_any, lse_top)
    nv = cpu(plan.q_cmp_nvis)
    print(f"[case] {name}: {int((nv > pack.topk).sum())} of {pack.Tq} queries read their row", flush=True)


def test_any_kind_takes_rows_in_any_order_with_holes():
    """Rows shuffled, with -1 holes and entries past the compressed rows: the valid
    entries are the set (oracle attention on the same set)."""
    import sparse_attention_thd_amd as s
    pack = pack_from_lengths("select16", [600, 300, 1201], seed=4, topk=16)
    print("[case] select16: shuffled rows with holes -> CSA_IDX_ANY", flush=True)
    plan = run_pack(pack, return_topk_score=False)
    idx = cpu(plan.topk_idx)
    Tc = int(cpu(plan.cu_seqlens_cmp)[-1])
    rng = np.random.default_rng(77)
    wide = np.full((pack.Tq, 2 * pack.topk), -1, dtype=np.int32)
    for i in range(pack.Tq):
        row = np.concatenate([idx[i], np.full(pack.topk, -1, np.int32)])
        junk = rng.random(row.size) < 0.2
        row[junk & (row < 0)] = Tc + rng.integers(0, 50, size=int((junk & (row < 0)).sum()))  # past the rows
        wide[i] = rng.permutation(row)
    got, _ = _mla(plan, pack, torch.as_tensor(wide, device="cuda"), s.CSA_IDX_ANY)
    tabs = oracle_tables(pack)
    cmp_kv = oracle.round_to(oracle.compress(host_view(pack, "ori_kv"), pack.cu_seqlens_kv, 4), pack.dtype)
    qs = list(range(pack.Tq))
    ref, _ = oracle_attention(pack, tabs, qs, cmp_kv, idx, oracle.INDEXER)
    print("   ", assert_out_close(cpu(got), ref), flush=True)



def _any_rows(rng, tabs, Tq, Tc, width):
    """Per query: a random set of distinct compressed rows (its visible range, at times
    a few rows from anywhere in [0, Tc)), scattered over `width` entries among -1
    holes, other negative entries and entries at or past Tc.  Returns (rows, sets):
    the scattered rows and the same sets packed in front of -1 padding."""
    rows = np.full((Tq, width), -1, dtype=np.int64)
    sets = np.full((Tq, width), -1, dtype=np.int64)
    for i in range(Tq):
        lo, nv = int(tabs["q_cmp_lo"][i]), int(tabs["q_cmp_nvis"][i])
        pool = list(range(lo, lo + nv))
        if Tc > 0 and rng.random() < 0.3:
            pool += [int(c) for c in rng.integers(0, Tc, size=int(rng.integers(1, 8)))]
        pool = np.unique(np.asarray(pool, dtype=np.int64))
        n = int(rng.integers(0, min(pool.size, width) + 1)) if pool.size else 0
        chosen = rng.choice(pool, size=n, replace=False) if n else np.zeros(0, np.int64)
        sets[i, :n] = chosen
        junk = np.full(width - n, -1, dtype=np.int64)
        u = rng.random(junk.size)
        neg, past = u < 0.15, u >= 0.6
        junk[neg] = rng.integers(-(2 ** 31), -1, size=int(neg.sum()))
        junk[past] = np.where(rng.random(int(past.sum())) < 0.5, Tc + rng.integers(0, 1000, size=int(past.sum())),
                              rng.integers(Tc, 2 ** 31 - 1, size=int(past.sum())))
        rows[i] = rng.permutation(np.concatenate([chosen, junk]))
    return rows.astype(np.int32), sets


@pytest.mark.parametrize("seed", list(range(6)))
def test_any_kind_random_sets_on_random_layouts(seed):
    """Seeded random layouts (those of the random-layout tests, drawn from other seeds,
    ratio 4): out and lse of CSA_IDX_ANY rows against oracle attention on each row's
    set, for row widths from 1 to 2048."""
    import sparse_attention_thd_amd as s
    from test_gpu_random import _draw
    p = _draw(500 + seed)
    lengths = p.pop("lengths")
    p["cmp_ratio"] = 4
    pack = pack_from_lengths(f"any{seed}", lengths, seed=seed, indexer=True, **p)
    rng = np.random.default_rng(61000 + seed)
    width = int(rng.choice([1, 2, 16, 64, 128, 129, 200, 511, 1024, 2048]))
    plan = run_pack(pack, return_topk_score=False)
    tabs = oracle_tables(pack)
    Tc = int(tabs["cu_seqlens_cmp"][-1])
    print(f"[case] any{seed}: lengths={lengths} Tq={pack.Tq} Tc={Tc} width={width} -> CSA_IDX_ANY", flush=True)
    rows, sets = _any_rows(rng, tabs, pack.Tq, Tc, width)
    got, got_lse = _mla(plan, pack, torch.as_tensor(rows, device="cuda"), s.CSA_IDX_ANY)
    cmp_kv = oracle.round_to(oracle.compress(host_view(pack, "ori_kv"), pack.cu_seqlens_kv, 4), pack.dtype)
    ref, ref_lse = oracle_attention(pack, tabs, list(range(pack.Tq)), cmp_kv, sets, oracle.INDEXER)
    print("   ", assert_out_close(cpu(got), ref), flush=True)
    assert np.abs(cpu(got_lse) - ref_lse).max() <= LSE_ABS

def test_residual_argument_matches_or_poisons_its_segment():
    import sparse_attention_thd_amd as s
    pack = pack_from_lengths("edges", [1, 3, 4, 5, 130, 257, 700], seed=3)
    print("[case] edges: cmp_residual given (right, then one segment wrong)", flush=True)
    plan = run_pack(pack, return_topk_score=False)
    L = plan.L
    res_ok = plan.cmp_residual.clone()
    out_ok, lse_ok = _mla(plan, pack, plan.topk_idx, s.CSA_IDX_TOPK, res_ok)
    assert torch.equal(out_ok, plan.out)
    bad_seg = 5  # 257 rows: residual 1
    res_bad = res_ok.clone()
    res_bad[bad_seg] = 3
    out_bad, lse_bad = _mla(plan, pack, plan.topk_idx, s.CSA_IDX_TOPK, res_bad)
    cu = [int(v) for v in pack.cu_seqlens_q]
    inside = torch.zeros(L.Tq, dtype=torch.bool, device="cuda")
    inside[cu[bad_seg]:cu[bad_seg + 1]] = True
    assert torch.isnan(out_bad[inside].float()).all() and torch.isnan(lse_bad[inside]).all()
    assert torch.equal(out_bad[~inside], out_ok[~inside]) and torch.equal(lse_bad[~inside], lse_ok[~inside])
    # the indexer: the same segment's rows become all -1, the rest are unchanged
    idx = torch.empty_like(plan.topk_idx)
    for residual, expect_bad in ((res_ok, False), (res_bad, True)):
        s.csa_indexer_topk(to_device(pack.q_I), to_device(pack.w), plan.k_I_cmp, L.Tq, plan.Tc_cap, plan.H_I,
                           plan.d_I, L.cu_seqlens_q, L.cu_seqlens_kv, plan.cu_seqlens_cmp, residual, L.B,
                           L.global_start, plan.r, L.max_seqlen_kv, plan.topk, idx, workspace=plan.indexer_ws)
        torch.cuda.synchronize()
        assert torch.equal(idx[~inside], plan.topk_idx[~inside])
        if expect_bad:
            assert (idx[inside] == -1).all()
        else:
            assert torch.equal(idx, plan.topk_idx)
    # the validation call finds the wrong entry
    s.csa_validate_layout(L.cu_seqlens_q, L.cu_seqlens_kv, L.B, L.Tq, L.Tkv, L.global_start, L.max_seqlen_kv, 4,
                          plan.cu_seqlens_cmp, res_ok)
    with pytest.raises(s.CsaError, match="cmp_residual"):
        s.csa_validate_layout(L.cu_seqlens_q, L.cu_seqlens_kv, L.B, L.Tq, L.Tkv, L.global_start, L.max_seqlen_kv, 4,
                              plan.cu_seqlens_cmp, res_bad)
    cu_bad = plan.cu_seqlens_cmp.clone()
    cu_bad[-1] += 1
    with pytest.raises(s.CsaError, match="cu_seqlens_cmp"):
        s.csa_validate_layout(L.cu_seqlens_q, L.cu_seqlens_kv, L.B, L.Tq, L.Tkv, L.global_start, L.max_seqlen_kv, 4,
                              cu_bad, None)


def test_compressed_rows_bounded_by_the_buffer_rows():
    """Tc smaller than the layout's compressed count: rows past Tc are neither read
    by the indexer nor attended (attend-all mode), as if the segment had fewer rows."""
    import sparse_attention_thd_amd as s
    pack = pack_from_lengths("hca_small", [300, 701, 130], seed=7, cmp_ratio=128, indexer=False)
    print("[case] hca_small: attend-all forward with Tc cut to 3 rows", flush=True)
    plan = run_pack(pack, return_topk_score=False)
    L = plan.L
    Tc_cut = 3
    out = torch.empty_like(plan.out)
    s.csa_sparse_mla_fwd(to_device(pack.q), to_device(pack.ori_kv), plan.cmp_kv[:Tc_cut], None, 0, s.CSA_IDX_ANY,
                         L.Tq, L.Tkv, Tc_cut, plan.H, plan.d, L.cu_seqlens_q, L.cu_seqlens_kv, plan.cu_seqlens_cmp,
                         None, L.B, L.global_start, plan.r, plan.wl, plan.wr, to_device(pack.sinks), plan.scale, out)
    torch.cuda.synchronize()
    tabs = oracle_tables(pack)
    cmp_kv = oracle.round_to(oracle.compress(host_view(pack, "ori_kv"), pack.cu_seqlens_kv, 128), pack.dtype)
    # the same cut expressed as explicit rows: every visible row below Tc_cut
    lo, nv = tabs["q_cmp_lo"], tabs["q_cmp_nvis"]
    rows = np.full((pack.Tq, 8), -1, dtype=np.int64)
    for i in range(pack.Tq):
        keep = [c for c in range(int(lo[i]), int(lo[i]) + int(nv[i])) if c < Tc_cut]
        rows[i, :len(keep)] = keep
    qs = list(range(pack.Tq))
    ref, _ = oracle_attention(pack, tabs, qs, cmp_kv, rows, oracle.INDEXER)
    print("   ", assert_out_close(cpu(out), ref), flush=True)
