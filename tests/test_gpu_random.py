"""GPU parity on seeded random layouts: segment lengths, window sides, top-k, ratio
(indexer, attend-every-visible-row, or window only) and query slices are drawn per
case, and the whole forward is checked against the fp64 oracle as in the fixed cases:
indices and compression bit-exact, top-k sets outside the tie band, attention and
log-sum-exp within the forward's tolerances on every query (the packs are small);
the first six layouts also run the sparse-MLA backward against the oracle backward,
and the layouts drawn with the indexer run its KL-loss gradient against the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_support import LSE_ABS, assert_out_close, check_topk_row, cpu, host_view, oracle_attention, oracle_tables, \
    run_pack
from synth import pack_from_lengths

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SEEDS = list(range(24))


def _draw(seed):
    """The layout parameters of one seed (cheap: no tensors)."""
    rng = np.random.default_rng(9000 + seed)
    nseg = int(rng.integers(1, 9))
    lengths = [int(v) for v in rng.integers(1, 900, size=nseg)]
    total = sum(lengths)
    ratio = int(rng.choice([4, 4, 4, 4, 8, 1, 3, 5, 128]))
    wl, wr = int(rng.integers(0, 200)), int(rng.choice([0, 0, 0, int(rng.integers(1, 6))]))
    topk = int(rng.choice([1, 7, 32, 64, 512]))
    q_rows = kv_rows = None
    if total > 8 and rng.random() < 0.4:   # a query slice of the stream with its prefix KV
        a = int(rng.integers(0, total // 2))
        b = int(rng.integers(a + 1, total + 1))
        q_rows, kv_rows = (a, b), b
    return dict(lengths=lengths, cmp_ratio=ratio, ori_win_left=wl, ori_win_right=wr, topk=topk, q_rows=q_rows,
                kv_rows=kv_rows)


def _random_pack(seed):
    p = _draw(seed)
    lengths = p.pop("lengths")
    return pack_from_lengths(f"random{seed}", lengths, seed=seed, indexer=(p["cmp_ratio"] == 4), **p)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_layout_matches_oracle(seed):
    pack = _random_pack(seed)
    print(f"[case] random{seed}: lengths={np.diff(pack.cu_seqlens_kv).tolist()} Tq={pack.Tq} gs={pack.global_start} "
          f"r={pack.cmp_ratio} window=({pack.ori_win_left},{pack.ori_win_right}) topk={pack.topk}", flush=True)
    plan = run_pack(pack)
    tabs = oracle_tables(pack)
    Tc = int(tabs["cu_seqlens_cmp"][-1])
    for k in ("q_seg", "q_pos", "win_idx", "q_cmp_lo", "q_cmp_nvis", "cu_seqlens_cmp", "cmp_residual"):
        np.testing.assert_array_equal(cpu(getattr(plan, k)), tabs[k], err_msg=k)
    mode = oracle.layer_compress_mode(pack.cmp_ratio, Tc)
    cmp_kv = None
    if mode != oracle.NO_COMPRESS:
        cmp_kv = oracle.round_to(oracle.compress(host_view(pack, "ori_kv"), pack.cu_seqlens_kv, pack.cmp_ratio),
                                 pack.dtype)
        np.testing.assert_array_equal(cpu(plan.cmp_kv)[:Tc].astype(np.float64), cmp_kv)
    rows = None
    if mode == oracle.INDEXER:
        kc = oracle.round_to(oracle.compress(host_view(pack, "k_I"), pack.cu_seqlens_kv, pack.cmp_ratio), pack.dtype)
        np.testing.assert_array_equal(cpu(plan.k_I_cmp)[:Tc].astype(np.float64), kc)
        idx, qI, w = cpu(plan.topk_idx), host_view(pack, "q_I"), host_view(pack, "w")
        for i in range(pack.Tq):
            lo, nv = int(tabs["q_cmp_lo"][i]), int(tabs["q_cmp_nvis"][i])
            s = oracle.indexer_scores(qI[i], w[i], kc[lo:lo + nv]) if nv else np.zeros(0)
            check_topk_row(idx[i], lo, nv, s, pack.topk)
        rows = idx
    qs = list(range(pack.Tq))
    out, lse = oracle_attention(pack, tabs, qs, cmp_kv, rows, mode)
    print("   ", assert_out_close(cpu(plan.out), out), flush=True)
    assert np.abs(cpu(plan.lse) - lse).max() <= LSE_ABS


@pytest.mark.parametrize("seed", SEEDS[:6])
def test_random_layout_backward_matches_oracle(seed):
    """The sparse-MLA backward on the same random layouts: dq, row gradients, sink
    gradient and the probability outputs against the oracle backward."""
    from test_gpu_bwd import L1_ABS, _close, _oracle, _run_bwd
    pack = _random_pack(seed)
    print(f"[case] random{seed}: backward Tq={pack.Tq} r={pack.cmp_ratio} topk={pack.topk}", flush=True)
    plan = run_pack(pack)
    got, dout, attend_all, slots = _run_bwd(pack, plan, seed=300 + seed)
    tabs = oracle_tables(pack)
    ref = _oracle(pack, tabs, plan, dout, attend_all, slots)
    _close(got["dq"], ref["dq"], "dq")
    _close(got["d_ori_kv"], ref["d_ori_kv"], "d_ori_kv")
    if ref["d_cmp_kv"] is not None:
        tc = ref["d_cmp_kv"].shape[0]
        _close(got["d_cmp_kv"][:tc], ref["d_cmp_kv"], "d_cmp_kv")
    _close(got["d_sinks"], ref["d_sinks"], "d_sinks")
    assert np.abs(got["ori_l1"] - ref["ori_l1"]).max() <= L1_ABS
    if slots:
        assert np.abs(got["cmp_l1"] - ref["cmp_l1"]).max() <= L1_ABS


def _indexer_seeds():
    """The seeds whose layouts run the indexer (ratio 4), from the draws alone."""
    return [s for s in SEEDS if _draw(s)["cmp_ratio"] == 4]


INDEXER_SEEDS = _indexer_seeds()


@pytest.mark.parametrize("seed", INDEXER_SEEDS)
def test_random_layout_kl_grad_matches_oracle(seed):
    """The indexer KL gradient on the random layouts that run the indexer."""
    from test_gpu_kl import _check, _targets
    pack = _random_pack(seed)
    assert pack.has_indexer and pack.cmp_ratio == 4
    print(f"[case] random{seed}: KL gradient Tq={pack.Tq} topk={pack.topk}", flush=True)
    plan = run_pack(pack)
    _check(pack, plan, _targets(plan, 400 + seed), 1.0 / max(pack.Tq, 1))
