"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Each test ties one oracle function to something other than itself: hand-evaluated
fixtures from the pages' definitions (tests/golden), brute-force enumeration on
tiny packs, special cases that reduce to library routines (torch's scaled dot
product attention, numpy's stable argsort, torch's bfloat16 cast), closed forms,
and the packing / context-parallel-slice invariants the pages state.
"""
from __future__ import annotations

import glob
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from dense_reference import dense_forward
from synth import make_pack

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_lengths(rng, nseg, lo=1, hi=40):
    return [int(v) for v in rng.integers(lo, hi + 1, size=nseg)]


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def _torch_round(dtype):
    if dtype == "bf16":
        return lambda x: torch.from_numpy(np.asarray(x, np.float64)).float().bfloat16().double().numpy()
    return lambda x: np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------- golden fixtures

@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "*.json"))))
def test_golden_layout(path):
    g = json.load(open(path))
    if "cu_seqlens_q" in g:
        out = oracle.build_indices(g["cu_seqlens_q"], g["cu_seqlens_kv"], g["global_start"], g["Tq"],
                                   g["cmp_ratio"], g["ori_win_left"], g["ori_win_right"])
    else:
        cu_cmp, res, grp = oracle.segment_table(g["cu_seqlens_kv"], g["cmp_ratio"])
        out = dict(cu_seqlens_cmp=cu_cmp, cmp_residual=res, cmp_group=grp)
    for k, v in g["expect"].items():
        np.testing.assert_array_equal(np.asarray(out[k]), np.asarray(v), err_msg=k)


def test_workload_check_values():
    # compressed layout of the 16k pack (lengths are never multiples of 4)
    p = make_pack("pack16k")
    cu_cmp, res, _ = oracle.segment_table(p.cu_seqlens_kv, 4)
    assert int(cu_cmp[-1]) == sum(int(L) // 4 for L in np.diff(p.cu_seqlens_kv))
    assert (res > 0).all()


# ----------------------------------------------------------------- index tensors

def _brute_layout(cu_q, cu_kv, gs, Tq, r, wl, wr):
    """Enumerate every stream row; no range arithmetic."""
    Tkv = int(cu_kv[-1])
    seg_of, pos_of = {}, {}
    for b in range(len(cu_kv) - 1):
        for n, k in enumerate(range(int(cu_kv[b]), int(cu_kv[b + 1]))):
            seg_of[k], pos_of[k] = b, n
    res = []
    for i in range(Tq):
        t = gs + i
        win = [k for k in range(Tkv) if seg_of[k] == seg_of[t] and t - wl <= k <= t + wr]
        res.append((seg_of[t], pos_of[t], win))
    # compressed cells: rows sharing (segment, pos // r), complete only
    cells = {}
    for k in range(Tkv):
        cells.setdefault((seg_of[k], pos_of[k] // r), []).append(k)
    full = sorted(c for c, m in cells.items() if len(m) == r)
    return res, full, cells


@pytest.mark.parametrize("seed", range(12))
def test_layout_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    L = _rand_lengths(rng, int(rng.integers(1, 6)), 1, 30)
    cu = _cu(L)
    total = int(cu[-1])
    r = int(rng.choice([1, 2, 4, 8]))
    wl, wr = int(rng.integers(0, 10)), int(rng.integers(0, 3))
    # either the whole stream or a context-parallel share with a prefix KV
    if seed % 2 and total > 2:
        a = int(rng.integers(0, total - 1))
        bq = int(rng.integers(a + 1, total + 1))
        kv_end = bq
    else:
        a, bq, kv_end = 0, total, total
    nb = int(np.searchsorted(cu, kv_end, side="left"))
    cu_kv = np.minimum(cu[:max(nb, 1) + 1], kv_end)
    cu_q = np.clip(cu_kv - a, 0, bq - a)
    Tq = bq - a
    out = oracle.build_indices(cu_q, cu_kv, a, Tq, r, wl, wr)
    res, full, cells = _brute_layout(cu_q, cu_kv, a, Tq, r, wl, wr)
    for i, (seg, pos, win) in enumerate(res):
        assert out["q_seg"][i] == seg and out["q_pos"][i] == pos
        row = out["win_idx"][i]
        valid = [int(v) for v in row if v >= 0]
        assert valid == win
        assert list(row[:len(valid)]) == valid and (row[len(valid):] == -1).all()
        vis = [c for c, (s, g) in enumerate(full) if s == seg and max(cells[(s, g)]) - int(cu_kv[s]) <= pos]
        lo, nv = int(out["q_cmp_lo"][i]), int(out["q_cmp_nvis"][i])
        assert vis == list(range(lo, lo + nv))
    assert int(out["cu_seqlens_cmp"][-1]) == len(full)
    assert list(out["cmp_group"]) == [g for _, g in full]
    for b in range(len(cu_kv) - 1):
        n = int(cu_kv[b + 1] - cu_kv[b])
        assert out["cmp_residual"][b] == n - r * sum(1 for s, _ in full if s == b)


def test_layout_rejects_query_outside_segment():
    with pytest.raises(ValueError):
        oracle.build_indices([0, 2], [0, 1, 4], 0, 2, 4, 3, 0)


# ----------------------------------------------------------------- rounding / compression

def test_round_to_bf16_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.0e-39], np.float32)])
    ref = torch.from_numpy(x).bfloat16().double().numpy()
    np.testing.assert_array_equal(oracle.round_to_bf16(x.astype(np.float64)), ref)


def test_compress_identity_at_ratio_one():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((23, 5))
    np.testing.assert_array_equal(oracle.compress(x, [0, 7, 23], 1), x)


@pytest.mark.parametrize("seed", range(10))
def test_compress_matches_cell_means_and_ignores_tails(seed):
    rng = np.random.default_rng(200 + seed)
    L = _rand_lengths(rng, 4, 1, 35)
    cu = _cu(L)
    r = int(rng.choice([2, 3, 4, 5, 8]))
    x = rng.standard_normal((int(cu[-1]), 6))
    got = oracle.compress(x, cu, r)
    _, full, cells = _brute_layout(cu, cu, 0, int(cu[-1]), r, 0, 0)
    ref = np.stack([np.mean(x[cells[c]], axis=0) for c in full]) if full else np.zeros((0, 6))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)
    # tail rows never enter a compressed row
    tail = [k for c, m in cells.items() if len(m) < r for k in m]
    x2 = x.copy()
    x2[tail] = 1e6
    np.testing.assert_array_equal(oracle.compress(x2, cu, r), got)


def test_compress_exact_mean_of_constant_groups():
    x = np.repeat(np.arange(12, dtype=np.float64)[:, None], 3, axis=1)
    x = np.repeat(x, 4, axis=0)           # 48 rows, each group of 4 is constant
    got = oracle.compress(x, [0, 48], 4)
    np.testing.assert_array_equal(got, np.repeat(np.arange(12.0)[:, None], 3, axis=1))


# ----------------------------------------------------------------- indexer

def _indexer_case(seed, H_I=3, d_I=8, nseg=3, maxlen=60):
    rng = np.random.default_rng(300 + seed)
    L = _rand_lengths(rng, nseg, 1, maxlen)
    cu = _cu(L)
    T = int(cu[-1])
    tabs = oracle.build_indices(cu, cu, 0, T, 4, 3, 0)
    Tc = int(tabs["cu_seqlens_cmp"][-1])
    qI = rng.standard_normal((T, H_I, d_I))
    w = rng.standard_normal((T, H_I))
    kc = rng.standard_normal((Tc, d_I))
    return tabs, qI, w, kc


def test_indexer_takes_every_candidate_when_topk_covers_them():
    tabs, qI, w, kc = _indexer_case(0)
    idx, _ = oracle.indexer_topk(qI, w, kc, tabs, topk=64)
    for i in range(len(idx)):
        lo, nv = int(tabs["q_cmp_lo"][i]), int(tabs["q_cmp_nvis"][i])
        assert list(idx[i][idx[i] >= 0]) == list(range(lo, lo + nv))


def test_indexer_zero_query_keeps_lowest_rows():
    tabs, qI, w, kc = _indexer_case(1, maxlen=80)
    idx, sc = oracle.indexer_topk(np.zeros_like(qI), w, kc, tabs, topk=3)
    for i in range(len(idx)):
        lo, nv = int(tabs["q_cmp_lo"][i]), int(tabs["q_cmp_nvis"][i])
        assert list(idx[i][idx[i] >= 0]) == list(range(lo, lo + min(nv, 3)))
        assert np.all(sc[i][idx[i] >= 0] == 0)


@pytest.mark.parametrize("seed", range(4))
def test_indexer_single_head_is_a_stable_sort(seed):
    tabs, qI, _, kc = _indexer_case(2 + seed, H_I=1, maxlen=90)
    w = np.ones((len(qI), 1))
    topk = 5
    idx, _ = oracle.indexer_topk(qI, w, kc, tabs, topk=topk)
    for i in range(len(idx)):
        lo, nv = int(tabs["q_cmp_lo"][i]), int(tabs["q_cmp_nvis"][i])
        s = np.maximum(kc[lo:lo + nv] @ qI[i, 0], 0)
        best = np.argsort(-s, kind="stable")[:topk]
        assert list(idx[i][idx[i] >= 0]) == sorted(lo + int(j) for j in best)


@pytest.mark.parametrize("h0", range(3))
def test_indexer_one_hot_weights_rank_by_that_head_alone(h0):
    """Weights e_h0 reduce the head-weighted sum to head h0's ReLU logits: the kept rows
    are the stable top-k of ReLU(q[h0] . k) (the other heads' q must not matter)."""
    tabs, qI, _, kc = _indexer_case(20 + h0, H_I=3, maxlen=90)
    w = np.zeros((len(qI), 3))
    w[:, h0] = 1.0
    noise = np.random.default_rng(5).standard_normal(qI.shape)
    qI2 = qI.copy()
    qI2[:, [h for h in range(3) if h != h0]] = noise[:, [h for h in range(3) if h != h0]]
    topk = 4
    a, sa = oracle.indexer_topk(qI, w, kc, tabs, topk=topk)
    b, _ = oracle.indexer_topk(qI2, w, kc, tabs, topk=topk)
    np.testing.assert_array_equal(a, b)
    for i in range(len(a)):
        lo, nv = int(tabs["q_cmp_lo"][i]), int(tabs["q_cmp_nvis"][i])
        s = np.array([max(float(np.dot(kc[lo + j], qI[i, h0])), 0.0) for j in range(nv)])
        best = np.argsort(-s, kind="stable")[:topk]
        kept = a[i][a[i] >= 0]
        assert list(kept) == sorted(lo + int(j) for j in best)
        # the reported score of a kept row is that head's ReLU logit itself (weight 1)
        np.testing.assert_allclose(sa[i][:len(kept)], s[kept - lo], rtol=1e-12, atol=1e-12)


def test_indexer_negated_weights_reverse_the_order_of_positive_logits():
    """With every logit of the weighted head positive, -w ranks the rows in the reverse
    order: the kept rows are the topk smallest logits (ties to the lower row)."""
    tabs, qI, _, kc = _indexer_case(30, H_I=2, maxlen=90)
    qI, kc = np.abs(qI), np.abs(kc)          # positive vectors: every logit > 0
    w = np.zeros((len(qI), 2))
    w[:, 1] = -0.5
    topk = 3
    idx, _ = oracle.indexer_topk(qI, w, kc, tabs, topk=topk)
    for i in range(len(idx)):
        lo, nv = int(tabs["q_cmp_lo"][i]), int(tabs["q_cmp_nvis"][i])
        logit = kc[lo:lo + nv] @ qI[i, 1]
        assert np.all(logit > 0)
        worst = np.argsort(logit, kind="stable")[:topk]
        assert list(idx[i][idx[i] >= 0]) == sorted(lo + int(j) for j in worst)


def test_indexer_scores_are_linear_in_the_head_weights():
    """score(w) = sum_h w_h score(e_h): the weighted sum over heads, each head's term
    taken from the one-hot score (all candidates kept, so every score is reported)."""
    tabs, qI, w, kc = _indexer_case(40, H_I=3, maxlen=50)
    topk = 64
    _, full = oracle.indexer_topk(qI, w, kc, tabs, topk=topk)
    parts = []
    for h in range(3):
        e = np.zeros_like(w)
        e[:, h] = 1.0
        parts.append(oracle.indexer_topk(qI, e, kc, tabs, topk=topk)[1])
    for i in range(len(full)):
        nv = int(tabs["q_cmp_nvis"][i])
        combo = sum(w[i, h] * parts[h][i][:nv] for h in range(3))
        np.testing.assert_allclose(full[i][:nv], combo, rtol=1e-12, atol=1e-12)
        for h in range(3):
            assert np.all(parts[h][i][:nv] >= 0)   # each head's term is a ReLU


def test_indexer_scores_only_own_segment_packing_invariant():
    tabs, qI, w, kc = _indexer_case(7, nseg=4, maxlen=70)
    idx, sc = oracle.indexer_topk(qI, w, kc, tabs, topk=4)
    cu_cmp = tabs["cu_seqlens_cmp"]
    for i in range(len(idx)):
        b = int(tabs["q_seg"][i])
        sel = idx[i][idx[i] >= 0]
        assert np.all((sel >= cu_cmp[b]) & (sel < cu_cmp[b + 1]))


# ----------------------------------------------------------------- sparse MLA

def _mla_case(rng, L, H=3, d=8, wl=1000, wr=0, sink=True):
    cu = _cu(L)
    T = int(cu[-1])
    q = rng.standard_normal((T, H, d))
    kv = rng.standard_normal((T, d))
    sinks = rng.standard_normal(H) if sink else None
    tabs = oracle.build_indices(cu, cu, 0, T, 4, wl, wr)
    return cu, T, q, kv, sinks, tabs


@pytest.mark.parametrize("seed", range(4))
def test_mla_window_only_is_causal_varlen_attention(seed):
    rng = np.random.default_rng(400 + seed)
    L = _rand_lengths(rng, 3, 1, 30)
    cu, T, q, kv, _, tabs = _mla_case(rng, L, sink=False)
    scale = 0.37
    out, _ = oracle.sparse_mla_fwd(q, kv, None, None, tabs, None, scale, 1000, 0, cu, 0)
    for b in range(len(L)):
        s, e = int(cu[b]), int(cu[b + 1])
        qq = torch.from_numpy(q[s:e]).permute(1, 0, 2)           # [H, L, d]
        kk = torch.from_numpy(kv[s:e])[None].expand(qq.shape[0], -1, -1)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, kk, is_causal=True, scale=scale)
        np.testing.assert_allclose(out[s:e], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_mla_band_window_with_right_side_is_masked_attention(seed):
    """A window with both sides, clamped to the query's segment: per segment, torch's
    attention with an explicit band mask (keys outside the segment do not exist there)."""
    rng = np.random.default_rng(450 + seed)
    L = _rand_lengths(rng, 3, 1, 30)
    wl, wr = int(rng.integers(0, 6)), int(rng.integers(1, 5))
    cu, T, q, kv, _, tabs = _mla_case(rng, L, wl=wl, wr=wr, sink=False)
    scale = 0.29
    out, _ = oracle.sparse_mla_fwd(q, kv, None, None, tabs, None, scale, wl, wr, cu, 0)
    for b in range(len(L)):
        s, e = int(cu[b]), int(cu[b + 1])
        pos = np.arange(e - s)
        band = (pos[None, :] >= pos[:, None] - wl) & (pos[None, :] <= pos[:, None] + wr)  # [query, key]
        qq = torch.from_numpy(q[s:e]).permute(1, 0, 2)
        kk = torch.from_numpy(kv[s:e])[None].expand(qq.shape[0], -1, -1)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, kk, attn_mask=torch.from_numpy(band),
                                                               scale=scale)
        np.testing.assert_allclose(out[s:e], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_mla_sink_is_an_extra_zero_valued_logit(seed):
    rng = np.random.default_rng(500 + seed)
    L = _rand_lengths(rng, 2, 1, 25)
    cu, T, q, kv, sinks, tabs = _mla_case(rng, L, wl=5)
    scale = 0.5
    out, _ = oracle.sparse_mla_fwd(q, kv, None, None, tabs, sinks, scale, 5, 0, cu, 0)
    H = q.shape[1]
    for b in range(len(L)):
        s, e = int(cu[b]), int(cu[b + 1])
        n = e - s
        qq = torch.from_numpy(q[s:e]).permute(1, 0, 2)
        kk = torch.cat([torch.from_numpy(kv[s:e]), torch.zeros(1, kv.shape[1], dtype=torch.float64)])
        kk = kk[None].expand(H, -1, -1)
        band = torch.full((n, n + 1), -math.inf, dtype=torch.float64)
        for a in range(n):
            band[a, max(0, a - 5):a + 1] = 0.0
        mask = band[None].repeat(H, 1, 1)
        mask[:, :, n] = torch.from_numpy(sinks)[:, None]
        # the appended zero key has logit 0, so its masked logit is exactly sink[h]; its value is 0
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, kk, attn_mask=mask, scale=scale)
        np.testing.assert_allclose(out[s:e], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_mla_zero_query_closed_form():
    rng = np.random.default_rng(6)
    cu, T, q, kv, sinks, tabs = _mla_case(rng, [9, 14], wl=3)
    q[:] = 0
    out, lse = oracle.sparse_mla_fwd(q, kv, None, None, tabs, sinks, 1.0, 3, 0, cu, 0)
    for i in range(T):
        b = int(tabs["q_seg"][i])
        lo = max(int(cu[b]), i - 3)
        n = i - lo + 1
        for h in range(q.shape[1]):
            den = n + math.exp(sinks[h])
            np.testing.assert_allclose(out[i, h], kv[lo:i + 1].sum(0) / den, rtol=1e-13, atol=1e-15)
            assert abs(lse[i, h] - math.log(den)) < 1e-13


def test_mla_single_key_closed_form_and_large_sink():
    rng = np.random.default_rng(7)
    cu, T, q, kv, sinks, tabs = _mla_case(rng, [5, 6], wl=0)
    scale = 0.3
    out, _ = oracle.sparse_mla_fwd(q, kv, None, None, tabs, sinks, scale, 0, 0, cu, 0)
    for i in range(T):
        for h in range(q.shape[1]):
            z = scale * q[i, h] @ kv[i]
            np.testing.assert_allclose(out[i, h], kv[i] / (1 + math.exp(sinks[h] - z)), rtol=1e-13)
    big = np.full(q.shape[1], 1e3)
    out, _ = oracle.sparse_mla_fwd(q, kv, None, None, tabs, big, scale, 0, 0, cu, 0)
    assert np.abs(out).max() < 1e-300


# ----------------------------------------------------------------- whole forward

def _tiny_forward_case(seed, dtype, mode_ratio=4):
    rng = np.random.default_rng(600 + seed)
    L = _rand_lengths(rng, int(rng.integers(1, 4)), 1, 45)
    cu = _cu(L)
    T = int(cu[-1])
    H, d, HI, dI = 3, 8, 2, 4
    f = (lambda a: torch.from_numpy(a).float().bfloat16().double().numpy()) if dtype == "bf16" else \
        (lambda a: a.astype(np.float32).astype(np.float64))
    args = dict(q=f(rng.standard_normal((T, H, d))), ori_kv=f(rng.standard_normal((T, d))),
                q_I=f(rng.standard_normal((T, HI, dI))), k_I=f(rng.standard_normal((T, dI))),
                w=f(rng.standard_normal((T, HI))), sinks=rng.standard_normal(H),
                cu_seqlens_q=cu, cu_seqlens_kv=cu, global_start=0, cmp_ratio=mode_ratio,
                ori_win_left=int(rng.integers(0, 8)), ori_win_right=0, topk=int(rng.integers(1, 5)),
                softmax_scale=0.4)
    return args


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("ratio", [4, 8, 1])
def test_forward_matches_dense_bruteforce(seed, ratio):
    dtype = "bf16" if seed % 2 else "f32"
    args = _tiny_forward_case(seed, dtype, ratio)
    res = oracle.csa_forward(dtype=dtype, **args)
    mode = {oracle.NO_COMPRESS: 0, oracle.COMPRESSOR_ONLY: 1, oracle.INDEXER: 2}[res["mode"]]
    ref = dense_forward(mode=mode, round_cmp=_torch_round(dtype), **args)
    np.testing.assert_allclose(res["out"], ref["out"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(res["lse"], ref["lse"], rtol=1e-11, atol=1e-12)
    if mode == 2:
        T = ref["sel"].shape[0]
        for i in range(T):
            got = sorted(int(c) for c in res["topk_idx"][i] if c >= 0)
            assert got == np.nonzero(ref["sel"][i])[0].tolist()


def test_forward_packing_equals_separate_segments():
    args = _tiny_forward_case(11, "bf16")
    cu = args["cu_seqlens_kv"]
    full = oracle.csa_forward(dtype="bf16", **args)
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        one = dict(args)
        for k in ("q", "ori_kv", "q_I", "k_I", "w"):
            one[k] = args[k][s:e]
        one["cu_seqlens_q"] = one["cu_seqlens_kv"] = np.array([0, e - s])
        sep = oracle.csa_forward(dtype="bf16", **one)
        np.testing.assert_array_equal(full["out"][s:e], sep["out"])
        c0 = int(full["tables"]["cu_seqlens_cmp"][b])
        fi = full["topk_idx"][s:e]
        np.testing.assert_array_equal(np.where(fi >= 0, fi - c0, -1), sep["topk_idx"])


def test_forward_cp_slice_equals_rows_of_full_run():
    rng = np.random.default_rng(12)
    L = [23, 40, 17, 31]
    cu = _cu(L)
    T = int(cu[-1])
    H, d, HI, dI = 2, 8, 2, 4
    full_args = dict(q=rng.standard_normal((T, H, d)), ori_kv=rng.standard_normal((T, d)),
                     q_I=rng.standard_normal((T, HI, dI)), k_I=rng.standard_normal((T, dI)),
                     w=rng.standard_normal((T, HI)), sinks=rng.standard_normal(H),
                     cu_seqlens_q=cu, cu_seqlens_kv=cu, global_start=0, cmp_ratio=4,
                     ori_win_left=6, ori_win_right=0, topk=3, softmax_scale=0.3)
    a, b = 30, 75                          # both cuts fall inside segments
    kv_end = b
    full_args_prefix = dict(full_args)
    nb = int(np.searchsorted(cu, kv_end, side="left"))
    cu_kv = np.minimum(cu[:nb + 1], kv_end)
    for k in ("q", "ori_kv", "q_I", "k_I", "w"):
        full_args_prefix[k] = full_args[k][:kv_end]
    full_args_prefix["cu_seqlens_q"] = full_args_prefix["cu_seqlens_kv"] = cu_kv
    full = oracle.csa_forward(dtype="f32", **full_args_prefix)
    sl = dict(full_args_prefix)
    sl["q"], sl["q_I"], sl["w"] = full_args["q"][a:b], full_args["q_I"][a:b], full_args["w"][a:b]
    sl["cu_seqlens_q"] = np.clip(cu_kv - a, 0, b - a)
    sl["global_start"] = a
    part = oracle.csa_forward(dtype="f32", **sl)
    np.testing.assert_array_equal(part["out"], full["out"][a:b])
    np.testing.assert_array_equal(part["topk_idx"], full["topk_idx"][a:b])
    for k in ("q_pos", "win_idx", "q_cmp_lo", "q_cmp_nvis", "q_seg"):
        np.testing.assert_array_equal(part["tables"][k], full["tables"][k][a:b])


def test_layer_compress_mode():
    assert oracle.layer_compress_mode(4) == oracle.INDEXER
    assert oracle.layer_compress_mode(128) == oracle.COMPRESSOR_ONLY
    assert oracle.layer_compress_mode(1) == oracle.NO_COMPRESS
    assert oracle.layer_compress_mode(4, 0) == oracle.NO_COMPRESS


def test_tiny_workload_runs_end_to_end():
    p = make_pack("tiny")
    res = oracle.csa_forward(q=p.q, ori_kv=p.ori_kv, q_I=p.q_I, k_I=p.k_I, w=p.w, sinks=p.sinks,
                             cu_seqlens_q=p.cu_seqlens_q, cu_seqlens_kv=p.cu_seqlens_kv,
                             global_start=0, cmp_ratio=4, ori_win_left=15, ori_win_right=0,
                             topk=8, softmax_scale=p.softmax_scale, dtype="f32")
    assert res["out"].shape == (128, 4, 64) and np.isfinite(res["out"]).all()
    assert int(res["tables"]["cu_seqlens_cmp"][-1]) == 31
