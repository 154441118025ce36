"""CPU checks of host-side logic around the library.

* the seeded workload recipes (segment lengths of the named packs) hold the
  structure their descriptions state;
* the bench's algorithmic-work accounting, the numerator of its roofline figure,
  equals a brute-force count over every (query, stream row) pair;
* the bench keeps its one-GPU contract: asked for several GPUs it exits with a
  message before touching a device.
"""
from __future__ import annotations

import os
import subprocess
import sys
import types

import numpy as np
import pytest

import oracle
from synth import packs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_pack16k_length_recipe(seed):
    L = packs._lengths_pack16k(np.random.default_rng(seed))
    assert sum(L) == 16384
    assert all(17 <= n <= 8192 for n in L)
    assert all(n % 4 != 0 for n in L), "every segment leaves a tail that forms no compressed row"
    assert len(L) >= 2


def test_pack16k_seed0_has_twelve_segments():
    assert len(packs._lengths_pack16k(np.random.default_rng(0))) == 12


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_hca32k_length_recipe(seed):
    L = packs._lengths_hca32k(np.random.default_rng(seed))
    assert len(L) == 8 and sum(L) == 32768
    assert all(1024 <= n <= 7000 for n in L)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_cp_length_recipe_straddles_the_cuts(seed):
    L = packs._lengths_cp(np.random.default_rng(seed))
    assert sum(L) == 131072 and min(L) >= 1
    bounds = set(np.cumsum(L)[:-1].tolist())
    assert 65536 not in bounds and 98304 not in bounds, "each share boundary falls inside a segment"


def test_query_slice_layout():
    """A query slice [a, b) of a stream with the KV prefix cut at kv_end: local query
    counts per segment, KV truncated at the prefix end, stream-absolute start."""
    p = packs.pack_from_lengths("slice", [50, 70, 40, 90], seed=1, H=2, d=8, H_I=2, d_I=8, q_rows=(60, 150),
                                kv_rows=170)
    assert p.global_start == 60 and p.Tq == 90 and p.Tkv == 170
    assert p.cu_seqlens_kv.tolist() == [0, 50, 120, 160, 170]
    assert p.cu_seqlens_q.tolist() == [0, 0, 60, 90, 90]
    assert p.q.shape == (90, 2, 8) and p.ori_kv.shape == (170, 8)


def _bench_module():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def _fake_plan(pack_like, tabs, topk, with_indexer=True):
    torch = pytest.importorskip("torch")
    nvis = np.asarray(tabs["q_cmp_nvis"], dtype=np.int64)
    Tq = len(nvis)
    idx = np.full((Tq, topk), -1, dtype=np.int64)
    for i in range(Tq):
        k = min(int(nvis[i]), topk)
        idx[i, :k] = np.arange(k)          # the count of valid entries is what is accounted
    return types.SimpleNamespace(
        q_pos=torch.from_numpy(np.asarray(tabs["q_pos"], dtype=np.int64)),
        q_seg=torch.from_numpy(np.asarray(tabs["q_seg"], dtype=np.int64)),
        q_cmp_nvis=torch.from_numpy(nvis),
        topk_idx=torch.from_numpy(idx) if with_indexer else None,
        cmp_kv=object(),
        L=types.SimpleNamespace(cu_seqlens_kv=torch.from_numpy(np.asarray(pack_like.cu_seqlens_kv, dtype=np.int64))))


@pytest.mark.parametrize("with_indexer", [True, False])
@pytest.mark.parametrize("wl,wr,gs,q_rows", [(15, 0, 0, None), (7, 3, 0, None), (15, 0, 60, (60, 150))])
def test_bench_work_accounting_matches_brute_force(with_indexer, wl, wr, gs, q_rows):
    bench = _bench_module()
    lengths = [50, 70, 40, 90]
    topk = 6
    p = packs.pack_from_lengths("acct", lengths, seed=2, H=2, d=8, H_I=2, d_I=8, ori_win_left=wl, ori_win_right=wr,
                                topk=topk, q_rows=q_rows, kv_rows=170 if q_rows else None)
    tabs = oracle.build_indices(p.cu_seqlens_q, p.cu_seqlens_kv, p.global_start, p.Tq, 4, wl, wr)
    plan = _fake_plan(p, tabs, topk, with_indexer)
    nwin, ncmp, need = bench.algorithmic_work(plan, p)
    # brute force: every stream row of the query's own segment within [t - wl, t + wr]
    cu = np.asarray(p.cu_seqlens_kv, dtype=np.int64)
    seg_of = np.repeat(np.arange(len(cu) - 1), np.diff(cu))
    want_win = 0
    for i in range(p.Tq):
        t = p.global_start + i
        want_win += sum(1 for k in range(p.Tkv) if seg_of[k] == seg_of[t] and t - wl <= k <= t + wr)
    nvis = np.asarray(tabs["q_cmp_nvis"], dtype=np.int64)
    assert nwin == want_win
    if with_indexer:
        assert ncmp == int(np.minimum(nvis, topk).sum())
        assert need == int(nvis[nvis > topk].sum())
    else:
        assert ncmp == int(nvis.sum()) and need == 0


@pytest.mark.parametrize("n", ["2", "8"])
def test_bench_refuses_several_gpus(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
