"""GPU checks of the indexer's top-k selection where the set is unique to the bit.

The inputs are small integers held exactly in bf16: every head of q_I is one integer
repeated over d_I, every compressed key row one integer v_c repeated, the head weights
integers.  Each logit is then 128 a v_c and each score an integer below 2^24, which
float32 (in any summation order) and the oracle's float64 both hold exactly.  The
oracle's rule (top-k by score, exact ties to the lower row, kept rows ascending; page
"【RFC】DeepSeek-V4 CSA/HCA ...", 1. npu_lightning_indexer) then fixes every row, and
the GPU rows and scores must equal the oracle's exactly.

The cases drive each branch of the selection: every score equal (one key), zero
weights (every score 0), heavy exact ties, one outlier far above scores that take two
values (the threshold bin then holds most candidates, more than the per-wavefront
list), negative weights (every score <= 0), and a wide integer spread.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

H_I, D_I, R = 64, 128, 4
LENGTHS = [8003, 1501, 37, 4]     # 2000, 375, 9 and 1 compressed rows
CASES = ["equal", "zero_w", "ties", "outlier", "negative", "spread"]


def _case(name, Tc, Tq, rng):
    v = np.zeros(Tc, np.int64)
    a = np.ones((Tq, H_I), np.int64)
    w = np.ones((Tq, H_I), np.int64)
    if name == "equal":
        v[:] = 3
    elif name == "zero_w":
        v[:] = rng.integers(-8, 9, Tc)
        w[:] = 0
    elif name == "ties":
        v[:] = rng.integers(0, 8, Tc)
        a[:] = rng.choice([-1, 1], (Tq, H_I))
        w[:] = rng.integers(0, 3, (Tq, H_I))
    elif name == "outlier":
        v[:] = rng.integers(1, 3, Tc)
        v[rng.integers(0, Tc, 3)] = 64
    elif name == "negative":
        v[:] = rng.integers(1, 41, Tc)
        w[:] = rng.integers(-2, 0, (Tq, H_I))
    elif name == "spread":
        v[:] = rng.integers(-64, 65, Tc)
        a[:] = rng.choice([-2, -1, 1, 2], (Tq, H_I))
        w[:] = rng.integers(0, 5, (Tq, H_I))
    else:
        raise KeyError(name)
    return a, w.astype(np.float32), v


class _Rows:
    """q_I[i] = a[i] repeated over d_I, built row by row for the oracle."""

    def __init__(self, a):
        self.a = a

    def __getitem__(self, i):
        return np.repeat(self.a[i][:, None].astype(np.float64), D_I, axis=1)


def _bf16(x):
    bits = f32_to_bf16_bits(np.ascontiguousarray(x, np.float32))
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("topk", [512, 64])
@pytest.mark.parametrize("name", CASES)
def test_selection_is_exact_on_integer_scores(name, topk):
    import sparse_attention_thd_amd as s
    cu = np.concatenate([[0], np.cumsum(LENGTHS)]).astype(np.int32)
    Tq = int(cu[-1])
    tabs = oracle.build_indices(cu, cu, 0, Tq, R, 127, 0)
    cu_cmp = tabs["cu_seqlens_cmp"].astype(np.int32)
    Tc = int(cu_cmp[-1])
    rng = np.random.default_rng([CASES.index(name), topk])
    a, w, v = _case(name, Tc, Tq, rng)
    k = np.repeat(v[:, None], D_I, axis=1).astype(np.float32)       # [Tc, D_I]
    print(f"[case] {name} topk={topk}: Tq={Tq} Tc={Tc} -> csa_indexer_topk", flush=True)
    max_kv = int(np.diff(cu).max())
    idx = torch.empty((Tq, topk), dtype=torch.int32, device="cuda")
    sc = torch.empty((Tq, topk), dtype=torch.float32, device="cuda")
    ws = torch.empty(s.csa_indexer_topk_workspace_bytes(Tq, max_kv, R), dtype=torch.uint8, device="cuda")
    dcu = torch.from_numpy(cu).cuda()
    q_dev = _bf16(a.astype(np.float32))[:, :, None].expand(Tq, H_I, D_I).contiguous()  # integers: exact in bf16
    s.csa_indexer_topk(q_dev, _bf16(w), _bf16(k), Tq, Tc, H_I, D_I, dcu, dcu, torch.from_numpy(cu_cmp).cuda(), None,
                       len(LENGTHS), 0, R, max_kv, topk, idx, topk_score=sc, workspace=ws)
    torch.cuda.synchronize()
    ref_idx, ref_sc = oracle.indexer_topk(_Rows(a), w, k, tabs, topk)
    got_idx = idx.cpu().numpy().astype(np.int64)
    got_sc = sc.cpu().numpy().astype(np.float64)
    bad = np.nonzero((got_idx != ref_idx).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first query {bad[0]}: got {got_idx[bad[0]][:8]} ref {ref_idx[bad[0]][:8]}"
    valid = ref_idx >= 0
    np.testing.assert_array_equal(got_sc[valid], ref_sc[valid])
    assert np.all(np.isneginf(got_sc[~valid]))
    sel = int((tabs["q_cmp_nvis"] > topk).sum())
    print(f"    {sel} of {Tq} queries selected; rows and scores exact", flush=True)


def _random_draw(seed):
    """Layout and top-k of one seed."""
    rng = np.random.default_rng(47000 + seed)
    nseg = int(rng.integers(1, 5))
    lengths = []
    for _ in range(nseg):
        kind = rng.random()
        lengths.append(int(rng.integers(1, 41)) if kind < 0.3 else
                       int(rng.integers(100, 3001)) if kind < 0.75 else int(rng.integers(4000, 9001)))
    topk = int(rng.choice([1, 7, 64, 512, 1024, 2048]))
    return rng, lengths, topk


def _random_values(rng, Tc, Tq):
    """Integer query signs, head weights and key values (scores stay exact in float32)."""
    vmax = int(rng.choice([1, 2, 8, 64]))
    v = rng.integers(-vmax if rng.random() < 0.5 else 0, vmax + 1, Tc)
    if rng.random() < 0.3 and Tc > 0:
        v[rng.integers(0, Tc, int(rng.integers(1, 6)))] = 64
    a = rng.choice([[1], [-1, 1], [-2, -1, 1, 2], [0, 1]][int(rng.integers(0, 4))], (Tq, H_I))
    wlo, whi = [(1, 2), (0, 3), (-2, 0), (-4, 5), (0, 1)][int(rng.integers(0, 5))]
    w = rng.integers(wlo, whi, (Tq, H_I))
    return a, w.astype(np.float32), v


@pytest.mark.parametrize("seed", list(range(8)))
def test_selection_is_exact_on_random_layouts(seed):
    """Seeded random layouts (1-4 segments of 1 to 9000 tokens, top-k 1 to 2048) with random
    integer distributions: key ranges, signed or not, query signs, zero / negative / mixed
    head weights, planted outliers; rows and scores exact as above."""
    import sparse_attention_thd_amd as s
    rng, lengths, topk = _random_draw(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    Tq = int(cu[-1])
    tabs = oracle.build_indices(cu, cu, 0, Tq, R, 127, 0)
    cu_cmp = tabs["cu_seqlens_cmp"].astype(np.int32)
    Tc = int(cu_cmp[-1])
    a, w, v = _random_values(rng, Tc, Tq)
    k = np.repeat(v[:, None], D_I, axis=1).astype(np.float32)
    print(f"[case] select random{seed}: lengths={lengths} topk={topk} Tc={Tc}", flush=True)
    max_kv = int(np.diff(cu).max())
    idx = torch.empty((Tq, topk), dtype=torch.int32, device="cuda")
    sc = torch.empty((Tq, topk), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(s.csa_indexer_topk_workspace_bytes(Tq, max_kv, R), 1), dtype=torch.uint8, device="cuda")
    dcu = torch.from_numpy(cu).cuda()
    q_dev = _bf16(a.astype(np.float32))[:, :, None].expand(Tq, H_I, D_I).contiguous()
    k_dev = _bf16(k) if Tc > 0 else _bf16(np.zeros((1, D_I), np.float32))
    s.csa_indexer_topk(q_dev, _bf16(w), k_dev, Tq, Tc, H_I, D_I, dcu, dcu, torch.from_numpy(cu_cmp).cuda(), None,
                       len(lengths), 0, R, max_kv, topk, idx, topk_score=sc, workspace=ws)
    torch.cuda.synchronize()
    ref_idx, ref_sc = oracle.indexer_topk(_Rows(a), w, k, tabs, topk)
    got_idx = idx.cpu().numpy().astype(np.int64)
    got_sc = sc.cpu().numpy().astype(np.float64)
    bad = np.nonzero((got_idx != ref_idx).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first query {bad[0]}"
    valid = ref_idx >= 0
    np.testing.assert_array_equal(got_sc[valid], ref_sc[valid])
    assert np.all(np.isneginf(got_sc[~valid]))
