"""GPU parity of the indexer KL-loss gradient (csa_indexer_kl_grad) against the fp64 oracle.

The GPU forward supplies the compressed indexer keys and the top-k lists; the targets
are seeded positive values at the selected slots (any target is a valid input), and one
case feeds the sparse-MLA backward's cmp_l1 through, as training does.

Tolerances (from the arithmetic): scores and the softmax are float32 (relative
~1e-6); M = G w [u > 0] enters the d_q and d_k products rounded to bf16 (u = 2^-9),
so d_q, d_k carry relative L2 errors of a few u: rel-L2 <= 1e-2, max <= 3e-2 max|ref|.
d_w and the loss stay float32: rel-L2 <= 1e-3 and |loss diff| <= 1e-4 (1 + loss).
A score within 1e-3 of the ReLU kink may take the other side on the GPU (float32
against float64): such (query, head) rows are left out of d_q's max-norm check, as a
tie band (their effect on the sums stays inside the rel-L2 bound).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_support import cpu, host_view, oracle_tables, run_pack, to_device
from synth import make_pack, pack_from_lengths

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

REL_L2 = 1e-2
REL_INF = 3e-2
DW_REL_L2 = 1e-3
KINK = 1e-3


def _pack(name):
    if name == "select16":
        return pack_from_lengths("select16", [600, 300, 1201], seed=4, topk=16)
    if name == "long":
        return pack_from_lengths("long", [2500, 37], seed=5, topk=64)
    if name == "edges":
        return pack_from_lengths("edges", [1, 3, 4, 5, 130, 257, 700], seed=3)
    if name == "many_segs":
        return pack_from_lengths("many_segs", [5 + (37 * k) % 120 for k in range(80)], seed=13, topk=32)
    if name == "cp_small":
        return pack_from_lengths("cp_small", [700, 1500, 900, 400], seed=8, q_rows=(1000, 2600), kv_rows=2600,
                                 topk=32)
    if name == "topk1024":  # the top-k > 512 instance (up to 650 kept rows per query)
        return pack_from_lengths("topk1024", [2600, 150], seed=23, topk=1024)
    if name == "max_limits":  # the largest candidate list (32768) and top-k (2048) the calls accept
        return pack_from_lengths("max_limits", [131072], seed=25, topk=2048, q_rows=(131072 - 48, 131072))
    raise KeyError(name)


def _targets(plan, seed):
    rng = np.random.default_rng(seed)
    idx = cpu(plan.topk_idx)
    p = rng.random(idx.shape).astype(np.float32) * (idx >= 0)
    return p


def _run_kl(pack, plan, p, loss_scale):
    import sparse_attention_thd_amd as s
    L = plan.L
    T = pack.Tq
    Tc = plan.k_I_cmp.shape[0]
    nb = s.csa_indexer_kl_grad_workspace_bytes(T, pack.topk, pack.max_seqlen_kv, pack.cmp_ratio)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    d_q = torch.empty((T, pack.H_I, pack.d_I), dtype=torch.bfloat16, device="cuda")
    d_w = torch.empty((T, pack.H_I), dtype=torch.float32, device="cuda")
    d_k = torch.empty((Tc, pack.d_I), dtype=torch.float32, device="cuda")
    loss = torch.empty(T, dtype=torch.float32, device="cuda")
    pt = torch.from_numpy(np.ascontiguousarray(p, dtype=np.float32)).cuda()
    print(f"[case] {pack.name}: csa_indexer_kl_grad Tq={T} Tc={Tc} topk={pack.topk} workspace={nb / 2**20:.1f} MiB",
          flush=True)
    s.csa_indexer_kl_grad(to_device(pack.q_I), to_device(pack.w), plan.k_I_cmp, plan.topk_idx, pt, pack.topk, T, Tc,
                          pack.H_I, pack.d_I, L.cu_seqlens_q, L.cu_seqlens_kv, plan.cu_seqlens_cmp, L.B,
                          L.global_start, pack.cmp_ratio, pack.max_seqlen_kv, loss_scale, d_q, d_w, d_k, loss, ws)
    torch.cuda.synchronize()
    return dict(d_q=cpu(d_q), d_w=cpu(d_w), d_k=cpu(d_k), loss=cpu(loss))


def _kink_rows(pack, plan, queries):
    """(query position, head) pairs with a selected row whose score is within KINK of 0."""
    qI = host_view(pack, "q_I")
    kc = cpu(plan.k_I_cmp).astype(np.float64)
    idx = cpu(plan.topk_idx)
    bad = []
    for n, i in enumerate(queries):
        rows = idx[i][idx[i] >= 0]
        if len(rows):
            u = np.asarray(qI[i], dtype=np.float64) @ kc[rows].T
            for h in np.nonzero((np.abs(u) < KINK).any(axis=1))[0]:
                bad.append((n, int(h)))
    return bad


def _rel(got, ref, what, bound=REL_L2, inf=REL_INF, skip=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(got - ref)
    l2 = float(np.linalg.norm(diff)) / max(float(np.linalg.norm(ref)), 1e-300)
    if skip:
        diff = diff.copy()
        for n, h in skip:
            diff[n, h] = 0.0
    rinf = float(np.abs(ref).max()) if ref.size else 0.0
    msg = f"{what}: max|d|={float(diff.max()) if diff.size else 0:.3e} |ref|inf={rinf:.3e} relL2={l2:.3e}"
    print("   ", msg, flush=True)
    if ref.size and rinf > 0:
        assert l2 <= bound, msg
        if inf is not None:
            assert float(diff.max()) <= inf * rinf, msg


def _check(pack, plan, p, scale, queries=None):
    got = _run_kl(pack, plan, p, scale)
    tabs = oracle_tables(pack)
    idx = cpu(plan.topk_idx)
    kc = cpu(plan.k_I_cmp)[:int(tabs["cu_seqlens_cmp"][-1])]
    qs = list(range(pack.Tq)) if queries is None else list(queries)
    ref = oracle.indexer_kl_grad(host_view(pack, "q_I"), host_view(pack, "w"), kc, idx, p, tabs, scale,
                                 queries=None if queries is None else qs)
    skip = _kink_rows(pack, plan, qs)
    _rel(got["d_q"][qs], ref["d_q"], "d_q", skip=skip)
    _rel(got["d_w"][qs], ref["d_w"], "d_w", bound=DW_REL_L2)
    lossd = np.abs(got["loss"][qs] - ref["loss"])
    assert (lossd <= 1e-4 * (1 + np.abs(ref["loss"]))).all(), f"loss: max diff {lossd.max():.3e}"
    if queries is None:
        tc = ref["d_k"].shape[0]
        _rel(got["d_k"][:tc], ref["d_k"], "d_k")
        assert not np.any(got["d_k"][tc:]), "rows past the compressed count stay zero"
    return got


@pytest.mark.parametrize("name", ["select16", "long", "edges", "many_segs", "cp_small", "topk1024", "max_limits"])
def test_kl_grad_matches_oracle(name):
    pack = _pack(name)
    print(f"\n[case] {name}: Tq={pack.Tq} -> forward on GPU", flush=True)
    plan = run_pack(pack)
    _check(pack, plan, _targets(plan, 200), 1.0 / pack.Tq)


@pytest.mark.parametrize("name", ["select16", "long", "cp_small"])
def test_kl_grad_unordered_rows_and_holes(name):
    """Index rows in any order and with holes (-1) between entries: every third query's
    row shuffled, every third a hole punched, the rest as the indexer wrote them (sorted),
    so neighbouring queries pair sorted with sorted, sorted with unordered and unordered
    with unordered lists."""
    pack = _pack(name)
    print(f"\n[case] {name} (unordered rows, holes): Tq={pack.Tq} -> forward on GPU", flush=True)
    plan = run_pack(pack)
    idx = cpu(plan.topk_idx).copy()
    rng = np.random.default_rng(17)
    for i in range(idx.shape[0]):
        if i % 3 == 0:
            rng.shuffle(idx[i])
        elif i % 3 == 1:
            idx[i, rng.integers(0, idx.shape[1])] = -1
    plan.topk_idx = torch.from_numpy(idx).cuda()
    _check(pack, plan, _targets(plan, 202), 1.0 / pack.Tq)


def test_kl_grad_with_backward_targets():
    """The sparse-MLA backward's cmp_l1 (head-averaged probabilities) as the target."""
    import sparse_attention_thd_amd as s
    pack = _pack("select16")
    plan = run_pack(pack)
    L = plan.L
    T, H, d = pack.Tq, pack.H, pack.d
    dout = torch.from_numpy(np.random.default_rng(3).standard_normal((T, H, d)).astype(np.float32)).to(
        torch.bfloat16).cuda()
    Tc = plan.cmp_kv.shape[0]
    nb = s.csa_sparse_mla_bwd_workspace_bytes(T, pack.ori_win_left, pack.ori_win_right, plan.cmp_kv, plan.topk_idx,
                                              pack.topk, pack.max_seqlen_kv, pack.cmp_ratio)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dq = torch.empty_like(plan.out)
    d_ori = torch.empty((L.Tkv, d), dtype=torch.float32, device="cuda")
    d_cmp = torch.empty((Tc, d), dtype=torch.float32, device="cuda")
    d_s = torch.empty(H, dtype=torch.float32, device="cuda")
    ol1 = torch.empty((T, pack.ori_win_left + pack.ori_win_right + 1), dtype=torch.float32, device="cuda")
    cl1 = torch.empty((T, pack.topk), dtype=torch.float32, device="cuda")
    s.csa_sparse_mla_bwd(to_device(pack.q), to_device(pack.ori_kv), plan.cmp_kv, plan.topk_idx, pack.topk, T, L.Tkv,
                         Tc, H, d, L.cu_seqlens_q, L.cu_seqlens_kv, plan.cu_seqlens_cmp, L.B, L.global_start,
                         pack.cmp_ratio, pack.ori_win_left, pack.ori_win_right, pack.max_seqlen_kv,
                         to_device(pack.sinks), pack.softmax_scale, plan.out, plan.lse, dout, dq, d_ori, d_cmp, d_s,
                         ol1, cl1, pack.topk, ws)
    torch.cuda.synchronize()
    _check(pack, plan, cpu(cl1), 0.5 / pack.Tq)


def test_kl_grad_zero_scale_and_determinism():
    pack = _pack("many_segs")
    plan = run_pack(pack)
    p = _targets(plan, 5)
    a = _run_kl(pack, plan, p, 0.0)
    assert not a["d_q"].any() and not a["d_w"].any() and not a["d_k"].any()
    b1 = _run_kl(pack, plan, p, 1e-3)
    b2 = _run_kl(pack, plan, p, 1e-3)
    assert np.array_equal(b1["d_q"], b2["d_q"]) and np.array_equal(b1["d_w"], b2["d_w"])
    assert np.array_equal(b1["loss"], b2["loss"])


def test_kl_grad_pack16k_every_query():
    """Full-size pack: d_q, d_w and the loss of every query, d_k summed over all of them."""
    pack = make_pack("pack16k")
    print(f"\n[case] pack16k: Tq={pack.Tq} -> forward on GPU", flush=True)
    plan = run_pack(pack)
    _check(pack, plan, _targets(plan, 201), 1.0 / pack.Tq)


def test_kl_grad_empty_query_slice():
    """Tq = 0 (a CP share past every query): d_k is still overwritten with zeros."""
    import sparse_attention_thd_amd as s
    print("[case] Tq = 0 -> csa_indexer_kl_grad", flush=True)
    i32 = dict(dtype=torch.int32, device="cuda")
    cu_q, cu_kv, cu_cmp = (torch.tensor(v, **i32) for v in ([0, 0], [0, 64], [0, 16]))
    bf = dict(dtype=torch.bfloat16, device="cuda")
    k = torch.randn((16, 128), **bf)
    d_k = torch.full((16, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(1, dtype=torch.uint8, device="cuda")
    s.csa_indexer_kl_grad(torch.empty((0, 64, 128), **bf), torch.empty((0, 64), **bf), k,
                          torch.empty((0, 512), **i32), torch.empty((0, 512), dtype=torch.float32, device="cuda"),
                          512, 0, 16, 64, 128, cu_q, cu_kv, cu_cmp, 1, 64, 4, 64, 1.0,
                          torch.empty((0, 64, 128), **bf), torch.empty((0, 64), dtype=torch.float32, device="cuda"),
                          d_k, None, ws)
    torch.cuda.synchronize()
    assert not d_k.isnan().any() and not d_k.any()
