"""GPU parity of the sparse-MLA backward (csa_sparse_mla_bwd) against the fp64 oracle.

The forward runs on the GPU first (its out, lse, compressed rows and top-k lists feed
the backward, as in training); a seeded bf16 dout drives both sides.  Every pack, the 16k one included, compares
every output: dq and the head-averaged probabilities of every query, and the row
and sink gradients (sums over all queries).

Tolerances (derived from the arithmetic): P and scale * dS enter the MFMA products
rounded to bf16 (unit roundoff u = 2^-9), and D = dout . out uses the forward's bf16
output, so every gradient term carries a relative error <= u.  Sums of such terms
with moderate cancellation give a relative L2 error of a few u; the bounds are
rel-L2 <= 1e-2 and max|diff| <= 3e-2 * max|ref| per gradient tensor, and 2e-4
absolute for the probabilities (float32 exp of float32 logits).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle
from gpu_support import cpu, host_view, oracle_tables, run_pack, to_device
from synth import make_pack, pack_from_lengths

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GRAD_REL_L2 = 1e-2
GRAD_REL_INF = 3e-2
L1_ABS = 2e-4


def _small(name):
    if name == "select16":
        return pack_from_lengths("select16", [600, 300, 1201], seed=4, topk=16)
    if name == "edges":
        return pack_from_lengths("edges", [1, 3, 4, 5, 130, 257, 700], seed=3)
    if name == "long":
        return pack_from_lengths("long", [2500, 37], seed=5, topk=64)
    if name == "short_only":
        return pack_from_lengths("short_only", [1, 2, 3, 1], seed=6)
    if name == "hca_small":
        return pack_from_lengths("hca_small", [300, 701, 130], seed=7, cmp_ratio=128, indexer=False)
    if name == "cp_small":
        return pack_from_lengths("cp_small", [700, 1500, 900, 400], seed=8, q_rows=(1000, 2600), kv_rows=2600,
                                 topk=32)
    if name == "win_right":
        return pack_from_lengths("win_right", [300, 411], seed=9, ori_win_left=20, ori_win_right=5, topk=32)
    if name == "no_compress":
        return pack_from_lengths("no_compress", [200, 333], seed=10, cmp_ratio=1, indexer=False)
    if name == "ratio5":  # every visible compressed row attended, a ratio that is not a power of two
        return pack_from_lengths("ratio5", [17, 999, 4, 260], seed=28, cmp_ratio=5, indexer=False)
    if name == "many_segs":
        return pack_from_lengths("many_segs", [5 + (37 * k) % 120 for k in range(80)], seed=13, topk=32)
    if name == "stress_small":  # peaky softmax (q, kv ~ N(0,1))
        return pack_from_lengths("stress_small", [900], seed=14, topk=32, q_scale=1.0, kv_scale=1.0)
    if name == "topk1024":  # the top-k > 512 instances (up to 650 kept rows per query)
        return pack_from_lengths("topk1024", [2600, 150], seed=23, topk=1024)
    if name == "max_limits":  # the largest candidate list (32768) and top-k (2048) the calls accept
        return pack_from_lengths("max_limits", [131072], seed=25, topk=2048, q_rows=(131072 - 48, 131072))
    if name == "no_sinks":
        return dataclasses.replace(pack_from_lengths("no_sinks", [400, 90], seed=15, topk=32), sinks=None)
    raise KeyError(name)


def _run_bwd(pack, plan, seed, deterministic=False):
    """csa_sparse_mla_bwd (or its deterministic form) on the forward's results; returns host
    copies, the dout used, whether the layer attends to every visible compressed row, and
    the slot count."""
    import sparse_attention_thd_amd as s
    rng = np.random.default_rng(seed)
    T, H, d = pack.Tq, pack.H, pack.d
    dout = torch.from_numpy(rng.standard_normal((T, H, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    L = plan.L
    cmp_kv, cmp_idx = plan.cmp_kv, plan.topk_idx
    attend_all = cmp_kv is not None and cmp_idx is None
    topk = pack.topk if cmp_idx is not None else 0
    W = pack.ori_win_left + pack.ori_win_right + 1
    slots = topk if cmp_idx is not None else (max(1, pack.max_seqlen_kv // pack.cmp_ratio) if attend_all else 0)
    Tc = 0 if cmp_kv is None else cmp_kv.shape[0]
    if deterministic:
        nbytes = s.csa_sparse_mla_bwd_deterministic_workspace_bytes(T, L.B, pack.ori_win_left, pack.ori_win_right,
                                                                    cmp_kv, cmp_idx, topk, pack.max_seqlen_kv,
                                                                    pack.cmp_ratio)
    else:
        nbytes = s.csa_sparse_mla_bwd_workspace_bytes(T, pack.ori_win_left, pack.ori_win_right, cmp_kv, cmp_idx,
                                                      topk, pack.max_seqlen_kv, pack.cmp_ratio)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    dq = torch.empty_like(plan.out)
    d_ori = torch.empty((L.Tkv, d), dtype=torch.float32, device="cuda")
    d_cmp = torch.empty((Tc, d), dtype=torch.float32, device="cuda") if cmp_kv is not None else None
    d_sinks = torch.empty(H, dtype=torch.float32, device="cuda") if pack.sinks is not None else None
    ori_l1 = torch.empty((T, W), dtype=torch.float32, device="cuda")
    cmp_l1 = torch.empty((T, slots), dtype=torch.float32, device="cuda") if slots else None
    call = s.csa_sparse_mla_bwd_deterministic if deterministic else s.csa_sparse_mla_bwd
    print(f"[case] {pack.name}: {call.__name__} Tq={T} Tc={Tc} topk={topk} attend_all={attend_all} "
          f"workspace={nbytes / 2**20:.1f} MiB", flush=True)
    call(to_device(pack.q), to_device(pack.ori_kv), cmp_kv, cmp_idx, topk, T, L.Tkv, Tc, H, d,
         L.cu_seqlens_q, L.cu_seqlens_kv, plan.cu_seqlens_cmp if cmp_kv is not None else None, L.B,
         L.global_start, pack.cmp_ratio, pack.ori_win_left, pack.ori_win_right, pack.max_seqlen_kv,
         to_device(pack.sinks), pack.softmax_scale, plan.out, plan.lse, dout, dq, d_ori, d_cmp,
         d_sinks, ori_l1, cmp_l1, slots, ws)
    torch.cuda.synchronize()
    got = dict(dq=cpu(dq), d_ori_kv=cpu(d_ori), d_cmp_kv=cpu(d_cmp), d_sinks=cpu(d_sinks), ori_l1=cpu(ori_l1),
               cmp_l1=cpu(cmp_l1))
    return got, cpu(dout), attend_all, slots


def _close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(got - ref)
    rinf = float(np.abs(ref).max()) if ref.size else 0.0
    l2 = float(np.linalg.norm(diff)) / max(float(np.linalg.norm(ref)), 1e-300)
    msg = f"{what}: max|d|={float(diff.max()) if diff.size else 0:.3e} |ref|inf={rinf:.3e} relL2={l2:.3e}"
    print("   ", msg, flush=True)
    if ref.size and rinf > 0:
        assert l2 <= GRAD_REL_L2, msg
        assert float(diff.max()) <= GRAD_REL_INF * rinf, msg


def _oracle(pack, tabs, plan, dout, attend_all, slots, queries=None):
    """The oracle backward on the GPU forward's compressed rows (the actual count) and top-k lists."""
    cmp_kv = None
    if plan.cmp_kv is not None:
        cmp_kv = cpu(plan.cmp_kv)[:int(tabs["cu_seqlens_cmp"][-1])]
    rows = cpu(plan.topk_idx) if plan.topk_idx is not None else None
    if rows is not None and queries is not None:
        rows = {i: rows[i] for i in queries}
    dsel = dout if queries is None else dout[queries]
    return oracle.sparse_mla_bwd(host_view(pack, "q"), host_view(pack, "ori_kv"), cmp_kv, rows, tabs, pack.sinks,
                                 pack.softmax_scale, pack.ori_win_left, pack.ori_win_right, pack.cu_seqlens_kv,
                                 pack.global_start, dsel, cmp_slots=slots, attend_all_visible=attend_all,
                                 queries=queries)


SMALL = ["select16", "edges", "long", "short_only", "hca_small", "ratio5", "cp_small", "win_right", "no_compress",
         "many_segs", "stress_small", "no_sinks", "topk1024", "max_limits"]


@pytest.mark.parametrize("name", SMALL)
def test_backward_matches_oracle(name):
    pack = _small(name)
    print(f"\n[case] {name}: Tq={pack.Tq} Tkv={pack.Tkv} -> forward on GPU", flush=True)
    plan = run_pack(pack)
    got, dout, attend_all, slots = _run_bwd(pack, plan, seed=100)
    tabs = oracle_tables(pack)
    ref = _oracle(pack, tabs, plan, dout, attend_all, slots)
    _close(got["dq"], ref["dq"], "dq")
    _close(got["d_ori_kv"], ref["d_ori_kv"], "d_ori_kv")
    if ref["d_cmp_kv"] is not None:
        tc = ref["d_cmp_kv"].shape[0]
        _close(got["d_cmp_kv"][:tc], ref["d_cmp_kv"], "d_cmp_kv")
        assert not np.any(got["d_cmp_kv"][tc:]), "rows past the compressed count stay zero"
    if pack.sinks is not None:
        _close(got["d_sinks"], ref["d_sinks"], "d_sinks")
    assert np.abs(got["ori_l1"] - ref["ori_l1"]).max() <= L1_ABS
    if slots:
        assert np.abs(got["cmp_l1"] - ref["cmp_l1"]).max() <= L1_ABS


def test_backward_is_deterministic_except_row_sums():
    """dq and the probabilities are bit-identical across runs; the row gradients use
    float atomics, so only their values within rounding are stable."""
    pack = _small("select16")
    plan = run_pack(pack)
    a, _, _, _ = _run_bwd(pack, plan, seed=7)
    b, _, _, _ = _run_bwd(pack, plan, seed=7)
    assert np.array_equal(a["dq"], b["dq"])
    assert np.array_equal(a["ori_l1"], b["ori_l1"])
    assert np.array_equal(a["cmp_l1"], b["cmp_l1"])
    np.testing.assert_allclose(a["d_ori_kv"], b["d_ori_kv"], rtol=1e-4, atol=1e-6)


class _CloseAcc:
    """_close over a tensor compared in query chunks (same bounds, from running sums)."""

    def __init__(self, what):
        self.what, self.sq, self.ref_sq, self.mx, self.rinf = what, 0.0, 0.0, 0.0, 0.0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        diff = np.abs(got - ref)
        self.sq += float((diff * diff).sum())
        self.ref_sq += float((ref * ref).sum())
        self.mx = max(self.mx, float(diff.max()) if diff.size else 0.0)
        self.rinf = max(self.rinf, float(np.abs(ref).max()) if ref.size else 0.0)

    def check(self):
        l2 = float(np.sqrt(self.sq)) / max(float(np.sqrt(self.ref_sq)), 1e-300)
        msg = f"{self.what}: max|d|={self.mx:.3e} |ref|inf={self.rinf:.3e} relL2={l2:.3e}"
        print("   ", msg, flush=True)
        assert l2 <= GRAD_REL_L2, msg
        assert self.mx <= GRAD_REL_INF * self.rinf, msg


def test_backward_pack16k_every_query():
    """Full-size pack, every output against the oracle backward over all 16384 queries:
    dq and the probabilities query by query, the row gradients and the sink gradient as
    the sums over every query (the oracle runs in query chunks; its row gradients are
    added up across the chunks)."""
    pack = make_pack("pack16k")
    print(f"\n[case] pack16k: Tq={pack.Tq} -> forward on GPU", flush=True)
    plan = run_pack(pack)
    got, dout, attend_all, slots = _run_bwd(pack, plan, seed=101)
    tabs = oracle_tables(pack)
    dq = _CloseAcc("dq")
    d_ori = d_cmp = d_s = None
    l1_err = 0.0
    step = 2048
    for a in range(0, pack.Tq, step):
        qs = list(range(a, min(a + step, pack.Tq)))
        print(f"[case] pack16k: oracle backward, queries {a}..{qs[-1] + 1} of {pack.Tq}", flush=True)
        ref = _oracle(pack, tabs, plan, dout, attend_all, slots, queries=qs)
        dq.add(got["dq"][qs], ref["dq"])
        l1_err = max(l1_err, float(np.abs(got["ori_l1"][qs] - ref["ori_l1"]).max()),
                     float(np.abs(got["cmp_l1"][qs] - ref["cmp_l1"]).max()))
        d_ori = ref["d_ori_kv"] if d_ori is None else d_ori + ref["d_ori_kv"]
        d_cmp = ref["d_cmp_kv"] if d_cmp is None else d_cmp + ref["d_cmp_kv"]
        d_s = ref["d_sinks"] if d_s is None else d_s + ref["d_sinks"]
    dq.check()
    print(f"    probabilities: max|d|={l1_err:.3e}", flush=True)
    assert l1_err <= L1_ABS
    _close(got["d_ori_kv"], d_ori, "d_ori_kv (sum over every query)")
    tc = d_cmp.shape[0]
    _close(got["d_cmp_kv"][:tc], d_cmp, "d_cmp_kv (sum over every query)")
    _close(got["d_sinks"], d_s, "d_sinks (sum over every query)")


def test_backward_empty_query_slice():
    """Tq = 0: the row gradients and the sink gradient are overwritten with zeros."""
    import sparse_attention_thd_amd as s
    print("[case] Tq = 0 -> csa_sparse_mla_bwd", flush=True)
    i32 = dict(dtype=torch.int32, device="cuda")
    cu_q, cu_kv, cu_cmp = (torch.tensor(v, **i32) for v in ([0, 0], [0, 64], [0, 16]))
    bf = dict(dtype=torch.bfloat16, device="cuda")
    kv, ckv = torch.randn((64, 512), **bf), torch.randn((16, 512), **bf)
    nan = lambda *shape: torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    d_ori, d_cmp, d_s = nan(64, 512), nan(16, 512), nan(64)
    sinks = torch.randn(64, dtype=torch.float32, device="cuda")
    nb = s.csa_sparse_mla_bwd_workspace_bytes(0, 127, 0, ckv, torch.empty((0, 512), **i32), 512, 64, 4)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    empty = torch.empty((0, 64, 512), **bf)
    s.csa_sparse_mla_bwd(empty, kv, ckv, torch.empty((0, 512), **i32), 512, 0, 64, 16, 64, 512, cu_q, cu_kv, cu_cmp,
                         1, 64, 4, 127, 0, 64, sinks, 512 ** -0.5, empty,
                         torch.empty((0, 64), dtype=torch.float32, device="cuda"), empty, empty, d_ori, d_cmp, d_s,
                         None, None, 0, ws)
    torch.cuda.synchronize()
    for t in (d_ori, d_cmp, d_s):
        assert not t.isnan().any() and not t.any()


@pytest.mark.parametrize("name", ["select16", "edges", "hca_small", "cp_small", "win_right", "no_compress",
                                  "many_segs", "topk1024", "pack16k"])
def test_deterministic_backward_is_bit_reproducible(name):
    """csa_sparse_mla_bwd_deterministic: two calls give identical outputs to the bit; dq, the
    probabilities and d_sinks equal the atomic call's exactly (the same kernels), the row
    gradients equal it up to float32 summation order, and they meet the oracle's bounds
    (every query, through the atomic call they match)."""
    pack = make_pack("pack16k") if name == "pack16k" else _small(name)
    plan = run_pack(pack)
    a, dout, attend_all, slots = _run_bwd(pack, plan, seed=71)
    d1, _, _, _ = _run_bwd(pack, plan, seed=71, deterministic=True)
    d2, _, _, _ = _run_bwd(pack, plan, seed=71, deterministic=True)
    for k in d1:
        if d1[k] is None:
            continue
        assert np.array_equal(d1[k], d2[k]), f"{k} differs between two deterministic calls"
    for k in ("dq", "ori_l1", "cmp_l1", "d_sinks"):
        if a[k] is not None:
            assert np.array_equal(a[k], d1[k]), f"{k} differs from the atomic call"
    for k in ("d_ori_kv", "d_cmp_kv"):
        if a[k] is None:
            continue
        ref = np.asarray(a[k], np.float64)
        got = np.asarray(d1[k], np.float64)
        scale = max(float(np.abs(ref).max()), 1e-30)
        err = float(np.abs(got - ref).max())
        print(f"    {k}: max|det - atomic| = {err:.3e} (|ref|inf {scale:.3e})", flush=True)
        assert err <= 1e-5 * scale, k
