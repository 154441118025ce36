"""Helpers for the GPU parity tests: upload synthetic packs, run the library,
and compare against the oracle with the stated tolerances."""
from __future__ import annotations

import math

import numpy as np

import oracle
from synth import bf16_bits_to_f32

# bf16-in / fp32-accumulate outputs: the stated max-abs and mean-abs bounds plus
# scale-aware relative bounds (at the workloads' value scale an all-zero output
# sits close to the absolute bounds, the relative ones do not let it pass).
OUT_MAX_ABS = 2e-2
OUT_MEAN_ABS = 2e-3
OUT_REL_INF = 1e-2
OUT_REL_L2 = 5e-3
OUT_F32_MAX_ABS = 1e-4
LSE_ABS = 2e-3
TIE_BAND = 1e-3


class Decoded:
    """Row access to a bf16 bit array as float32, without decoding it whole."""

    def __init__(self, bits):
        self.bits = bits
        self.shape = bits.shape

    def __len__(self):
        return self.bits.shape[0]

    def __getitem__(self, idx):
        return bf16_bits_to_f32(self.bits[idx])


def host_view(pack, name):
    a = getattr(pack, name)
    if a is None:
        return None
    return Decoded(a) if a.dtype == np.uint16 else a


def to_device(a):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_pack(pack, *, return_lse=True, return_topk_score=True, emit_window=True):
    """Run the whole forward through the C ABI; returns the plan (device tensors)."""
    import torch
    from sparse_attention_thd_amd import CsaPlan, ThdLayout
    layout = ThdLayout.from_host(pack.cu_seqlens_q, pack.cu_seqlens_kv, pack.global_start)
    assert layout.Tq == pack.Tq and layout.Tkv == pack.Tkv
    dt = torch.bfloat16 if pack.dtype == "bf16" else torch.float32
    plan = CsaPlan(layout, H=pack.H, d=pack.d, H_I=pack.H_I, d_I=pack.d_I, cmp_ratio=pack.cmp_ratio,
                   ori_win_left=pack.ori_win_left, ori_win_right=pack.ori_win_right, topk=pack.topk,
                   softmax_scale=pack.softmax_scale, dtype=dt, emit_window=emit_window, return_lse=return_lse,
                   return_topk_score=return_topk_score and pack.has_indexer)
    plan.run(to_device(pack.q), to_device(pack.ori_kv), sinks=to_device(pack.sinks), q_I=to_device(pack.q_I),
             k_I=to_device(pack.k_I), w=to_device(pack.w))
    torch.cuda.synchronize()
    return plan


def cpu(t):
    import torch
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def oracle_tables(pack):
    return oracle.build_indices(pack.cu_seqlens_q, pack.cu_seqlens_kv, pack.global_start, pack.Tq,
                                pack.cmp_ratio, pack.ori_win_left, pack.ori_win_right)


def sample_queries(pack, tabs, n=160, seed=0):
    """Random queries plus the structural edges: first/last rows of every segment,
    rows where the visible compressed count crosses top-k, the first and last row."""
    rng = np.random.default_rng(seed)
    Tq = pack.Tq
    qs = set(int(v) for v in rng.choice(Tq, size=min(n, Tq), replace=False))
    cu = [int(v) for v in pack.cu_seqlens_q]
    for b in range(len(cu) - 1):
        if cu[b + 1] > cu[b]:
            qs.update([cu[b], min(cu[b] + 1, cu[b + 1] - 1), cu[b + 1] - 1])
    nv = tabs["q_cmp_nvis"]
    for k in (pack.topk, pack.topk + 1):
        hit = np.nonzero(nv == k)[0]
        if hit.size:
            qs.add(int(hit[0]))
    qs.update([0, Tq - 1])
    return sorted(q for q in qs if 0 <= q < Tq)


def check_topk_row(row, lo, nv, scores, topk, gpu_scores=None):
    """Set-level check of one query's top-k list against oracle fp64 scores."""
    row = np.asarray(row)
    valid = row[row >= 0]
    assert (row[len(valid):] == -1).all(), "padding must follow the kept rows"
    assert (np.diff(valid) > 0).all(), "kept rows must be ascending"
    if nv <= topk:
        np.testing.assert_array_equal(valid, np.arange(lo, lo + nv))
        return 0
    assert len(valid) == topk
    sel = valid - lo
    assert sel.min() >= 0 and sel.max() < nv
    s_star = np.sort(scores)[::-1][topk - 1]
    beta = TIE_BAND * max(1.0, abs(s_star))
    must = set(np.nonzero(scores > s_star + beta)[0].tolist())
    mustnot = set(np.nonzero(scores < s_star - beta)[0].tolist())
    chosen = set(sel.tolist())
    assert must <= chosen, f"missing rows clearly inside the top-k: {sorted(must - chosen)[:8]}"
    assert not (mustnot & chosen), f"rows clearly outside the top-k kept: {sorted(mustnot & chosen)[:8]}"
    if gpu_scores is not None:
        ref = scores[sel]
        got = np.asarray(gpu_scores)[:topk]
        assert np.all(np.abs(got - ref) <= 1e-3 * np.maximum(1.0, np.abs(ref)))
    oracle_set = set(np.argsort(-scores, kind="stable")[:topk].tolist())
    return len(chosen ^ oracle_set) // 2


def assert_out_close(got, ref, fp32=False, what="out"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(got - ref)
    mx, mean = float(d.max()), float(d.mean())
    ref_inf = float(np.abs(ref).max())
    l2 = float(np.linalg.norm(d)) / max(float(np.linalg.norm(ref)), 1e-300)
    msg = f"{what}: max|d|={mx:.3e} mean|d|={mean:.3e} |ref|inf={ref_inf:.3e} relL2={l2:.3e}"
    assert mx <= OUT_MAX_ABS, msg
    assert mean <= OUT_MEAN_ABS, msg
    assert mx <= OUT_REL_INF * ref_inf, msg
    assert l2 <= OUT_REL_L2, msg
    if fp32:
        assert mx <= OUT_F32_MAX_ABS, msg
    return msg


class OutClose:
    """assert_out_close over an output compared chunk by chunk (same bounds, computed
    from running sums), so a full-size output never has to sit in float64 whole."""

    def __init__(self, what="out"):
        self.what = what
        self.n = 0
        self.mx = self.sum_abs = self.sum_sq = self.ref_sq = self.ref_inf = 0.0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        d = np.abs(got - ref)
        self.n += d.size
        self.mx = max(self.mx, float(d.max()) if d.size else 0.0)
        self.sum_abs += float(d.sum())
        self.sum_sq += float((d * d).sum())
        self.ref_sq += float((ref * ref).sum())
        self.ref_inf = max(self.ref_inf, float(np.abs(ref).max()) if ref.size else 0.0)

    def check(self, fp32=False):
        mean = self.sum_abs / max(self.n, 1)
        l2 = math.sqrt(self.sum_sq) / max(math.sqrt(self.ref_sq), 1e-300)
        msg = (f"{self.what}: max|d|={self.mx:.3e} mean|d|={mean:.3e} |ref|inf={self.ref_inf:.3e} "
               f"relL2={l2:.3e} over {self.n} values")
        assert self.mx <= OUT_MAX_ABS, msg
        assert mean <= OUT_MEAN_ABS, msg
        assert self.mx <= OUT_REL_INF * self.ref_inf, msg
        assert l2 <= OUT_REL_L2, msg
        if fp32:
            assert self.mx <= OUT_F32_MAX_ABS, msg
        return msg


def oracle_attention(pack, tabs, queries, cmp_kv, cmp_idx_rows=None, mode=None):
    """Oracle sparse MLA for `queries` with the given compressed rows and selection."""
    if mode is None:
        mode = oracle.layer_compress_mode(pack.cmp_ratio, int(tabs["cu_seqlens_cmp"][-1]))
    cmp_idx = None
    if mode == oracle.INDEXER:
        cmp_idx = {i: cmp_idx_rows[n] for n, i in enumerate(queries)}
    return oracle.sparse_mla_fwd(host_view(pack, "q"), host_view(pack, "ori_kv"),
                                 cmp_kv if mode != oracle.NO_COMPRESS else None, cmp_idx, tabs, pack.sinks,
                                 pack.softmax_scale, pack.ori_win_left, pack.ori_win_right, pack.cu_seqlens_kv,
                                 pack.global_start, queries=queries,
                                 attend_all_visible=(mode == oracle.COMPRESSOR_ONLY))


def scale_summary(x):
    x = np.asarray(x, dtype=np.float64)
    return dict(absmax=float(np.abs(x).max()), mean_abs=float(np.abs(x).mean()), l2=float(math.sqrt((x ** 2).sum())))
