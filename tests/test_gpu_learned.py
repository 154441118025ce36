"""GPU parity of the learned gated compressor (csa_compress_learned) against the fp64 oracle.

Inputs are seeded (synth.compressor_inputs); the compressed cu_seqlens come from the
library's csa_build_indices.  The oracle runs on the same bf16 values in float64.

Tolerance (from the arithmetic): the projections are float32 sums of exact bf16
products (relative error ~1e-6 of the kv scale), the softmax is float32, and the
result is rounded once to bf16 (at most 2^-9 relative).  Bound per element:
|got - ref| <= 2^-8 |ref| + 1e-4 max|ref|, and rel-L2 <= 3e-3.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_support import cpu, to_device
from synth import bf16_bits_to_f32, compressor_inputs, make_pack

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SENTINEL = 0x4B3C  # bf16 bits written into rows past the compressed count beforehand


def _cu_cmp(cu_kv, r):
    from sparse_attention_thd_amd import _lib
    cu = torch.from_numpy(np.asarray(cu_kv, dtype=np.int32)).cuda()
    B = len(cu_kv) - 1
    T = int(cu_kv[-1])
    cu_cmp = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    res = torch.zeros(B, dtype=torch.int32, device="cuda")
    _lib.csa_build_indices(cu, cu, B, T, T, 0, r, 127, 0, None, None, None, cu_cmp, res, None, None, None,
                           max(T // r, 1))
    return cu, cu_cmp


def _run(cu_kv, ci, Tc_cap=None):
    import sparse_attention_thd_amd as s
    T = int(cu_kv[-1])
    r = ci.cmp_ratio
    Tc_cap = max(T // r, 1) if Tc_cap is None else Tc_cap
    cu, cu_cmp = _cu_cmp(cu_kv, r)
    out = torch.full((Tc_cap, ci.hd), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    print(f"[case] csa_compress_learned Tkv={T} D={ci.D} hd={ci.hd} overlap={ci.overlap} B={len(cu_kv) - 1} "
          f"Tc_cap={Tc_cap}", flush=True)
    s.csa_compress_learned(to_device(ci.x), T, ci.D, to_device(ci.wkv), to_device(ci.wgate), to_device(ci.ape),
                           ci.hd, ci.overlap, cu, cu_cmp, len(cu_kv) - 1, r, out, Tc_cap)
    torch.cuda.synchronize()
    bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return bits, int(cu_cmp[-1].item())


def _ref(cu_kv, ci, x_rows=None):
    x = bf16_bits_to_f32(ci.x if x_rows is None else x_rows)
    return oracle.compress_learned(x, bf16_bits_to_f32(ci.wkv), bf16_bits_to_f32(ci.wgate), ci.ape, cu_kv,
                                   ci.cmp_ratio, ci.overlap)


def _close(got_bits, ref, what):
    got = bf16_bits_to_f32(got_bits).astype(np.float64)
    diff = np.abs(got - ref)
    rmax = float(np.abs(ref).max())
    l2 = float(np.linalg.norm(diff)) / max(float(np.linalg.norm(ref)), 1e-300)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4 * rmax
    worst = float((diff - bound).max())
    print(f"    {what}: max|d|={float(diff.max()):.3e} |ref|inf={rmax:.3e} relL2={l2:.3e}", flush=True)
    assert l2 <= 3e-3, what
    assert worst <= 0.0, f"{what}: exceeds the element bound by {worst:.3e}"


def _lengths(name):
    if name == "small":
        return [37, 91, 2, 260, 3, 130, 1, 700]
    if name == "tiles":
        return [1200, 37, 900, 1201, 5]
    if name == "many_segs":
        return [5 + (37 * k) % 120 for k in range(60)]
    if name == "empty_segs":
        return [0, 410, 0, 0, 3, 257, 0]
    raise KeyError(name)


CASES = [
    ("small", dict(D=256, hd=64, overlap=True)),
    ("small", dict(D=256, hd=128, overlap=False)),
    ("tiles", dict(D=512, hd=512, overlap=True)),
    ("tiles", dict(D=512, hd=256, overlap=False)),
    ("many_segs", dict(D=1024, hd=128, overlap=True)),
    ("empty_segs", dict(D=192, hd=192, overlap=True)),
    ("tiles", dict(D=320, hd=128, overlap=True, gate_scale=24.0, ape_scale=6.0)),  # peaky softmax
    ("small", dict(D=64, hd=64, overlap=True)),      # one K step
    ("empty_segs", dict(D=128, hd=128, overlap=False)),  # two K steps
]


@pytest.mark.parametrize("name,kw", CASES, ids=[f"{n}-{'-'.join(f'{k}{v}' for k, v in kw.items())}" for n, kw in CASES])
def test_learned_compressor_matches_oracle(name, kw):
    lengths = _lengths(name)
    cu_kv = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    ci = compressor_inputs(int(cu_kv[-1]), seed=11, **kw)
    bits, Tc = _run(cu_kv, ci)
    ref = _ref(cu_kv, ci)
    assert Tc == ref.shape[0]
    _close(bits[:Tc], ref, name)
    assert (bits[Tc:] == SENTINEL).all(), "rows past the compressed count stay untouched"


def test_learned_compressor_is_deterministic():
    lengths = _lengths("tiles")
    cu_kv = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    ci = compressor_inputs(int(cu_kv[-1]), D=512, hd=128, overlap=True, seed=12)
    a, _ = _run(cu_kv, ci)
    b, _ = _run(cu_kv, ci)
    assert np.array_equal(a, b)


def test_learned_compressor_pack16k_every_segment():
    """The 16k pack at hidden size 4096 for the latent (hd 512) and the indexer keys
    (hd 128); the oracle checks every segment."""
    pack = make_pack("pack16k")
    cu_kv = pack.cu_seqlens_kv.astype(np.int64)
    T = int(cu_kv[-1])
    lens = np.diff(cu_kv)
    segs = list(range(len(lens)))
    cmp_cu = np.concatenate([[0], np.cumsum(lens // 4)])
    for hd in (512, 128):
        ci = compressor_inputs(T, D=4096, hd=hd, overlap=True, seed=13)
        print(f"[case] pack16k: learned compressor hd {hd}, {len(segs)} segments", flush=True)
        bits, Tc = _run(cu_kv, ci)
        assert Tc == int(cmp_cu[-1])
        for b in segs:
            s, e = int(cu_kv[b]), int(cu_kv[b + 1])
            ref = _ref(np.array([0, e - s]), ci, x_rows=ci.x[s:e])
            _close(bits[int(cmp_cu[b]):int(cmp_cu[b + 1])], ref, f"hd{hd} segment {b} ({e - s} rows)")


def test_plan_with_learned_compressors():
    """CsaPlan.run with learned compressors for the latent rows and the indexer keys (hidden
    size 256): compressed rows against the oracle, top-k sets against oracle scores of the
    GPU's compressed keys, attention against the oracle on those rows and sets."""
    import sparse_attention_thd_amd as s
    from gpu_support import assert_out_close, check_topk_row, host_view, oracle_attention, oracle_tables
    from synth import pack_from_lengths
    pack = pack_from_lengths("learned_plan", [600, 300, 1201], seed=4, topk=16)
    ckv = compressor_inputs(pack.Tkv, D=256, hd=512, overlap=True, seed=31)
    ckey = compressor_inputs(pack.Tkv, D=256, hd=128, overlap=True, seed=32)
    x = ckv.x  # both compressors read the same hidden rows
    layout = s.ThdLayout.from_host(pack.cu_seqlens_q, pack.cu_seqlens_kv, pack.global_start)
    plan = s.CsaPlan(layout, H=pack.H, d=pack.d, H_I=pack.H_I, d_I=pack.d_I, cmp_ratio=4, topk=pack.topk,
                     softmax_scale=pack.softmax_scale, return_topk_score=True)
    kvc = s.LearnedCompressor(to_device(ckv.wkv), to_device(ckv.wgate), to_device(ckv.ape))
    keyc = s.LearnedCompressor(to_device(ckey.wkv), to_device(ckey.wgate), to_device(ckey.ape))
    print("[case] learned_plan: CsaPlan.run with learned compressors", flush=True)
    plan.run(to_device(pack.q), to_device(pack.ori_kv), sinks=to_device(pack.sinks), q_I=to_device(pack.q_I),
             w=to_device(pack.w), x=to_device(x), kv_compressor=kvc, key_compressor=keyc)
    torch.cuda.synchronize()
    tabs = oracle_tables(pack)
    Tc = int(tabs["cu_seqlens_cmp"][-1])
    xf = bf16_bits_to_f32(x)
    for got, ci, what in ((plan.cmp_kv, ckv, "latent"), (plan.k_I_cmp, ckey, "keys")):
        ref = oracle.compress_learned(xf, bf16_bits_to_f32(ci.wkv), bf16_bits_to_f32(ci.wgate), ci.ape,
                                      pack.cu_seqlens_kv, 4, True)
        bits = got.view(torch.int16).cpu().numpy().view(np.uint16)[:Tc]
        _close(bits, ref, what)
    kc = cpu(plan.k_I_cmp)[:Tc].astype(np.float64)
    idx = cpu(plan.topk_idx)
    qI, w = host_view(pack, "q_I"), host_view(pack, "w")
    for i in range(pack.Tq):
        lo, nv = int(tabs["q_cmp_lo"][i]), int(tabs["q_cmp_nvis"][i])
        sc = oracle.indexer_scores(qI[i], w[i], kc[lo:lo + nv]) if nv else np.zeros(0)
        check_topk_row(idx[i], lo, nv, sc, pack.topk)
    qs = list(range(0, pack.Tq, 5))
    out, _ = oracle_attention(pack, tabs, qs, cpu(plan.cmp_kv)[:Tc].astype(np.float64), idx[qs], oracle.INDEXER)
    print("   ", assert_out_close(cpu(plan.out)[qs], out), flush=True)


def test_learned_compressor_without_complete_groups():
    """Every segment shorter than the ratio: no compressed row, nothing written."""
    cu_kv = np.array([0, 1, 3, 6, 7])
    ci = compressor_inputs(7, D=64, hd=64, overlap=True, seed=14)
    bits, Tc = _run(cu_kv, ci)
    assert Tc == 0 and (bits == SENTINEL).all()


def _random_shape(seed):
    """Hidden size, head width, overlap, segment lengths (empty, 1-3 rows, short, long), gates."""
    rng = np.random.default_rng(31000 + seed)
    overlap = bool(rng.random() < 0.6)
    D = 64 * int(rng.integers(1, 17))
    hd = 64 * int(rng.integers(1, 9)) if overlap else 128 * int(rng.integers(1, 5))
    nseg = int(rng.integers(1, 11))
    kinds = rng.integers(0, 4, size=nseg)
    lengths = [int(v) for v in np.where(kinds == 0, rng.integers(0, 4, size=nseg),
                                        np.where(kinds == 1, rng.integers(4, 21, size=nseg),
                                                 rng.integers(100, 1500, size=nseg)))]
    if sum(lengths) < 4:
        lengths.append(9)
    peaky = rng.random() < 0.2
    scales = dict(gate_scale=12.0, ape_scale=4.0) if peaky else {}
    return lengths, dict(D=D, hd=hd, overlap=overlap, **scales)


@pytest.mark.parametrize("seed", list(range(16)))
def test_learned_compressor_random_shapes(seed):
    """Seeded random shapes and layouts against the oracle, with the element bound above."""
    lengths, kw = _random_shape(seed)
    cu_kv = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    print(f"[case] learned random{seed}: lengths={lengths} {kw}", flush=True)
    ci = compressor_inputs(int(cu_kv[-1]), seed=100 + seed, **kw)
    bits, Tc = _run(cu_kv, ci)
    ref = _ref(cu_kv, ci)
    assert Tc == ref.shape[0]
    if Tc:
        _close(bits[:Tc], ref, f"random{seed}")
    assert (bits[Tc:] == SENTINEL).all()
