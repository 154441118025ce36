"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects invalid arguments on the host before any HIP call.

Every call here is built to fail validation, so nothing is launched.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

lib_mod = pytest.importorskip("sparse_attention_thd_amd._lib", reason="libcsa.so not built")
LIB = lib_mod.LIB
EINVAL, EUNSUP = lib_mod.CSA_EINVAL, lib_mod.CSA_EUNSUPPORTED
FAKE = 0x1000  # a non-NULL pointer value; validation fails before it could be used


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_steps():
    names = declared_functions()
    for n in ("csa_build_indices", "csa_compress", "csa_indexer_topk", "csa_sparse_mla_fwd"):
        assert n in names


def test_library_exports_every_declared_symbol():
    raw = C.CDLL(lib_mod.LIB_PATH)
    for n in declared_functions():
        assert hasattr(raw, n), n
        assert n in lib_mod.SIGNATURES, f"binding lacks {n}"


def test_debug_build_exports_every_declared_symbol():
    if not os.path.exists(lib_mod.DEBUG_LIB_PATH):
        pytest.skip("libcsa_debug.so not built")
    dbg = lib_mod.load(lib_mod.DEBUG_LIB_PATH)
    for n in declared_functions():
        assert hasattr(dbg, n), n
    assert dbg.csa_version().endswith(b"+debug")
    assert not lib_mod.csa_version().endswith("+debug")


@pytest.mark.parametrize("kw", [dict(cidx=None), dict(topk=0), dict(B=0), dict(r=0), dict(gs=-1), dict(Tc=-1),
                                dict(cu_cmp=None), dict(Tq=-1)])
def test_validate_topk_rows_rejects(kw):
    a = dict(cidx=FAKE, topk=512, Tq=8, Tc=2, cu_q=FAKE, cu_kv=FAKE, cu_cmp=FAKE, B=1, gs=0, r=4, stream=None)
    a.update(kw)
    assert LIB.csa_validate_topk_rows(*a.values()) == EINVAL
    assert b"csa_validate_topk_rows" in LIB.csa_last_error()


def test_version_and_empty_error():
    assert lib_mod.csa_version().startswith("csa-gfx950")


def _bi(**kw):
    a = dict(cu_q=FAKE, cu_kv=FAKE, B=1, Tq=4, Tkv=4, gs=0, r=4, wl=127, wr=0, q_seg=None, q_pos=None, win=None,
             cu_cmp=FAKE, res=FAKE, lo=None, nv=None, grp=None, Tc_cap=1, stream=None)
    a.update(kw)
    return LIB.csa_build_indices(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(cu_q=None), EINVAL), (dict(cu_kv=None), EINVAL), (dict(cu_cmp=None), EINVAL), (dict(res=None), EINVAL),
    (dict(B=0), EINVAL), (dict(Tq=-1), EINVAL), (dict(Tq=5), EINVAL), (dict(gs=1), EINVAL),
    (dict(r=0), EINVAL), (dict(wl=-1), EINVAL), (dict(wr=-2), EINVAL), (dict(grp=FAKE, Tc_cap=0, r=2), EINVAL),
    (dict(wl=2**31 - 4), EINVAL), (dict(wl=2**30, wr=2**30), EINVAL),
])
def test_build_indices_rejects(kw, code):
    assert _bi(**kw) == code
    assert "csa_build_indices" in lib_mod.csa_last_error()


def _cmp(**kw):
    a = dict(x=FAKE, Tkv=16, d=512, dtype=1, cu_kv=FAKE, cu_cmp=FAKE, B=1, r=4, out=FAKE, Tc_cap=4, stream=None)
    a.update(kw)
    return LIB.csa_compress(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), EINVAL), (dict(out=None), EINVAL), (dict(B=0), EINVAL), (dict(d=0), EINVAL),
    (dict(r=0), EINVAL), (dict(dtype=7), EINVAL), (dict(Tc_cap=3), EINVAL), (dict(d=12), EUNSUP),
    (dict(d=6, dtype=0), EUNSUP),
])
def test_compress_rejects(kw, code):
    assert _cmp(**kw) == code


def _learned(**kw):
    a = dict(x=FAKE, Tkv=16, D=4096, dtype=1, wkv=FAKE, wgate=FAKE, ape=FAKE, hd=512, overlap=1, cu_kv=FAKE,
             cu_cmp=FAKE, B=1, r=4, out=FAKE, Tc_cap=4, stream=None)
    a.update(kw)
    return LIB.csa_compress_learned(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), EINVAL), (dict(wkv=None), EINVAL), (dict(wgate=None), EINVAL), (dict(ape=None), EINVAL),
    (dict(out=None), EINVAL), (dict(cu_cmp=None), EINVAL), (dict(B=0), EINVAL), (dict(D=0), EINVAL),
    (dict(hd=0), EINVAL), (dict(r=0), EINVAL), (dict(overlap=2), EINVAL), (dict(dtype=7), EINVAL),
    (dict(Tc_cap=3), EINVAL), (dict(r=8, Tc_cap=2), EUNSUP), (dict(D=4000), EUNSUP), (dict(D=32), EUNSUP), (dict(hd=96), EUNSUP),
    (dict(hd=64, overlap=0), EUNSUP), (dict(dtype=0), EUNSUP), (dict(Tkv=1 << 20, Tc_cap=1 << 18), EUNSUP),
])
def test_compress_learned_rejects(kw, code):
    assert _learned(**kw) == code


def test_compress_learned_accepts_empty_streams():
    # nothing to launch: no row reaches a complete group, or no rows at all
    assert _learned(Tkv=0, Tc_cap=0, x=None, out=None) == 0
    assert _learned(x=None, wkv=None, wgate=None, ape=None, Tkv=0, Tc_cap=0, out=None) == 0


def _idx(**kw):
    a = dict(q=FAKE, w=FAKE, k=FAKE, Tq=8, Tc=2, H_I=64, d_I=128, dtype=1, cu_q=FAKE, cu_kv=FAKE, cu_cmp=FAKE,
             res=None, B=1, gs=0, r=4, maxlen=8, topk=512, idx=FAKE, sc=None, ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return LIB.csa_indexer_topk(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), EINVAL), (dict(idx=None), EINVAL), (dict(topk=0), EINVAL), (dict(B=0), EINVAL),
    (dict(maxlen=-1), EINVAL), (dict(dtype=3), EINVAL), (dict(Tc=-1), EINVAL), (dict(k=None), EINVAL),
    (dict(ws=None), EINVAL), (dict(ws_bytes=8 * 2 * 4 - 1), EINVAL), (dict(topk=4096), EUNSUP),
    (dict(maxlen=4 * 40000), EUNSUP), (dict(H_I=128, d_I=128), EUNSUP), (dict(H_I=2, d_I=12, dtype=0), EUNSUP),
])
def test_indexer_rejects(kw, code):
    assert _idx(**kw) == code


def test_indexer_workspace_size_formula():
    # one row of floor(max_seqlen_kv / r) uint32 score keys per query
    assert LIB.csa_indexer_topk_workspace_bytes(10, 4039, 4) == 10 * 1009 * 4
    assert LIB.csa_indexer_topk_workspace_bytes(32768, 22999, 4) == 32768 * 5749 * 4
    assert LIB.csa_indexer_topk_workspace_bytes(5, 3, 4) == 0
    assert LIB.csa_indexer_topk_workspace_bytes(-1, 8, 4) == -1
    assert LIB.csa_indexer_topk_workspace_bytes(1, 8, 0) == -1


def _mla(**kw):
    a = dict(q=FAKE, kv=FAKE, ckv=FAKE, cidx=FAKE, topk=512, kind=1, Tq=8, Tkv=8, Tc=2, H=64, d=512, dtype=1,
             cu_q=FAKE, cu_kv=FAKE, cu_cmp=FAKE, res=None, B=1, gs=0, r=4, wl=127, wr=0, sinks=None, scale=0.04,
             out=FAKE, lse=None, stream=None)
    a.update(kw)
    return LIB.csa_sparse_mla_fwd(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), EINVAL), (dict(out=None), EINVAL), (dict(ckv=None), EINVAL), (dict(topk=0), EINVAL),
    (dict(ckv=FAKE, cu_cmp=None), EINVAL), (dict(B=0), EINVAL), (dict(gs=1), EINVAL), (dict(wl=-1), EINVAL),
    (dict(kind=2), EINVAL), (dict(kind=-1), EINVAL), (dict(Tc=-1), EINVAL),
    (dict(dtype=5), EINVAL), (dict(scale=0.0), EINVAL), (dict(scale=-0.04), EINVAL),
    (dict(wl=2**31 - 8), EINVAL), (dict(wr=2**31 - 8), EINVAL),
    (dict(scale=float("inf")), EINVAL), (dict(scale=float("nan")), EINVAL), (dict(topk=4096), EUNSUP),
    (dict(H=128), EUNSUP), (dict(H=64, d=256), EUNSUP),
])
def test_sparse_mla_rejects(kw, code):
    assert _mla(**kw) == code


def _mla_bwd(**kw):
    a = dict(q=FAKE, kv=FAKE, ckv=FAKE, cidx=FAKE, topk=512, Tq=8, Tkv=8, Tc=2, H=64, d=512, dtype=1, cu_q=FAKE,
             cu_kv=FAKE, cu_cmp=FAKE, B=1, gs=0, r=4, wl=127, wr=0, maxlen=8, sinks=FAKE, scale=0.04, out=FAKE,
             lse=FAKE, dout=FAKE, dq=FAKE, dkv=FAKE, dcmp=FAKE, dsinks=FAKE, ol1=None, cl1=None, slots=0,
             ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return LIB.csa_sparse_mla_bwd(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), EINVAL), (dict(dout=None), EINVAL), (dict(lse=None), EINVAL), (dict(dq=None), EINVAL),
    (dict(ws=None), EINVAL), (dict(dkv=None), EINVAL), (dict(dcmp=None), EINVAL), (dict(dsinks=None), EINVAL),
    (dict(ckv=None), EINVAL), (dict(topk=0), EINVAL), (dict(cl1=FAKE, slots=0), EINVAL), (dict(B=0), EINVAL),
    (dict(gs=1), EINVAL), (dict(wr=-1), EINVAL), (dict(wl=2**31 - 8), EINVAL), (dict(scale=0.0), EINVAL),
    (dict(scale=float("nan")), EINVAL), (dict(ws_bytes=1024), EINVAL), (dict(topk=4096), EUNSUP),
    (dict(H=16), EUNSUP), (dict(dtype=0), EUNSUP),
])
def test_sparse_mla_bwd_rejects(kw, code):
    assert _mla_bwd(**kw) == code


def test_sparse_mla_bwd_workspace_size_formula():
    # per query: 32-rounded key slots x 256 B of scale*dS and P + 4 B + 64 sink terms x 4 B,
    # plus a 2 B selection-map entry per visible compressed row in the sparse mode; then, 16-byte aligned,
    # one 256 B row of zeros
    def total(Tq, per_query):
        return (Tq * per_query + 15) // 16 * 16 + 256
    n = LIB.csa_sparse_mla_bwd_workspace_bytes(10, 127, 0, FAKE, FAKE, 512, 4096, 4)
    assert n == total(10, 640 * 256 + 4 + 256 + 2 * 1024)
    n_all = LIB.csa_sparse_mla_bwd_workspace_bytes(3, 127, 0, FAKE, None, 0, 1000, 4)  # attend-all: 128 + 250 keys
    assert n_all == total(3, 384 * 256 + 4 + 256)
    assert LIB.csa_sparse_mla_bwd_workspace_bytes(-1, 127, 0, None, None, 0, 0, 4) == -1
    assert LIB.csa_sparse_mla_bwd_workspace_bytes(1, 2**31 - 1, 1, None, None, 0, 0, 4) == -1  # sides overflow int32
    # a window wider than the longest segment holds at most max_seqlen_kv keys
    n_wide = LIB.csa_sparse_mla_bwd_workspace_bytes(2, 100000, 0, None, None, 0, 300, 4)
    assert n_wide == total(2, 320 * 256 + 4 + 256)


def _mla_bwd_det(**kw):
    a = dict(q=FAKE, kv=FAKE, ckv=FAKE, cidx=FAKE, topk=512, Tq=8, Tkv=8, Tc=2, H=64, d=512, dtype=1, cu_q=FAKE,
             cu_kv=FAKE, cu_cmp=FAKE, B=1, gs=0, r=4, wl=127, wr=0, maxlen=8, sinks=FAKE, scale=0.04, out=FAKE,
             lse=FAKE, dout=FAKE, dq=FAKE, dkv=FAKE, dcmp=FAKE, dsinks=FAKE, ol1=None, cl1=None, slots=0,
             ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return LIB.csa_sparse_mla_bwd_deterministic(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), EINVAL), (dict(ws=None), EINVAL), (dict(dkv=None), EINVAL), (dict(B=0), EINVAL),
    (dict(topk=0), EINVAL), (dict(scale=0.0), EINVAL), (dict(ws_bytes=1024), EINVAL), (dict(H=16), EUNSUP),
])
def test_sparse_mla_bwd_deterministic_rejects(kw, code):
    assert _mla_bwd_det(**kw) == code
    assert b"csa_sparse_mla_bwd_deterministic" in LIB.csa_last_error()


def test_sparse_mla_bwd_deterministic_needs_the_partial_tiles():
    # the atomic call's workspace is not enough: the per-item tiles come on top of it
    base = LIB.csa_sparse_mla_bwd_workspace_bytes(8, 127, 0, FAKE, FAKE, 512, 8, 4)
    assert _mla_bwd_det(ws_bytes=base) == EINVAL
    assert b"workspace" in LIB.csa_last_error()


def test_sparse_mla_bwd_deterministic_workspace_size_formula():
    # the atomic workspace + (ceil(Tq / 128) + B) query chunks x 2 (n_w + n_c) items x 256 x 256 float32,
    # n_w = min(127 + wl + wr, max_seqlen_kv - 1) // 256 + 1, n_c = ceil(floor(max_seqlen_kv / r) / 256)
    base = LIB.csa_sparse_mla_bwd_workspace_bytes(10, 127, 0, FAKE, FAKE, 512, 4039, 4)
    n = LIB.csa_sparse_mla_bwd_deterministic_workspace_bytes(10, 1, 127, 0, FAKE, FAKE, 512, 4039, 4)
    assert n == base + (1 + 1) * 2 * (1 + 4) * 256 * 256 * 4
    base2 = LIB.csa_sparse_mla_bwd_workspace_bytes(300, 127, 0, None, None, 0, 700, 4)  # window only
    n2 = LIB.csa_sparse_mla_bwd_deterministic_workspace_bytes(300, 3, 127, 0, None, None, 0, 700, 4)
    assert n2 == base2 + (3 + 3) * 2 * (1 + 0) * 256 * 256 * 4
    assert LIB.csa_sparse_mla_bwd_deterministic_workspace_bytes(10, 0, 127, 0, FAKE, FAKE, 512, 4039, 4) == -1
    assert LIB.csa_sparse_mla_bwd_deterministic_workspace_bytes(-1, 1, 127, 0, None, None, 0, 0, 4) == -1


def _kl(**kw):
    a = dict(q=FAKE, w=FAKE, k=FAKE, cidx=FAKE, p=FAKE, topk=512, Tq=8, Tc=2, H=64, d=128, dtype=1, cu_q=FAKE,
             cu_kv=FAKE, cu_cmp=FAKE, B=1, gs=0, r=4, maxlen=8, scale=1.0, dq=FAKE, dw=FAKE, dk=FAKE, loss=None,
             ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return LIB.csa_indexer_kl_grad(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), EINVAL), (dict(w=None), EINVAL), (dict(cidx=None), EINVAL), (dict(p=None), EINVAL),
    (dict(dq=None), EINVAL), (dict(dw=None), EINVAL), (dict(dk=None), EINVAL), (dict(k=None), EINVAL),
    (dict(ws=None), EINVAL), (dict(cu_cmp=None), EINVAL), (dict(topk=0), EINVAL), (dict(B=0), EINVAL),
    (dict(r=0), EINVAL), (dict(gs=-1), EINVAL), (dict(ws_bytes=16), EINVAL), (dict(topk=4096), EUNSUP),
    (dict(H=16), EUNSUP), (dict(d=64), EUNSUP), (dict(dtype=0), EUNSUP),
])
def test_indexer_kl_grad_rejects(kw, code):
    assert _kl(**kw) == code


def _kl_noalloc(**kw):
    a = dict(q=FAKE, w=FAKE, k=FAKE, cidx=FAKE, p=FAKE, topk=512, Tq=8, Tc=2, H=64, d=128, dtype=1, cu_q=FAKE,
             cu_kv=FAKE, cu_cmp=FAKE, B=1, gs=0, r=4, maxlen=8, scale=1.0, dq=FAKE, dw=FAKE, dk=FAKE, loss=None,
             stream=None)
    a.update(kw)
    return LIB.csa_indexer_kl_grad_noalloc(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), EINVAL), (dict(cidx=None), EINVAL), (dict(p=None), EINVAL), (dict(dq=None), EINVAL),
    (dict(dk=None), EINVAL), (dict(topk=0), EINVAL), (dict(B=0), EINVAL), (dict(r=0), EINVAL),
    (dict(Tq=40000, topk=512), EINVAL),                  # 40000 * 2048 B of slot gradients > 64 MiB
    (dict(Tq=16384, maxlen=1 << 30), EINVAL),            # the visible-row map alone > 64 MiB
    (dict(topk=4096), EUNSUP), (dict(H=16), EUNSUP), (dict(dtype=0), EUNSUP),
])
def test_indexer_kl_grad_noalloc_rejects(kw, code):
    assert _kl_noalloc(**kw) == code
    assert "csa_indexer_kl_grad_noalloc" in lib_mod.csa_last_error()


def test_indexer_kl_grad_noalloc_limit_covers_the_16k_pack():
    # the 16384-token pack (longest segment 4039 rows, top-512) fits the 64 MiB the library holds
    assert LIB.csa_indexer_kl_grad_workspace_bytes(16384, 512, 4039, 4) <= 64 << 20


def test_indexer_kl_grad_workspace_size_formula():
    # per query: topk float32 slot gradients + a 2 B map entry per visible compressed row
    assert LIB.csa_indexer_kl_grad_workspace_bytes(10, 512, 4096, 4) == 10 * (512 * 4 + 2 * 1024)
    assert LIB.csa_indexer_kl_grad_workspace_bytes(3, 16, 1000, 128) == 3 * (16 * 4 + 2 * 7)
    assert LIB.csa_indexer_kl_grad_workspace_bytes(-1, 16, 10, 4) == -1
    assert LIB.csa_indexer_kl_grad_workspace_bytes(2, 0, 10, 4) == -1


def test_validate_layout_rejects_bad_arguments():
    assert LIB.csa_validate_layout(None, FAKE, 1, 0, 0, 0, -1, 0, None, None, None) == EINVAL
    assert LIB.csa_validate_layout(FAKE, FAKE, 0, 0, 0, 0, -1, 0, None, None, None) == EINVAL
    assert LIB.csa_validate_layout(FAKE, FAKE, 1, 0, 0, 0, -1, -1, None, None, None) == EINVAL


def test_plan_rejects_learned_compressor_misuse_before_any_call():
    """CsaPlan.run checks learned-compressor arguments on the host (CPU tensors here:
    the checks fire before the first library call)."""
    import torch
    from sparse_attention_thd_amd import CsaPlan, LearnedCompressor, ThdLayout
    layout = ThdLayout.from_host([0, 8], [0, 8], device="cpu")
    plan = CsaPlan(layout, H=4, d=64, H_I=2, d_I=32, cmp_ratio=4, topk=4, dtype=torch.float32)
    comp = LearnedCompressor(torch.zeros(128, 16), torch.zeros(128, 16), torch.zeros(4, 128))  # hd 64
    assert comp.hd() == 64
    assert LearnedCompressor(comp.wkv[:64], comp.wgate[:64], comp.ape[:, :64], overlap=False).hd() == 64
    with pytest.raises(ValueError, match="hidden rows"):
        plan.run(None, None, kv_compressor=comp)
    with pytest.raises(ValueError, match="32"):
        plan.run(None, None, x=torch.zeros(8, 16), key_compressor=comp)
