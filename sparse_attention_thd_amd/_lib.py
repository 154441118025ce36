"""ctypes binding of libcsa.so: the C ABI declared in include/csa.h, same names.

Argument marshalling only: tensors become device pointers, the stream is torch's
current stream, and a nonzero status raises ``CsaError`` with the library's
message.  Every computation happens in the HIP kernels; there is no fallback,
and importing this module fails loudly when libcsa.so has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

# CSA_LIBRARY may point at another build of the same library (e.g. a debug build).
LIB_PATH = os.environ.get("CSA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")

CSA_OK, CSA_EINVAL, CSA_EUNSUPPORTED, CSA_EHIP = 0, 1, 2, 4
CSA_F32, CSA_BF16 = 0, 1
CSA_IDX_ANY, CSA_IDX_TOPK = 0, 1

_P = C.c_void_p
_I = C.c_int32

# name -> argtypes, in the order of include/csa.h
SIGNATURES = {
    "csa_version": [],
    "csa_last_error": [],
    "csa_build_indices": [_P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P],
    "csa_compress": [_P, _I, _I, _I, _P, _P, _I, _I, _P, _I, _P],
    "csa_compress_learned": [_P, _I, _I, _I, _P, _P, _P, _I, _I, _P, _P, _I, _I, _P, _I, _P],
    "csa_indexer_topk_workspace_bytes": [_I, _I, _I],
    "csa_indexer_topk": [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, C.c_int64,
                         _P],
    "csa_sparse_mla_fwd": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P,
                           C.c_float, _P, _P, _P],
    "csa_sparse_mla_bwd_workspace_bytes": [_I, _I, _I, _P, _P, _I, _I, _I],
    "csa_sparse_mla_bwd": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P,
                           C.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, C.c_int64, _P],
    "csa_sparse_mla_bwd_deterministic_workspace_bytes": [_I, _I, _I, _I, _P, _P, _I, _I, _I],
    "csa_sparse_mla_bwd_deterministic": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _I, _I, _I, _I, _I,
                                         _I, _P, C.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, C.c_int64,
                                         _P],
    "csa_indexer_kl_grad_workspace_bytes": [_I, _I, _I, _I],
    "csa_indexer_kl_grad": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _I, _I, _I, _I, C.c_float,
                            _P, _P, _P, _P, _P, C.c_int64, _P],
    "csa_indexer_kl_grad_noalloc": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _I, _I, _I, _I,
                                    C.c_float, _P, _P, _P, _P, _P],
    "csa_validate_layout": [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P],
    "csa_validate_topk_rows": [_P, _I, _I, _I, _P, _P, _P, _I, _I, _I, _P],
}
RESTYPES = {"csa_version": C.c_char_p, "csa_last_error": C.c_char_p, "csa_sparse_mla_bwd_workspace_bytes": C.c_int64,
            "csa_sparse_mla_bwd_deterministic_workspace_bytes": C.c_int64,
            "csa_indexer_topk_workspace_bytes": C.c_int64,
            "csa_indexer_kl_grad_workspace_bytes": C.c_int64}


class CsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[csa status {code}] {msg}")
        self.code = code


def load(path: str = LIB_PATH) -> C.CDLL:
    """Open a build of the library (the product one by default; DEBUG_LIB_PATH is the
    CSA_DEBUG build) with the argument and result types of include/csa.h."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python sparse_attention_thd_amd/build.py`")
    lib = C.CDLL(path)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = RESTYPES.get(name, C.c_int)
    return lib


DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa_debug.so")
LIB = load()


def _check(code: int) -> None:
    if code != CSA_OK:
        raise CsaError(code, LIB.csa_last_error().decode())


def _ptr(t, name, dtype=None, optional=False, need=0):
    """Device pointer of `t` after checking device, layout, dtype and that it holds at
    least `need` elements (the extent the call's size arguments give it), so that a
    short tensor is refused here instead of being read or written past its end."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() < need:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {need}")
    return t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    if t.dtype == torch.float32:
        return CSA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def csa_version() -> str:
    return LIB.csa_version().decode()


def csa_last_error() -> str:
    return LIB.csa_last_error().decode()


def csa_build_indices(cu_seqlens_q, cu_seqlens_kv, B, Tq, Tkv, global_start, cmp_ratio, ori_win_left,
                      ori_win_right, q_seg, q_pos, win_idx, cu_seqlens_cmp, cmp_residual, q_cmp_lo, q_cmp_nvis,
                      cmp_group, Tc_cap, stream=None):
    i32 = torch.int32
    W = ori_win_left + ori_win_right + 1
    _check(LIB.csa_build_indices(
        _ptr(cu_seqlens_q, "cu_seqlens_q", i32, need=B + 1), _ptr(cu_seqlens_kv, "cu_seqlens_kv", i32, need=B + 1),
        B, Tq, Tkv, global_start, cmp_ratio, ori_win_left, ori_win_right,
        _ptr(q_seg, "q_seg", i32, True, Tq), _ptr(q_pos, "q_pos", i32, True, Tq),
        _ptr(win_idx, "win_idx", i32, True, Tq * W),
        _ptr(cu_seqlens_cmp, "cu_seqlens_cmp", i32, need=B + 1), _ptr(cmp_residual, "cmp_residual", i32, need=B),
        _ptr(q_cmp_lo, "q_cmp_lo", i32, True, Tq), _ptr(q_cmp_nvis, "q_cmp_nvis", i32, True, Tq),
        _ptr(cmp_group, "cmp_group", i32, True, Tc_cap), Tc_cap, _stream(stream)))


def csa_compress(x, Tkv, d, cu_seqlens_kv, cu_seqlens_cmp, B, cmp_ratio, x_cmp, Tc_cap, stream=None):
    i32 = torch.int32
    _check(LIB.csa_compress(_ptr(x, "x", need=Tkv * d), Tkv, d, _dtype_code(x),
                            _ptr(cu_seqlens_kv, "cu_seqlens_kv", i32, need=B + 1),
                            _ptr(cu_seqlens_cmp, "cu_seqlens_cmp", i32, need=B + 1), B, cmp_ratio,
                            _ptr(x_cmp, "x_cmp", x.dtype, need=Tc_cap * d), Tc_cap, _stream(stream)))


def csa_compress_learned(x, Tkv, D, wkv, wgate, ape, hd, overlap, cu_seqlens_kv, cu_seqlens_cmp, B, cmp_ratio,
                         x_cmp, Tc_cap, stream=None):
    i32 = torch.int32
    C = (2 if overlap else 1) * hd
    _check(LIB.csa_compress_learned(_ptr(x, "x", need=Tkv * D), Tkv, D, _dtype_code(x),
                                    _ptr(wkv, "wkv", x.dtype, need=C * D), _ptr(wgate, "wgate", x.dtype, need=C * D),
                                    _ptr(ape, "ape", torch.float32, need=cmp_ratio * C), hd, 1 if overlap else 0,
                                    _ptr(cu_seqlens_kv, "cu_seqlens_kv", i32, need=B + 1),
                                    _ptr(cu_seqlens_cmp, "cu_seqlens_cmp", i32, need=B + 1), B, cmp_ratio,
                                    _ptr(x_cmp, "x_cmp", x.dtype, need=Tc_cap * hd), Tc_cap, _stream(stream)))


def csa_indexer_topk_workspace_bytes(Tq, max_seqlen_kv, cmp_ratio):
    n = LIB.csa_indexer_topk_workspace_bytes(Tq, max_seqlen_kv, cmp_ratio)
    if n < 0:
        raise CsaError(CSA_EINVAL, "csa_indexer_topk_workspace_bytes: invalid arguments")
    return int(n)


def csa_indexer_topk(q_I, w, k_I_cmp, Tq, Tc, H_I, d_I, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_cmp, cmp_residual,
                     B, global_start, cmp_ratio, max_seqlen_kv, topk, topk_idx, topk_score=None, workspace=None,
                     stream=None):
    i32 = torch.int32
    dt = q_I.dtype
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.csa_indexer_topk(
        _ptr(q_I, "q_I", need=Tq * H_I * d_I), _ptr(w, "w", dt, need=Tq * H_I),
        _ptr(k_I_cmp, "k_I_cmp", dt, Tc == 0, Tc * d_I), Tq, Tc, H_I, d_I, _dtype_code(q_I),
        _ptr(cu_seqlens_q, "cu_seqlens_q", i32, need=B + 1), _ptr(cu_seqlens_kv, "cu_seqlens_kv", i32, need=B + 1),
        _ptr(cu_seqlens_cmp, "cu_seqlens_cmp", i32, need=B + 1), _ptr(cmp_residual, "cmp_residual", i32, True, B),
        B, global_start, cmp_ratio, max_seqlen_kv, topk, _ptr(topk_idx, "topk_idx", i32, need=Tq * topk),
        _ptr(topk_score, "topk_score", torch.float32, True, Tq * topk), _ptr(workspace, "workspace", optional=True),
        ws_bytes, _stream(stream)))


def csa_sparse_mla_fwd(q, ori_kv, cmp_kv, cmp_idx, topk, cmp_idx_kind, Tq, Tkv, Tc, H, d, cu_seqlens_q, cu_seqlens_kv,
                       cu_seqlens_cmp, cmp_residual, B, global_start, cmp_ratio, ori_win_left, ori_win_right, sinks,
                       softmax_scale, out, lse=None, stream=None):
    i32 = torch.int32
    dt = q.dtype
    _check(LIB.csa_sparse_mla_fwd(
        _ptr(q, "q", need=Tq * H * d), _ptr(ori_kv, "ori_kv", dt, need=Tkv * d),
        _ptr(cmp_kv, "cmp_kv", dt, True, Tc * d), _ptr(cmp_idx, "cmp_idx", i32, True, Tq * topk), topk, cmp_idx_kind,
        Tq, Tkv, Tc, H, d, _dtype_code(q),
        _ptr(cu_seqlens_q, "cu_seqlens_q", i32, need=B + 1), _ptr(cu_seqlens_kv, "cu_seqlens_kv", i32, need=B + 1),
        _ptr(cu_seqlens_cmp, "cu_seqlens_cmp", i32, True, B + 1), _ptr(cmp_residual, "cmp_residual", i32, True, B),
        B, global_start, cmp_ratio, ori_win_left, ori_win_right, _ptr(sinks, "sinks", torch.float32, True, H),
        float(softmax_scale), _ptr(out, "out", dt, need=Tq * H * d), _ptr(lse, "lse", torch.float32, True, Tq * H),
        _stream(stream)))


def csa_sparse_mla_bwd_workspace_bytes(Tq, ori_win_left, ori_win_right, cmp_kv, cmp_idx, topk, max_seqlen_kv,
                                       cmp_ratio):
    n = LIB.csa_sparse_mla_bwd_workspace_bytes(Tq, ori_win_left, ori_win_right, _ptr(cmp_kv, "cmp_kv", optional=True),
                                               _ptr(cmp_idx, "cmp_idx", torch.int32, True), topk, max_seqlen_kv,
                                               cmp_ratio)
    if n < 0:
        raise CsaError(CSA_EINVAL, "csa_sparse_mla_bwd_workspace_bytes: invalid arguments")
    return int(n)


def csa_sparse_mla_bwd_deterministic_workspace_bytes(Tq, B, ori_win_left, ori_win_right, cmp_kv, cmp_idx, topk,
                                                     max_seqlen_kv, cmp_ratio):
    n = LIB.csa_sparse_mla_bwd_deterministic_workspace_bytes(Tq, B, ori_win_left, ori_win_right,
                                                             _ptr(cmp_kv, "cmp_kv", optional=True),
                                                             _ptr(cmp_idx, "cmp_idx", torch.int32, True), topk,
                                                             max_seqlen_kv, cmp_ratio)
    if n < 0:
        raise CsaError(CSA_EINVAL, "csa_sparse_mla_bwd_deterministic_workspace_bytes: invalid arguments")
    return int(n)


def _bwd(fn, q, ori_kv, cmp_kv, cmp_idx, topk, Tq, Tkv, Tc, H, d, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_cmp, B,
         global_start, cmp_ratio, ori_win_left, ori_win_right, max_seqlen_kv, sinks, softmax_scale, out, lse, dout,
         dq, d_ori_kv, d_cmp_kv, d_sinks, ori_l1, cmp_l1, cmp_slots, workspace, stream):
    i32, f32 = torch.int32, torch.float32
    dt = q.dtype
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    nq, W = Tq * H * d, ori_win_left + ori_win_right + 1
    _check(fn(
        _ptr(q, "q", need=nq), _ptr(ori_kv, "ori_kv", dt, need=Tkv * d), _ptr(cmp_kv, "cmp_kv", dt, True, Tc * d),
        _ptr(cmp_idx, "cmp_idx", i32, True, Tq * topk), topk, Tq, Tkv, Tc, H, d, _dtype_code(q),
        _ptr(cu_seqlens_q, "cu_seqlens_q", i32, need=B + 1), _ptr(cu_seqlens_kv, "cu_seqlens_kv", i32, need=B + 1),
        _ptr(cu_seqlens_cmp, "cu_seqlens_cmp", i32, True, B + 1), B, global_start, cmp_ratio, ori_win_left,
        ori_win_right, max_seqlen_kv, _ptr(sinks, "sinks", f32, True, H), float(softmax_scale),
        _ptr(out, "out", dt, need=nq), _ptr(lse, "lse", f32, need=Tq * H), _ptr(dout, "dout", dt, need=nq),
        _ptr(dq, "dq", dt, need=nq), _ptr(d_ori_kv, "d_ori_kv", f32, need=Tkv * d),
        _ptr(d_cmp_kv, "d_cmp_kv", f32, True, Tc * d), _ptr(d_sinks, "d_sinks", f32, True, H),
        _ptr(ori_l1, "ori_l1", f32, True, Tq * W), _ptr(cmp_l1, "cmp_l1", f32, True, Tq * cmp_slots), cmp_slots,
        _ptr(workspace, "workspace", optional=True), ws_bytes, _stream(stream)))


def csa_sparse_mla_bwd(q, ori_kv, cmp_kv, cmp_idx, topk, Tq, Tkv, Tc, H, d, cu_seqlens_q, cu_seqlens_kv,
                       cu_seqlens_cmp, B, global_start, cmp_ratio, ori_win_left, ori_win_right, max_seqlen_kv,
                       sinks, softmax_scale, out, lse, dout, dq, d_ori_kv, d_cmp_kv=None, d_sinks=None,
                       ori_l1=None, cmp_l1=None, cmp_slots=0, workspace=None, stream=None):
    _bwd(LIB.csa_sparse_mla_bwd, q, ori_kv, cmp_kv, cmp_idx, topk, Tq, Tkv, Tc, H, d, cu_seqlens_q, cu_seqlens_kv,
         cu_seqlens_cmp, B, global_start, cmp_ratio, ori_win_left, ori_win_right, max_seqlen_kv, sinks, softmax_scale,
         out, lse, dout, dq, d_ori_kv, d_cmp_kv, d_sinks, ori_l1, cmp_l1, cmp_slots, workspace, stream)


def csa_sparse_mla_bwd_deterministic(q, ori_kv, cmp_kv, cmp_idx, topk, Tq, Tkv, Tc, H, d, cu_seqlens_q,
                                     cu_seqlens_kv, cu_seqlens_cmp, B, global_start, cmp_ratio, ori_win_left,
                                     ori_win_right, max_seqlen_kv, sinks, softmax_scale, out, lse, dout, dq, d_ori_kv,
                                     d_cmp_kv=None, d_sinks=None, ori_l1=None, cmp_l1=None, cmp_slots=0,
                                     workspace=None, stream=None):
    _bwd(LIB.csa_sparse_mla_bwd_deterministic, q, ori_kv, cmp_kv, cmp_idx, topk, Tq, Tkv, Tc, H, d, cu_seqlens_q,
         cu_seqlens_kv, cu_seqlens_cmp, B, global_start, cmp_ratio, ori_win_left, ori_win_right, max_seqlen_kv, sinks,
         softmax_scale, out, lse, dout, dq, d_ori_kv, d_cmp_kv, d_sinks, ori_l1, cmp_l1, cmp_slots, workspace, stream)


def csa_indexer_kl_grad_workspace_bytes(Tq, topk, max_seqlen_kv, cmp_ratio):
    n = LIB.csa_indexer_kl_grad_workspace_bytes(Tq, topk, max_seqlen_kv, cmp_ratio)
    if n < 0:
        raise CsaError(CSA_EINVAL, "csa_indexer_kl_grad_workspace_bytes: invalid arguments")
    return int(n)


def csa_indexer_kl_grad(q_I, w, k_I_cmp, cmp_idx, attn_l1, topk, Tq, Tc, H_I, d_I, cu_seqlens_q, cu_seqlens_kv,
                        cu_seqlens_cmp, B, global_start, cmp_ratio, max_seqlen_kv, loss_scale, d_q_I, d_w,
                        d_k_I_cmp, loss=None, workspace=None, stream=None):
    i32, f32 = torch.int32, torch.float32
    dt = q_I.dtype
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    nq = Tq * H_I * d_I
    _check(LIB.csa_indexer_kl_grad(
        _ptr(q_I, "q_I", need=nq), _ptr(w, "w", dt, need=Tq * H_I), _ptr(k_I_cmp, "k_I_cmp", dt, True, Tc * d_I),
        _ptr(cmp_idx, "cmp_idx", i32, need=Tq * topk), _ptr(attn_l1, "attn_l1", f32, need=Tq * topk), topk, Tq, Tc,
        H_I, d_I, _dtype_code(q_I), _ptr(cu_seqlens_q, "cu_seqlens_q", i32, need=B + 1),
        _ptr(cu_seqlens_kv, "cu_seqlens_kv", i32, need=B + 1), _ptr(cu_seqlens_cmp, "cu_seqlens_cmp", i32, need=B + 1),
        B, global_start, cmp_ratio, max_seqlen_kv, float(loss_scale), _ptr(d_q_I, "d_q_I", dt, need=nq),
        _ptr(d_w, "d_w", f32, need=Tq * H_I), _ptr(d_k_I_cmp, "d_k_I_cmp", f32, True, Tc * d_I),
        _ptr(loss, "loss", f32, True, Tq), _ptr(workspace, "workspace", optional=True), ws_bytes, _stream(stream)))


def csa_indexer_kl_grad_noalloc(q_I, w, k_I_cmp, cmp_idx, attn_l1, topk, Tq, Tc, H_I, d_I, cu_seqlens_q,
                                cu_seqlens_kv, cu_seqlens_cmp, B, global_start, cmp_ratio, max_seqlen_kv, loss_scale,
                                d_q_I, d_w, d_k_I_cmp, loss=None, stream=None):
    i32, f32 = torch.int32, torch.float32
    dt = q_I.dtype
    nq = Tq * H_I * d_I
    _check(LIB.csa_indexer_kl_grad_noalloc(
        _ptr(q_I, "q_I", need=nq), _ptr(w, "w", dt, need=Tq * H_I), _ptr(k_I_cmp, "k_I_cmp", dt, True, Tc * d_I),
        _ptr(cmp_idx, "cmp_idx", i32, need=Tq * topk), _ptr(attn_l1, "attn_l1", f32, need=Tq * topk), topk, Tq, Tc,
        H_I, d_I, _dtype_code(q_I), _ptr(cu_seqlens_q, "cu_seqlens_q", i32, need=B + 1),
        _ptr(cu_seqlens_kv, "cu_seqlens_kv", i32, need=B + 1), _ptr(cu_seqlens_cmp, "cu_seqlens_cmp", i32, need=B + 1),
        B, global_start, cmp_ratio, max_seqlen_kv, float(loss_scale), _ptr(d_q_I, "d_q_I", dt, need=nq),
        _ptr(d_w, "d_w", f32, need=Tq * H_I), _ptr(d_k_I_cmp, "d_k_I_cmp", f32, True, Tc * d_I),
        _ptr(loss, "loss", f32, True, Tq), _stream(stream)))


def csa_validate_layout(cu_seqlens_q, cu_seqlens_kv, B, Tq, Tkv, global_start, max_seqlen_kv=-1, cmp_ratio=0,
                        cu_seqlens_cmp=None, cmp_residual=None, stream=None):
    i32 = torch.int32
    _check(LIB.csa_validate_layout(_ptr(cu_seqlens_q, "cu_seqlens_q", i32, need=B + 1),
                                   _ptr(cu_seqlens_kv, "cu_seqlens_kv", i32, need=B + 1), B, Tq, Tkv, global_start,
                                   max_seqlen_kv, cmp_ratio,
                                   _ptr(cu_seqlens_cmp, "cu_seqlens_cmp", i32, True, B + 1),
                                   _ptr(cmp_residual, "cmp_residual", i32, True, B), _stream(stream)))


def csa_validate_topk_rows(cmp_idx, topk, Tq, Tc, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_cmp, B, global_start,
                           cmp_ratio, stream=None):
    i32 = torch.int32
    _check(LIB.csa_validate_topk_rows(
        _ptr(cmp_idx, "cmp_idx", i32, Tq == 0, Tq * topk), topk, Tq, Tc,
        _ptr(cu_seqlens_q, "cu_seqlens_q", i32, need=B + 1), _ptr(cu_seqlens_kv, "cu_seqlens_kv", i32, need=B + 1),
        _ptr(cu_seqlens_cmp, "cu_seqlens_cmp", i32, need=B + 1), B, global_start, cmp_ratio, _stream(stream)))
