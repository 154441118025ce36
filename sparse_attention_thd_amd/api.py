"""Whole CSA forward on a THD pack, composed from the four C-ABI calls.

``CsaPlan`` allocates every intermediate once for a fixed layout and shape (torch
device memory) and ``run`` enqueues the calls on the current stream:

    csa_build_indices -> csa_compress (latent KV) -> csa_compress (indexer keys)
    -> csa_indexer_topk -> csa_sparse_mla_fwd

The compressed branch follows the layer's compression mode (page "MindSpeed-LLM
pull 4842", 主要改动, LayerCompressMode): ratio 4 runs the lightning indexer,
another ratio above 1 attends every causally complete compressed row, ratio 1
(or a pack whose segments are all shorter than the ratio) keeps only the window.

Compressed rows are the segment-local mean of r rows by default; ``run`` can take
``LearnedCompressor`` parameters instead (the gated overlapping compressor of page
"PR #2038 完整报告", 关键源码片段 compressor.py), computed from the hidden rows ``x``
with csa_compress_learned, for the latent rows, the indexer keys, or both.
"""
from __future__ import annotations

import dataclasses
import enum

import torch

from . import _lib


class LayerCompressMode(enum.IntEnum):
    NO_COMPRESS = 0
    COMPRESSOR_ONLY = 1
    INDEXER = 2


def layer_compress_mode(cmp_ratio: int) -> LayerCompressMode:
    if cmp_ratio <= 1:
        return LayerCompressMode.NO_COMPRESS
    if cmp_ratio == 4:
        return LayerCompressMode.INDEXER
    return LayerCompressMode.COMPRESSOR_ONLY


@dataclasses.dataclass
class LearnedCompressor:
    """Parameters of one learned compressor: wkv, wgate [C, D] (call dtype), ape [r, C] float32,
    C = 2 * hd with overlap, hd otherwise."""
    wkv: torch.Tensor
    wgate: torch.Tensor
    ape: torch.Tensor
    overlap: bool = True

    def hd(self) -> int:
        C = int(self.wkv.shape[0])
        return C // 2 if self.overlap else C

    def run(self, x, layout, cu_seqlens_cmp, cmp_ratio, out, Tc_cap, stream=None):
        _lib.csa_compress_learned(x, layout.Tkv, int(x.shape[1]), self.wkv, self.wgate, self.ape, self.hd(),
                                  self.overlap, layout.cu_seqlens_kv, cu_seqlens_cmp, layout.B, cmp_ratio, out, Tc_cap,
                                  stream)


@dataclasses.dataclass
class ThdLayout:
    """THD layout of one call: int32 device prefix sums plus the host sizes that shape the grids."""
    cu_seqlens_q: torch.Tensor
    cu_seqlens_kv: torch.Tensor
    Tq: int
    Tkv: int
    global_start: int
    max_seqlen_kv: int

    @property
    def B(self) -> int:
        return int(self.cu_seqlens_kv.numel()) - 1

    @classmethod
    def from_host(cls, cu_seqlens_q, cu_seqlens_kv, global_start=0, device="cuda"):
        cq = torch.as_tensor(cu_seqlens_q, dtype=torch.int32)
        ck = torch.as_tensor(cu_seqlens_kv, dtype=torch.int32)
        L = (ck[1:] - ck[:-1])
        return cls(cq.to(device), ck.to(device), int(cq[-1]), int(ck[-1]), int(global_start),
                   int(L.max()) if L.numel() else 0)


class CsaPlan:
    """Buffers and launch sequence for one layout and one geometry."""

    def __init__(self, layout: ThdLayout, *, H: int, d: int, H_I: int = 0, d_I: int = 0, cmp_ratio: int = 4,
                 ori_win_left: int = 127, ori_win_right: int = 0, topk: int = 512, softmax_scale: float | None = None,
                 dtype=torch.bfloat16, emit_window: bool = True, return_lse: bool = False,
                 return_topk_score: bool = False, mode: LayerCompressMode | None = None):
        self.L = layout
        self.H, self.d, self.H_I, self.d_I = H, d, H_I, d_I
        self.r, self.wl, self.wr, self.topk = cmp_ratio, ori_win_left, ori_win_right, topk
        self.scale = softmax_scale if softmax_scale is not None else d ** -0.5
        self.dtype = dtype
        self.mode = layer_compress_mode(cmp_ratio) if mode is None else mode
        dev = layout.cu_seqlens_kv.device
        Tq, Tkv, B = layout.Tq, layout.Tkv, layout.B
        i32 = dict(dtype=torch.int32, device=dev)
        self.Tc_cap = max(Tkv // cmp_ratio, 1)
        W = ori_win_left + ori_win_right + 1
        self.q_seg = torch.empty(Tq, **i32)
        self.q_pos = torch.empty(Tq, **i32)
        self.win_idx = torch.empty((Tq, W), **i32) if emit_window else None
        self.cu_seqlens_cmp = torch.zeros(B + 1, **i32)
        self.cmp_residual = torch.zeros(B, **i32)
        self.q_cmp_lo = torch.empty(Tq, **i32)
        self.q_cmp_nvis = torch.empty(Tq, **i32)
        self.cmp_group = torch.full((self.Tc_cap,), -1, **i32)
        self.cmp_kv = self.k_I_cmp = self.topk_idx = self.topk_score = self.indexer_ws = None
        if self.mode != LayerCompressMode.NO_COMPRESS:
            self.cmp_kv = torch.zeros((self.Tc_cap, d), dtype=dtype, device=dev)
        if self.mode == LayerCompressMode.INDEXER:
            self.k_I_cmp = torch.zeros((self.Tc_cap, d_I), dtype=dtype, device=dev)
            self.topk_idx = torch.empty((Tq, topk), **i32)
            nb = _lib.csa_indexer_topk_workspace_bytes(Tq, layout.max_seqlen_kv, cmp_ratio)
            self.indexer_ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
            if return_topk_score:
                self.topk_score = torch.empty((Tq, topk), dtype=torch.float32, device=dev)
        self.out = torch.empty((Tq, H, d), dtype=dtype, device=dev)
        self.lse = torch.empty((Tq, H), dtype=torch.float32, device=dev) if return_lse else None

    def run(self, q, ori_kv, sinks=None, q_I=None, k_I=None, w=None, stream=None, x=None,
            kv_compressor: LearnedCompressor | None = None, key_compressor: LearnedCompressor | None = None):
        """Enqueue the forward.  With ``kv_compressor`` / ``key_compressor`` the compressed
        latent rows / indexer keys come from the hidden rows ``x`` [Tkv, D] through the
        learned compressor instead of the mean of ori_kv / k_I."""
        L = self.L
        if (kv_compressor is not None or key_compressor is not None) and x is None:
            raise ValueError("a learned compressor needs the hidden rows x")
        for comp, width, name in ((kv_compressor, self.d, "kv_compressor"), (key_compressor, self.d_I, "key_compressor")):
            if comp is not None and comp.hd() != width:
                raise ValueError(f"{name} produces {comp.hd()} channels, the plan needs {width}")
        _lib.csa_build_indices(L.cu_seqlens_q, L.cu_seqlens_kv, L.B, L.Tq, L.Tkv, L.global_start, self.r, self.wl,
                               self.wr, self.q_seg, self.q_pos, self.win_idx, self.cu_seqlens_cmp, self.cmp_residual,
                               self.q_cmp_lo, self.q_cmp_nvis, self.cmp_group, self.Tc_cap, stream)
        if self.cmp_kv is not None:
            if kv_compressor is not None:
                kv_compressor.run(x, L, self.cu_seqlens_cmp, self.r, self.cmp_kv, self.Tc_cap, stream)
            else:
                _lib.csa_compress(ori_kv, L.Tkv, self.d, L.cu_seqlens_kv, self.cu_seqlens_cmp, L.B, self.r,
                                  self.cmp_kv, self.Tc_cap, stream)
        cmp_idx = None
        if self.mode == LayerCompressMode.INDEXER:
            if key_compressor is not None:
                key_compressor.run(x, L, self.cu_seqlens_cmp, self.r, self.k_I_cmp, self.Tc_cap, stream)
            else:
                _lib.csa_compress(k_I, L.Tkv, self.d_I, L.cu_seqlens_kv, self.cu_seqlens_cmp, L.B, self.r,
                                  self.k_I_cmp, self.Tc_cap, stream)
            _lib.csa_indexer_topk(q_I, w, self.k_I_cmp, L.Tq, self.Tc_cap, self.H_I, self.d_I, L.cu_seqlens_q,
                                  L.cu_seqlens_kv, self.cu_seqlens_cmp, self.cmp_residual, L.B, L.global_start, self.r,
                                  L.max_seqlen_kv, self.topk, self.topk_idx, self.topk_score, self.indexer_ws, stream)
            cmp_idx = self.topk_idx
        _lib.csa_sparse_mla_fwd(q, ori_kv, self.cmp_kv, cmp_idx, self.topk if cmp_idx is not None else 0,
                                _lib.CSA_IDX_TOPK, L.Tq, L.Tkv, self.Tc_cap if self.cmp_kv is not None else 0, self.H,
                                self.d, L.cu_seqlens_q, L.cu_seqlens_kv, self.cu_seqlens_cmp, self.cmp_residual, L.B,
                                L.global_start, self.r, self.wl, self.wr, sinks, self.scale, self.out, self.lse, stream)
        return self.out


def csa_forward(q, ori_kv, *, cu_seqlens_q, cu_seqlens_kv, global_start=0, sinks=None, q_I=None, k_I=None, w=None,
                cmp_ratio=4, ori_win_left=127, ori_win_right=0, topk=512, softmax_scale=None, return_lse=False):
    """Functional form: one plan, one run.  Returns (out, plan) so callers can read intermediates."""
    layout = ThdLayout.from_host(cu_seqlens_q, cu_seqlens_kv, global_start, device=q.device)
    H, d = q.shape[1], q.shape[2]
    H_I, d_I = (q_I.shape[1], q_I.shape[2]) if q_I is not None else (0, 0)
    plan = CsaPlan(layout, H=H, d=d, H_I=H_I, d_I=d_I, cmp_ratio=cmp_ratio, ori_win_left=ori_win_left,
                   ori_win_right=ori_win_right, topk=topk, softmax_scale=softmax_scale, dtype=q.dtype,
                   return_lse=return_lse, mode=None if q_I is not None or cmp_ratio != 4 else
                   LayerCompressMode.COMPRESSOR_ONLY)
    out = plan.run(q, ori_kv, sinks=sinks, q_I=q_I, k_I=k_I, w=w)
    return out, plan
