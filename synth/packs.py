"""Synthetic THD workloads shaped like the pages' DeepSeek-V4 CSA runs.

Recipe (fixed draw order per seed, numpy PCG64 ``default_rng(seed)``):
segment lengths first, then q, ori_kv, q_I, k_I, w, sinks.  Every tensor is drawn
as float32 ``standard_normal``, multiplied by its scale in float32 and, for bf16
workloads, rounded once to bfloat16 (round to nearest, ties to even).  Sinks stay
float32.  Large tensors are drawn in chunks; numpy's generator yields the same
stream either way.

Workloads (geometry of the DeepSeek-V4 CSA pages: one shared 512-wide latent KV
row per token, 64 query heads, a 64x128 lightning indexer, cmp_ratio 4 or 128,
a 128-token window, top-512):

* ``tiny``      fp32, cu_seqlens [0,37,128], 4 heads, d 64, ratio 4, window 16,
                indexer 2x32, top-8.
* ``single4k``  one 4096-token segment, bf16.
* ``pack16k``   16384 tokens, lognormal(7,1) lengths clipped to [17,8192],
                never a multiple of 4.
* ``hca32k``    8 segments uniform in [1024,7000] summing to 32768, ratio 128,
                no indexer.
* ``cp32k``     one context-parallel share of a 131072-token stream
                (lognormal(9,0.8) lengths): local queries are stream rows
                [65536, 98304), KV is the prefix [0, 98304).
* ``stress``    single4k's shape with q and kv ~ N(0,1): peaky softmax.

Learned-compressor inputs (``compressor_inputs``, its own stream
``default_rng([seed, 7])``, drawn x, wkv, wgate, ape in that order): hidden rows
x [Tkv, D] ~ N(0,1), projections wkv, wgate [C, D] ~ N(0,1)/sqrt(D) (wgate times
``gate_scale``), C = 2 hd with overlap else hd, and the position table
ape [r, C] ~ N(0,1) * ``ape_scale`` in float32.  The pages do not give the model's
hidden size; D = 4096 is this workload's choice.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

_CHUNK = 1 << 24


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return raw uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Decode raw bfloat16 bits (uint16) to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(rng, shape, scale, bf16):
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    s = np.float32(scale)
    for a in range(0, n, _CHUNK):
        m = min(_CHUNK, n - a)
        v = rng.standard_normal(m, dtype=np.float32)
        if scale != 1.0:
            v = v * s
        out[a:a + m] = f32_to_bf16_bits(v) if bf16 else v
    return out.reshape(shape)


def _lengths_pack16k(rng, total=16384):
    L, s = [], 0
    while s < total:
        n = int(np.clip(round(rng.lognormal(7.0, 1.0)), 17, 8192))
        if n % 4 == 0:
            n -= 1
        L.append(n)
        s += n
    L[-1] = total - sum(L[:-1])
    while L[-1] < 17 or L[-1] % 4 == 0 or L[-2] % 4 == 0:
        L[-2] -= 1
        L[-1] += 1
    return L


def _lengths_hca32k(rng, total=32768):
    while True:
        L = [int(v) for v in rng.integers(1024, 7001, size=7)]
        last = total - sum(L)
        if 1024 <= last <= 7000:
            return L + [last]


def _lengths_cp(rng, total=131072, cuts=(65536, 98304)):
    L, s = [], 0
    while s < total:
        n = int(np.clip(round(rng.lognormal(9.0, 0.8)), 17, total))
        L.append(n)
        s += n
    L[-1] = total - sum(L[:-1])
    # every cut must fall strictly inside a segment
    for cut in cuts:
        while True:
            bounds = np.cumsum(L)[:-1]
            hit = np.nonzero(bounds == cut)[0]
            if hit.size == 0:
                break
            b = int(hit[0])
            if L[b + 1] > 1:
                L[b + 1] -= 1
                L[b] += 1
            else:
                L[b] -= 1
                L[b + 1] += 1
    return L


@dataclasses.dataclass
class Pack:
    """One synthetic workload.  bf16 tensors are uint16 bit arrays, fp32 ones float32."""
    name: str
    dtype: str                      # "bf16" or "f32"
    cu_seqlens_q: np.ndarray        # int32 [B+1] local query rows per segment
    cu_seqlens_kv: np.ndarray       # int32 [B+1] stream rows (truncated at the KV prefix end)
    global_start: int
    Tq: int
    Tkv: int
    H: int
    d: int
    H_I: int
    d_I: int
    cmp_ratio: int
    ori_win_left: int
    ori_win_right: int
    topk: int
    softmax_scale: float
    q: np.ndarray                   # [Tq, H, d]
    ori_kv: np.ndarray              # [Tkv, d]
    q_I: np.ndarray | None          # [Tq, H_I, d_I]
    k_I: np.ndarray | None          # [Tkv, d_I]
    w: np.ndarray | None            # [Tq, H_I]
    sinks: np.ndarray               # float32 [H]
    seed: int = 0

    @property
    def B(self) -> int:
        return len(self.cu_seqlens_kv) - 1

    @property
    def max_seqlen_kv(self) -> int:
        return int(np.diff(self.cu_seqlens_kv).max()) if self.B > 0 else 0

    @property
    def has_indexer(self) -> bool:
        return self.q_I is not None

    def f32(self, name: str) -> np.ndarray:
        """A tensor decoded to float32 (exact for bf16)."""
        a = getattr(self, name)
        return bf16_bits_to_f32(a) if (self.dtype == "bf16" and a.dtype == np.uint16) else a


def pack_from_lengths(name, lengths, *, seed=0, dtype="bf16", H=64, d=512, H_I=64, d_I=128,
                      cmp_ratio=4, ori_win_left=127, ori_win_right=0, topk=512,
                      q_scale=None, kv_scale=None, qI_scale=1.0, kI_scale=1.0, w_scale=1.0 / 8,
                      softmax_scale=None, indexer=True, q_rows=None, kv_rows=None, rng=None):
    """Draw tensors for a THD pack with the given segment lengths.

    ``q_rows=(a, b)`` keeps local queries for stream rows [a, b) (a context-parallel
    share); ``kv_rows`` truncates KV at that prefix end.  Defaults: the whole stream.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    bf16 = dtype == "bf16"
    total = int(np.sum(lengths))
    a, b = q_rows if q_rows is not None else (0, total)
    kv_end = kv_rows if kv_rows is not None else total
    assert 0 <= a <= b <= kv_end <= total
    cu_q, cu_kv, a, Tq, Tkv = _segments(lengths, q_rows, kv_rows)
    if q_scale is None:
        q_scale = 1.0 / math.sqrt(d)
    if kv_scale is None:
        kv_scale = 1.0 / math.sqrt(d)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    q = _draw(rng, (Tq, H, d), q_scale, bf16)
    ori_kv = _draw(rng, (Tkv, d), kv_scale, bf16)
    q_I = k_I = w = None
    if indexer:
        q_I = _draw(rng, (Tq, H_I, d_I), qI_scale, bf16)
        k_I = _draw(rng, (Tkv, d_I), kI_scale, bf16)
        w = _draw(rng, (Tq, H_I), w_scale, bf16)
    sinks = rng.standard_normal(H, dtype=np.float32)
    return Pack(name=name, dtype=dtype, cu_seqlens_q=cu_q, cu_seqlens_kv=cu_kv, global_start=int(a), Tq=int(Tq),
                Tkv=int(Tkv),
                H=H, d=d, H_I=H_I if indexer else 0, d_I=d_I if indexer else 0, cmp_ratio=cmp_ratio,
                ori_win_left=ori_win_left, ori_win_right=ori_win_right, topk=topk,
                softmax_scale=float(softmax_scale), q=q, ori_kv=ori_kv, q_I=q_I, k_I=k_I, w=w,
                sinks=sinks, seed=seed)


@dataclasses.dataclass
class Layout:
    """The THD layout and geometry of a workload, without its tensors (for callers that
    draw the tensors elsewhere, e.g. on the device, with the same scales)."""
    name: str
    cu_seqlens_q: np.ndarray
    cu_seqlens_kv: np.ndarray
    global_start: int
    Tq: int
    Tkv: int
    H: int = 64
    d: int = 512
    H_I: int = 64
    d_I: int = 128
    cmp_ratio: int = 4
    ori_win_left: int = 127
    ori_win_right: int = 0
    topk: int = 512
    q_scale: float = 512 ** -0.5
    kv_scale: float = 512 ** -0.5
    w_scale: float = 1.0 / 8
    softmax_scale: float = 512 ** -0.5
    indexer: bool = True

    @property
    def B(self) -> int:
        return len(self.cu_seqlens_kv) - 1


def _segments(lengths, q_rows=None, kv_rows=None):
    """cu_seqlens_q, cu_seqlens_kv, global_start, Tq, Tkv of a pack: segments that start
    before the KV prefix end, truncated at it; local query rows per segment."""
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    total = int(cu[-1])
    a, b = q_rows if q_rows is not None else (0, total)
    kv_end = kv_rows if kv_rows is not None else total
    nb = int(np.searchsorted(cu, kv_end, side="left"))
    nb = max(nb, 1) if kv_end > 0 else 1
    cu_kv = np.minimum(cu[:nb + 1], kv_end)
    if len(cu_kv) < 2:
        cu_kv = np.array([0, kv_end])
    cu_q = np.clip(cu_kv - a, 0, b - a)
    return cu_q.astype(np.int32), cu_kv.astype(np.int32), int(a), int(b - a), int(kv_end)


def workload_layout(name: str, seed: int = 0) -> Layout:
    """Layout of one of the bf16 workloads below (single4k, pack16k, hca32k, cp32k),
    drawn from the same generator stream as make_pack (segment lengths come first)."""
    rng = np.random.default_rng(seed)
    kw = {}
    if name == "single4k":
        seg = _segments([4096])
    elif name == "pack16k":
        seg = _segments(_lengths_pack16k(rng))
    elif name == "hca32k":
        seg = _segments(_lengths_hca32k(rng))
        kw = dict(cmp_ratio=128, indexer=False, H_I=0, d_I=0)
    elif name == "cp32k":
        seg = _segments(_lengths_cp(rng), q_rows=(65536, 98304), kv_rows=98304)
    else:
        raise KeyError(name)
    cu_q, cu_kv, gs, Tq, Tkv = seg
    return Layout(name=name, cu_seqlens_q=cu_q, cu_seqlens_kv=cu_kv, global_start=gs, Tq=Tq, Tkv=Tkv, **kw)


def _tiny(seed):
    return pack_from_lengths("tiny", [37, 91], seed=seed, dtype="f32", H=4, d=64, H_I=2, d_I=32,
                             cmp_ratio=4, ori_win_left=15, topk=8, q_scale=1.0, kv_scale=1.0,
                             w_scale=1.0 / math.sqrt(2), softmax_scale=1.0 / 8)


def _single4k(seed):
    return pack_from_lengths("single4k", [4096], seed=seed)


def _pack16k(seed):
    rng = np.random.default_rng(seed)
    return pack_from_lengths("pack16k", _lengths_pack16k(rng), seed=seed, rng=rng)


def _hca32k(seed):
    rng = np.random.default_rng(seed)
    return pack_from_lengths("hca32k", _lengths_hca32k(rng), seed=seed, rng=rng, cmp_ratio=128,
                             indexer=False)


def _cp32k(seed):
    rng = np.random.default_rng(seed)
    return pack_from_lengths("cp32k", _lengths_cp(rng), seed=seed, rng=rng,
                             q_rows=(65536, 98304), kv_rows=98304)


def _stress(seed):
    return pack_from_lengths("stress", [4096], seed=seed, q_scale=1.0, kv_scale=1.0)


CONFIGS = {
    "tiny": _tiny,
    "single4k": _single4k,
    "pack16k": _pack16k,
    "hca32k": _hca32k,
    "cp32k": _cp32k,
    "stress": _stress,
}


@dataclasses.dataclass
class CompressorInputs:
    x: np.ndarray        # [Tkv, D] bf16 bits
    wkv: np.ndarray      # [C, D] bf16 bits
    wgate: np.ndarray    # [C, D] bf16 bits
    ape: np.ndarray      # [r, C] float32
    D: int
    hd: int
    overlap: bool
    cmp_ratio: int


def compressor_inputs(Tkv, *, D=4096, hd=512, overlap=True, cmp_ratio=4, seed=0, gate_scale=1.0, ape_scale=1.0):
    rng = np.random.default_rng([seed, 7])
    C = 2 * hd if overlap else hd
    x = _draw(rng, (Tkv, D), 1.0, True)
    wkv = _draw(rng, (C, D), 1.0 / math.sqrt(D), True)
    wgate = _draw(rng, (C, D), gate_scale / math.sqrt(D), True)
    ape = rng.standard_normal((cmp_ratio, C), dtype=np.float32) * np.float32(ape_scale)
    return CompressorInputs(x=x, wkv=wkv, wgate=wgate, ape=ape, D=D, hd=hd, overlap=overlap, cmp_ratio=cmp_ratio)


def make_pack(name: str, seed: int = 0) -> Pack:
    return CONFIGS[name](seed)
