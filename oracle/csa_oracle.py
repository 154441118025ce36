"""Plain fp64 CPU oracle of the DeepSeek-V4 CSA forward on a THD-packed stream.

TEST INFRASTRUCTURE: imported only by ``tests/``, ``__graft_entry__.smoke`` and the
CPU-baseline leg of ``bench.py``.  Slow on purpose: per-query Python loops, numpy
float64 arithmetic, no blocking, fusion or reordering beyond the definitions.

Pages cited (by title; section names as they appear on the page):

* [MS]  "MindSpeed-LLM pull 4842" (DeepSeek-V4 TND context parallelism with
        prefix KV), sections 变更摘要 / 主要改动.
* [MI]  "PR #2038 完整报告: Enable THD packed-sequence training for
        DeepSeek-V4-Flash, with context parallelism", sections 功能与动机,
        实现拆解, 关键源码片段 (thd_utils.py, deepseek_v4.py, compressor.py),
        风险与影响.
* [HP]  "【RFC】DeepSeek-V4 CSA/HCA 自定义算子接入与对外接口对标 torch_extension",
        sections 背景, 1. npu_lightning_indexer, 2. npu_sparse_flash_mla,
        3. npu_sparse_lightning_indexer_kl_loss_grad, 4. npu_sparse_flash_mla_grad,
        缺失入参的用途分析（对照实验）.
* [ML]  "feat(deepseek_v4): faithful THD context-parallel path for DS4 CSA
        (bounded activation memory)", sections What, Design, GPU verification.

Notation.  Local query row i (0 <= i < Tq) is stream row t = global_start + i and
belongs to segment b with cu_seqlens_q[b] <= i < cu_seqlens_q[b+1].  Segment b
spans stream rows [s_b, e_b) = [cu_seqlens_kv[b], cu_seqlens_kv[b+1]).  The
segment-local position is p = t - s_b.  r = cmp_ratio.

Readings taken where the pages leave a step open (each is listed in the
design notes with its support):

* window: W = ori_win_left + ori_win_right + 1 slots; lo = max(s_b, t - left),
  hi = min(e_b - 1, t + right); slots past hi hold -1.
* compressed row j of segment b pools stream rows s_b + j*r + [0, r) by their
  arithmetic mean; the len % r tail forms no row.  Stored in the call dtype.
* compressed row j is visible at position p iff it is causally complete,
  (j+1)*r - 1 <= p, i.e. nvis = floor((p+1)/r).
* indexer score = sum_h w[h] * relu(<q_I[h], k_cmp>), no extra scale; ties keep
  the lower row; result rows ascending, padded with -1.
* one joint softmax over window rows, selected compressed rows and a per-head
  sink logit (not scaled by softmax_scale) with a zero value; K = V = the latent row.

Backward (sparse_mla_bwd): the exact gradients of that forward for a given dout,
with K = V, so a latent row's gradient is its key gradient plus its value gradient;
the sink receives -sum_i p_sink * D.  The two "softmax_l1_norm" outputs are the
attention probabilities averaged over the heads, per (query, key slot): window
slot k is stream row lo + k (win_idx order), compressed slot j is the j-th attended
compressed row in the order the forward lists them; unused slots hold 0.

Indexer KL loss (indexer_kl_grad): KL(p^ || softmax(I)) over a query's selected
compressed rows, p^ the main attention's head-averaged probabilities at those
slots renormalised to sum 1; gradients through I = sum_h w relu(<q_I, k>), with
relu'(0) = 0.

Every function is pinned in ``tests/test_oracle_pins.py`` (and the backward, KL
and learned-compressor pin files); a window with a right side (``ori_win_right > 0``,
clamped at the segment end) is pinned against torch's masked attention per segment.
"""
from __future__ import annotations

import math

import numpy as np

NO_COMPRESS = 0
COMPRESSOR_ONLY = 1
INDEXER = 2


def layer_compress_mode(cmp_ratio: int, n_compressed_rows: int | None = None) -> int:
    """[MS] 主要改动, first bullet: ratio 4 runs the indexer, any other ratio > 1
    attends every compressed row (compressor only), ratio 1 or a compressor that
    produced nothing means no compressed branch."""
    if cmp_ratio <= 1 or n_compressed_rows == 0:
        return NO_COMPRESS
    if cmp_ratio == 4:
        return INDEXER
    return COMPRESSOR_ONLY


# --------------------------------------------------------------------------- layout

def segment_table(cu_seqlens_kv, cmp_ratio):
    """Per-segment compressed prefix sums, tail counts and per-row group ids.

    [MI] 关键源码片段 compressor.py (_forward_thd): each segment yields
    floor(len / r) compressed rows, prefix-summed over segments; the len % r tail
    tokens produce none ([MI] 风险与影响, item 2; [HP] 背景, item 1 calls that count
    cmp_residual).  Row c of segment b has segment-local group id c - cu_cmp[b].
    """
    cu = [int(v) for v in cu_seqlens_kv]
    r = int(cmp_ratio)
    B = len(cu) - 1
    cu_cmp = [0]
    residual = []
    group = []
    for b in range(B):
        n = cu[b + 1] - cu[b]
        nc = n // r
        residual.append(n - nc * r)
        group.extend(range(nc))
        cu_cmp.append(cu_cmp[-1] + nc)
    return (np.array(cu_cmp, dtype=np.int64), np.array(residual, dtype=np.int64),
            np.array(group, dtype=np.int64))


def query_table(cu_seqlens_q, cu_seqlens_kv, global_start, Tq, cmp_ratio,
                ori_win_left, ori_win_right, cu_cmp):
    """Per-query segment, restarted position, window indices and visible compressed range.

    [MI] 功能与动机: the window clamps to the start of the query's own segment
    (not stream row 0), rotary positions restart at every segment, the indexer
    scores only the query's own segment.  [MI] 关键源码片段 thd_utils.py
    (get_window_topk_idxs_thd): stream-absolute slot k holds start + k, or -1 once
    past the query row; a context-parallel rank's rows begin at global_start.
    """
    cu_q = [int(v) for v in cu_seqlens_q]
    cu_kv = [int(v) for v in cu_seqlens_kv]
    r = int(cmp_ratio)
    W = int(ori_win_left) + int(ori_win_right) + 1
    q_seg = np.empty(Tq, dtype=np.int64)
    q_pos = np.empty(Tq, dtype=np.int64)
    win_idx = np.full((Tq, W), -1, dtype=np.int64)
    q_cmp_lo = np.empty(Tq, dtype=np.int64)
    q_cmp_nvis = np.empty(Tq, dtype=np.int64)
    b = 0
    for i in range(Tq):
        while not (cu_q[b] <= i < cu_q[b + 1]):
            b += 1
        t = int(global_start) + i
        s, e = cu_kv[b], cu_kv[b + 1]
        if not (s <= t < e):
            raise ValueError(f"query row {i} (stream row {t}) is outside its segment [{s},{e})")
        p = t - s
        lo = max(s, t - int(ori_win_left))
        hi = min(e - 1, t + int(ori_win_right))
        for k in range(W):
            if lo + k <= hi:
                win_idx[i, k] = lo + k
        q_seg[i] = b
        q_pos[i] = p
        q_cmp_lo[i] = cu_cmp[b]
        q_cmp_nvis[i] = (p + 1) // r
    return dict(q_seg=q_seg, q_pos=q_pos, win_idx=win_idx, q_cmp_lo=q_cmp_lo, q_cmp_nvis=q_cmp_nvis)


def build_indices(cu_seqlens_q, cu_seqlens_kv, global_start, Tq, cmp_ratio, ori_win_left, ori_win_right):
    """All index tensors of the layout step (the same set the library's first call emits)."""
    cu_cmp, residual, group = segment_table(cu_seqlens_kv, cmp_ratio)
    out = query_table(cu_seqlens_q, cu_seqlens_kv, global_start, Tq, cmp_ratio,
                      ori_win_left, ori_win_right, cu_cmp)
    out.update(cu_seqlens_cmp=cu_cmp, cmp_residual=residual, cmp_group=group)
    return out


# --------------------------------------------------------------------------- rounding

def round_to_bf16(x):
    """Round float64 values to the nearest bfloat16 value (ties to even), returned as float64.

    Written from the format: 8 significant bits, exponent range of float32,
    subnormal spacing 2**-133.  Overflow is not modelled (values here are O(1)).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                     # x = m * 2**e, 0.5 <= |m| < 1
    ulp_exp = np.maximum(e - 8, -133)
    ulp = np.ldexp(1.0, ulp_exp)
    return np.where(x == 0, x, np.rint(x / ulp) * ulp)


def round_to_f32(x):
    """Round float64 values to float32 (numpy's IEEE cast), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to(x, dtype):
    return round_to_bf16(x) if dtype == "bf16" else round_to_f32(x)


# --------------------------------------------------------------------------- compression

def compress(x, cu_seqlens_kv, cmp_ratio):
    """Segment-local mean pooling of r consecutive rows, exact in float64.

    [MI] 关键源码片段 compressor.py (_forward_thd): compressed row j of segment b
    gathers stream rows cu_seqlens[b] + j*r + [0, r); groups never cross a segment
    boundary and the tail rows are left to the window.  The learned gated pooling
    that follows on that page is elided there; the plain mean is the reading used
    for every workload.  Returns float64 [Tc, d] (unrounded).
    """
    cu = [int(v) for v in cu_seqlens_kv]
    r = int(cmp_ratio)
    rows = []
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        for j in range((e - s) // r):
            g = np.asarray(x[s + j * r: s + j * r + r], dtype=np.float64)
            rows.append(g.sum(axis=0) / r)
    d = np.asarray(x[:1]).shape[-1] if len(x) else 0
    if not rows:
        return np.zeros((0, d), dtype=np.float64)
    return np.stack(rows)


def compress_learned(x, wkv, wgate, ape, cu_seqlens_kv, cmp_ratio, overlap):
    """Learned gated compressor (the alternative to mean pooling), float64.

    [MI] 关键源码片段 compressor.py (_forward_thd and _overlap_transform_thd), in
    the page's order:
      1. two projections of the hidden rows, kv = x wkv^T and score = x wgate^T
         (linear_bf16_fp32: bf16 operands, float32 results; here float64);
      2. the rows of compressed row j of segment b are stream rows
         cu_seqlens[b] + j r + m, m in [0, r) (the len % r tail forms no row);
      3. the learned position table ape [r, C] is added to the scores by in-group
         position m (the page prints only ``ape.view(1, ratio, 1, -1)``; the
         reading is an addition, before the overlap step);
      4. with overlap (C = 2 hd) the group becomes 2r positions of hd channels:
         positions [0, r) hold the previous group's first-half channels [0, hd),
         positions [r, 2r) the group's own second-half channels [hd, 2 hd); a
         segment's first group has no predecessor and takes kv = 0, score = -inf
         there.  Without overlap (C = hd) the r positions are used as they are;
      5. the tail is elided on the page; the reading is a softmax of the scores
         over the positions, per channel, and the softmax-weighted sum of kv.
    x [Tkv, D]; wkv, wgate [C, D]; ape [r, C].  Returns float64 [Tc, hd].
    """
    cu = [int(v) for v in cu_seqlens_kv]
    r = int(cmp_ratio)
    kv = np.asarray(x, dtype=np.float64) @ np.asarray(wkv, dtype=np.float64).T       # step 1
    score = np.asarray(x, dtype=np.float64) @ np.asarray(wgate, dtype=np.float64).T
    ape = np.asarray(ape, dtype=np.float64)
    C = kv.shape[1]
    hd = C // 2 if overlap else C
    out = []
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        n = (e - s) // r
        g_kv = [kv[s + j * r: s + j * r + r] for j in range(n)]                      # step 2
        g_sc = [score[s + j * r: s + j * r + r] + ape for j in range(n)]             # step 3
        for j in range(n):
            if overlap:                                                               # step 4
                if j == 0:
                    prev_kv = np.zeros((r, hd))
                    prev_sc = np.full((r, hd), -np.inf)
                else:
                    prev_kv = g_kv[j - 1][:, :hd]
                    prev_sc = g_sc[j - 1][:, :hd]
                kvw = np.concatenate([prev_kv, g_kv[j][:, hd:]], axis=0)             # [2r, hd]
                scw = np.concatenate([prev_sc, g_sc[j][:, hd:]], axis=0)
            else:
                kvw, scw = g_kv[j], g_sc[j]
            m = scw.max(axis=0)                                                       # step 5
            p = np.exp(scw - m)
            p = p / p.sum(axis=0)
            out.append((p * kvw).sum(axis=0))
    if not out:
        return np.zeros((0, hd), dtype=np.float64)
    return np.stack(out)


# --------------------------------------------------------------------------- indexer

def indexer_scores(q_I_i, w_i, k_rows):
    """Lightning-indexer scores of one query against candidate compressed keys.

    [HP] 1. npu_lightning_indexer takes q, k and per-head weights w; the score of
    key c is sum over indexer heads h of w[h] * relu(<q[h], k[c]>).
    q_I_i [H_I, d_I], w_i [H_I], k_rows [n, d_I] -> float64 [n].
    """
    q = np.asarray(q_I_i, dtype=np.float64)
    w = np.asarray(w_i, dtype=np.float64)
    k = np.asarray(k_rows, dtype=np.float64)
    logits = q @ k.T                       # [H_I, n]
    return w @ np.maximum(logits, 0.0)


def indexer_topk(q_I, w, k_cmp, tables, topk, queries=None):
    """Top-k compressed rows per query, restricted to the query's own segment.

    [HP] 1. npu_lightning_indexer (sparse_count = topk, cmp_ratio 4) and
    [MI] 功能与动机 item 4: candidates are the causally complete compressed rows of
    the query's segment, addressed stream-absolutely ([MI] 评论区精华 item 1).
    With no more candidates than topk all of them are kept.  Ties keep the lower
    row.  Returns (idx int64 [nq, topk] ascending then -1, score float64 [nq, topk]
    aligned with idx, nan where idx is -1).
    """
    Tq = len(tables["q_seg"])
    qs = range(Tq) if queries is None else list(queries)
    nq = len(qs)
    idx = np.full((nq, topk), -1, dtype=np.int64)
    sc = np.full((nq, topk), np.nan, dtype=np.float64)
    for n, i in enumerate(qs):
        lo = int(tables["q_cmp_lo"][i])
        nv = int(tables["q_cmp_nvis"][i])
        if nv == 0:
            continue
        cand = np.arange(lo, lo + nv)
        s = indexer_scores(q_I[i], w[i], k_cmp[lo:lo + nv])
        if nv > topk:
            order = sorted(range(nv), key=lambda j: (-s[j], j))[:topk]
            keep = np.sort(np.array(order, dtype=np.int64))
        else:
            keep = np.arange(nv)
        idx[n, :len(keep)] = cand[keep]
        sc[n, :len(keep)] = s[keep]
    return idx, sc


def indexer_kl_grad(q_I, w, k_cmp, cmp_idx, attn_l1, tables, loss_scale, queries=None):
    """KL loss of the indexer against the main attention, and its gradients.

    [HP] 3. npu_sparse_lightning_indexer_kl_loss_grad takes the indexer's q, k and w,
    the sparse indices and attn_softmax_l1_norm; [HP] 4. says that tensor is the
    main attention's target distribution p (head-averaged probabilities at the
    compressed slots, shaped like the indices), fed to this operator directly.
    [MS] 主要改动 (TND num_seqs): the loss is a mean over the global token count, and
    the upstream gradient scale travels with it; ``loss_scale`` carries both.

    Reading (the page gives the operator's inputs only): for query i with selected
    rows c_j (the valid entries of cmp_idx[i], in order) and targets p_j =
    attn_l1[i, j],
        p^_j = p_j / sum_j p_j                    (the L1 normalisation of the name)
        I_j  = sum_h w[h] relu(u_hj),  u_hj = <q_I[i, h], k_cmp[c_j]>
        s_j  = softmax_j(I)
        loss_i = KL(p^ || s) = sum_j p^_j (log p^_j - log s_j)      (0 log 0 = 0)
        G_j  = loss_scale * (s_j - p^_j)          (d loss_i / d I_j = s_j - p^_j)
        d_w[i, h]  = sum_j G_j relu(u_hj)
        d_q[i, h]  = sum_j G_j w[h] [u_hj > 0] k_cmp[c_j]
        d_k[c_j]  += sum_h G_j w[h] [u_hj > 0] q_I[i, h]
    A query with no selected row or with sum_j p_j = 0 contributes nothing.
    Returns float64 d_q [nq, H_I, d_I], d_w [nq, H_I], d_k [len(k_cmp), d_I] and
    loss [nq] (the unscaled KL of each query).  With ``queries`` only those rows
    contribute (d_k is then a partial sum).
    """
    Tq = len(tables["q_seg"])
    qs = range(Tq) if queries is None else list(queries)
    nq = len(qs)
    H, dI = np.asarray(q_I[0]).shape if Tq else (0, 0)
    kk = np.asarray(k_cmp, dtype=np.float64)
    d_q = np.zeros((nq, H, dI), dtype=np.float64)
    d_w = np.zeros((nq, H), dtype=np.float64)
    d_k = np.zeros((len(kk), dI), dtype=np.float64)
    loss = np.zeros(nq, dtype=np.float64)
    for n, i in enumerate(qs):
        row = np.asarray(cmp_idx[i]).reshape(-1)
        rows = [int(c) for c in row if 0 <= int(c) < len(kk)]
        if not rows:
            continue
        p = np.asarray(attn_l1[i], dtype=np.float64).reshape(-1)[:len(rows)]
        psum = p.sum()
        if psum <= 0.0:
            continue
        ph = p / psum
        qi = np.asarray(q_I[i], dtype=np.float64)          # [H, dI]
        wi = np.asarray(w[i], dtype=np.float64)            # [H]
        K = kk[rows]                                       # [n, dI]
        u = qi @ K.T                                       # [H, n]
        I = wi @ np.maximum(u, 0.0)                        # [n]
        z = I - I.max()
        ls = z - math.log(np.exp(z).sum())                 # log softmax
        sm = np.exp(ls)
        nz = ph > 0
        loss[n] = float((ph[nz] * (np.log(ph[nz]) - ls[nz])).sum())
        G = loss_scale * (sm - ph)                         # [n]
        act = (u > 0.0).astype(np.float64)                 # [H, n]
        d_w[n] = np.maximum(u, 0.0) @ G
        coef = wi[:, None] * act * G[None, :]              # [H, n]
        d_q[n] = coef @ K
        contrib = coef.T @ qi                              # [n, dI]
        for j, c in enumerate(rows):
            d_k[c] += contrib[j]
    return dict(d_q=d_q, d_w=d_w, d_k=d_k, loss=loss)


# --------------------------------------------------------------------------- sparse MLA

def sparse_mla_fwd(q, ori_kv, cmp_kv, cmp_idx, tables, sinks, softmax_scale,
                   ori_win_left, ori_win_right, cu_seqlens_kv, global_start, queries=None,
                   attend_all_visible=False):
    """Sparse MLA forward with a window branch, a compressed branch and a sink.

    [HP] 背景 item 2 and 2. npu_sparse_flash_mla: one latent KV serves as keys and
    values (DS4 geometry head_dim = d_v = 512, [ML] Environment note); the ori_kv
    branch is a band of ori_win_left rows before the query plus ori_win_right after
    it, clamped to the query's segment (band parameters, not an index list: the
    page's control experiment shows ori_sparse_indices is ignored); the cmp_kv
    branch attends the rows listed in cmp_sparse_indices (-1 = empty slot) or,
    when ``attend_all_visible``, every causally complete row of the segment;
    sinks add exp(sink[h]) to each head's softmax denominator with no value.
    Returns out float64 [nq, H, d] and lse float64 [nq, H] (natural log of the full
    denominator in the scaled-logit domain, sink included).
    """
    Tq = len(tables["q_seg"])
    qs = range(Tq) if queries is None else list(queries)
    nq = len(qs)
    H, d = np.asarray(q[0]).shape if Tq else (0, 0)
    out = np.zeros((nq, H, d), dtype=np.float64)
    lse = np.zeros((nq, H), dtype=np.float64)
    cu_kv = [int(v) for v in cu_seqlens_kv]
    sk = None if sinks is None else np.asarray(sinks, dtype=np.float64)
    for n, i in enumerate(qs):
        b = int(tables["q_seg"][i])
        t = int(global_start) + i
        lo = max(cu_kv[b], t - int(ori_win_left))
        hi = min(cu_kv[b + 1] - 1, t + int(ori_win_right))
        keys = [np.asarray(ori_kv[lo:hi + 1], dtype=np.float64)]
        if cmp_kv is not None:
            if attend_all_visible:
                c0 = int(tables["q_cmp_lo"][i])
                rows = list(range(c0, c0 + int(tables["q_cmp_nvis"][i])))
            elif cmp_idx is not None:
                rows = [int(c) for c in cmp_idx[i] if c >= 0]
            else:
                rows = []
            if rows:
                keys.append(np.asarray(cmp_kv[rows], dtype=np.float64))
        K = np.concatenate(keys, axis=0)           # [n_keys, d], K = V
        qi = np.asarray(q[i], dtype=np.float64)    # [H, d]
        z = softmax_scale * (qi @ K.T)             # [H, n_keys]
        m = z.max(axis=1)
        if sk is not None:
            m = np.maximum(m, sk)
        e = np.exp(z - m[:, None])
        den = e.sum(axis=1)
        if sk is not None:
            den = den + np.exp(sk - m)
        out[n] = (e @ K) / den[:, None]
        lse[n] = m + np.log(den)
    return out, lse


def _query_keys(i, tables, ori_win_left, ori_win_right, cu_kv, global_start, cmp_idx, attend_all_visible,
                cmp_present):
    """Key list of query i in the forward's order: window rows, then compressed rows."""
    b = int(tables["q_seg"][i])
    t = int(global_start) + i
    lo = max(cu_kv[b], t - int(ori_win_left))
    hi = min(cu_kv[b + 1] - 1, t + int(ori_win_right))
    rows = []
    if cmp_present:
        if attend_all_visible:
            c0 = int(tables["q_cmp_lo"][i])
            rows = list(range(c0, c0 + int(tables["q_cmp_nvis"][i])))
        elif cmp_idx is not None:
            rows = [int(c) for c in cmp_idx[i] if c >= 0]
    return lo, hi, rows


def sparse_mla_bwd(q, ori_kv, cmp_kv, cmp_idx, tables, sinks, softmax_scale, ori_win_left, ori_win_right,
                   cu_seqlens_kv, global_start, dout, cmp_slots=0, attend_all_visible=False, queries=None):
    """Gradients of sparse_mla_fwd for the output gradient ``dout``.

    [HP] 4. npu_sparse_flash_mla_grad: the backward of the sparse MLA operator takes
    q, dout, the forward output and lse plus the forward's key sources, and returns
    d_query, d_ori_kv, d_cmp_kv, d_sinks and the window / compressed
    "softmax_l1_norm" (the head-averaged attention distribution, shaped like the
    index lists).  Written from the forward's definition (one joint softmax over
    window rows, compressed rows and the sink; K = V):
        P[h,k] = exp(z[h,k] - lse[h]),  z = scale * q[h] . kv[k],  p_sink = exp(sink[h] - lse[h])
        dP[h,k] = dout[h] . kv[k],  D[h] = sum_k P[h,k] dP[h,k] = dout[h] . out[h]
        dS[h,k] = P[h,k] (dP[h,k] - D[h])
        dq[h] = scale * sum_k dS[h,k] kv[k]
        dkv[k] += sum_h (scale * dS[h,k] q[h] + P[h,k] dout[h])
        dsink[h] += -p_sink[h] D[h]
    out and lse are recomputed here in fp64 (the operator receives them from the
    forward).  Returns float64 arrays: dq [nq, H, d], d_ori_kv [Tkv, d],
    d_cmp_kv [Tc, d] (None without compressed rows), d_sinks [H] (None without
    sinks), ori_l1 [nq, W], cmp_l1 [nq, cmp_slots].  With ``queries`` only those
    rows contribute (the kv gradients are then partial sums).
    """
    Tq = len(tables["q_seg"])
    qs = range(Tq) if queries is None else list(queries)
    nq = len(qs)
    H, d = np.asarray(q[0]).shape if Tq else (0, 0)
    W = int(ori_win_left) + int(ori_win_right) + 1
    cu_kv = [int(v) for v in cu_seqlens_kv]
    sk = None if sinks is None else np.asarray(sinks, dtype=np.float64)
    dq = np.zeros((nq, H, d), dtype=np.float64)
    d_ori = np.zeros((len(ori_kv), d), dtype=np.float64)
    d_cmp = None if cmp_kv is None else np.zeros((len(cmp_kv), d), dtype=np.float64)
    d_sinks = None if sk is None else np.zeros(H, dtype=np.float64)
    ori_l1 = np.zeros((nq, W), dtype=np.float64)
    cmp_l1 = np.zeros((nq, int(cmp_slots)), dtype=np.float64)
    for n, i in enumerate(qs):
        lo, hi, rows = _query_keys(i, tables, ori_win_left, ori_win_right, cu_kv, global_start, cmp_idx,
                                   attend_all_visible, cmp_kv is not None)
        nwin = hi - lo + 1
        parts = [np.asarray(ori_kv[lo:hi + 1], dtype=np.float64)]
        if rows:
            parts.append(np.asarray(cmp_kv[rows], dtype=np.float64))
        K = np.concatenate(parts, axis=0)             # [n_keys, d]; K = V
        qi = np.asarray(q[i], dtype=np.float64)       # [H, d]
        do = np.asarray(dout[n], dtype=np.float64)    # [H, d]
        z = softmax_scale * (qi @ K.T)                # [H, n_keys]
        m = z.max(axis=1)
        if sk is not None:
            m = np.maximum(m, sk)
        den = np.exp(z - m[:, None]).sum(axis=1)
        if sk is not None:
            den = den + np.exp(sk - m)
        lse = m + np.log(den)
        P = np.exp(z - lse[:, None])                  # [H, n_keys]
        out = P @ K                                   # [H, d]
        dP = do @ K.T                                 # [H, n_keys]
        D = (do * out).sum(axis=1)                    # [H]
        dS = P * (dP - D[:, None])
        dq[n] = softmax_scale * (dS @ K)
        dK = softmax_scale * (dS.T @ qi) + P.T @ do   # [n_keys, d]
        d_ori[lo:hi + 1] += dK[:nwin]
        for j, c in enumerate(rows):
            d_cmp[c] += dK[nwin + j]
        if sk is not None:
            d_sinks += -np.exp(sk - lse) * D
        l1 = P.mean(axis=0)
        ori_l1[n, :nwin] = l1[:nwin]
        ncs = min(len(rows), int(cmp_slots))
        cmp_l1[n, :ncs] = l1[nwin:nwin + ncs]
    return dict(dq=dq, d_ori_kv=d_ori, d_cmp_kv=d_cmp, d_sinks=d_sinks, ori_l1=ori_l1, cmp_l1=cmp_l1)


# --------------------------------------------------------------------------- forward

def csa_forward(*, q, ori_kv, q_I, k_I, w, sinks, cu_seqlens_q, cu_seqlens_kv, global_start,
                cmp_ratio, ori_win_left, ori_win_right, topk, softmax_scale, dtype="bf16",
                mode=None, queries=None, cmp_idx_override=None):
    """The whole forward: layout, compression, indexer top-k, sparse MLA.

    Compressed rows (latent and indexer keys) are rounded to the call dtype once,
    as the library stores them; everything after is float64 on those values.
    ``cmp_idx_override`` [nq, topk] replaces the oracle's own top-k selection (used
    to score another selection that lies inside the score-tie band).
    """
    Tq = int(np.asarray(q).shape[0]) if not hasattr(q, "shape") else int(q.shape[0])
    tabs = build_indices(cu_seqlens_q, cu_seqlens_kv, global_start, Tq, cmp_ratio,
                         ori_win_left, ori_win_right)
    Tc = int(tabs["cu_seqlens_cmp"][-1])
    if mode is None:
        mode = layer_compress_mode(cmp_ratio, Tc)
    res = dict(tables=tabs, mode=mode)
    cmp_kv = kI_cmp = None
    if mode != NO_COMPRESS:
        cmp_kv = round_to(compress(ori_kv, cu_seqlens_kv, cmp_ratio), dtype)
        res["cmp_kv"] = cmp_kv
    cmp_idx = None
    qs = range(Tq) if queries is None else list(queries)
    if mode == INDEXER:
        kI_cmp = round_to(compress(k_I, cu_seqlens_kv, cmp_ratio), dtype)
        res["k_I_cmp"] = kI_cmp
        if cmp_idx_override is None:
            idx, sc = indexer_topk(q_I, w, kI_cmp, tabs, topk, queries=qs)
            res["topk_idx"], res["topk_score"] = idx, sc
        else:
            idx = np.asarray(cmp_idx_override)
        # re-index to full query numbering for the attention call
        cmp_idx = {i: idx[n] for n, i in enumerate(qs)}
    out, lse = sparse_mla_fwd(q, ori_kv, cmp_kv, cmp_idx, tabs, sinks, softmax_scale,
                              ori_win_left, ori_win_right, cu_seqlens_kv, global_start,
                              queries=qs, attend_all_visible=(mode == COMPRESSOR_ONLY))
    res["out"], res["lse"] = out, lse
    return res
