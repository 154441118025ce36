"""Dense-mask brute force of the CSA forward, used only to pin the oracle on tiny packs.

Built from first principles over every (query row, key row) pair instead of the
oracle's per-query ranges: segment membership of each stream row comes from
``numpy.searchsorted``, compressed rows are enumerated as complete (segment,
group) cells of stream rows, visibility, window and top-k are boolean masks, and
the joint softmax with the sink is ``scipy.special.logsumexp`` over the
concatenated logits.  Shares no code with ``oracle/``.
"""
from __future__ import annotations

import numpy as np
from scipy.special import logsumexp


def dense_forward(*, q, ori_kv, q_I, k_I, w, sinks, cu_seqlens_q, cu_seqlens_kv, global_start,
                  cmp_ratio, ori_win_left, ori_win_right, topk, softmax_scale, mode, round_cmp):
    """mode: 0 window only, 1 all visible compressed rows, 2 indexer top-k.

    ``round_cmp`` rounds the pooled compressed rows to the storage dtype (a callable).
    Returns dict(out [Tq,H,d], lse [Tq,H], sel [Tq,Tc] bool, cmp_kv [Tc,d]).
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(ori_kv, dtype=np.float64)
    Tq, H, d = q.shape
    Tkv = kv.shape[0]
    cu = np.asarray(cu_seqlens_kv, dtype=np.int64)
    rows = np.arange(Tkv)
    seg_of = np.searchsorted(cu, rows, side="right") - 1
    pos_of = rows - cu[seg_of]
    t = global_start + np.arange(Tq)
    qseg = seg_of[t]
    qpos = pos_of[t]
    r = int(cmp_ratio)
    # every complete (segment, group) cell of r stream rows, in stream order
    cells = {}
    for k in range(Tkv):
        cells.setdefault((int(seg_of[k]), int(pos_of[k]) // r), []).append(k)
    full = sorted(key for key, members in cells.items() if len(members) == r) if mode else []
    Tc = len(full)
    cmp_seg = np.array([s for s, _ in full], dtype=np.int64)
    cmp_last = np.array([g * r + r - 1 for _, g in full], dtype=np.int64)
    pool = lambda x: np.stack([np.asarray(x, np.float64)[cells[key]].mean(axis=0) for key in full]) \
        if Tc else np.zeros((0, np.asarray(x).shape[1]))
    cmp_kv = round_cmp(pool(kv)) if mode else np.zeros((0, d))
    vis = (cmp_seg[None, :] == qseg[:, None]) & (cmp_last[None, :] <= qpos[:, None]) if mode else \
        np.zeros((Tq, 0), dtype=bool)
    sel = vis.copy()
    if mode == 2 and Tc:
        kI = round_cmp(pool(k_I))
        qi = np.asarray(q_I, dtype=np.float64)
        logit = np.einsum("ihd,cd->ihc", qi, kI)
        score = np.einsum("ih,ihc->ic", np.asarray(w, dtype=np.float64), np.maximum(logit, 0))
        for i in range(Tq):
            cand = np.nonzero(vis[i])[0]
            if len(cand) > topk:
                order = np.lexsort((cand, -score[i, cand]))  # score descending, row ascending
                sel[i] = False
                sel[i, cand[order[:topk]]] = True
    win = (seg_of[None, :] == qseg[:, None]) & (rows[None, :] >= t[:, None] - ori_win_left) & \
          (rows[None, :] <= t[:, None] + ori_win_right)
    z_ori = softmax_scale * np.einsum("ihd,kd->ihk", q, kv)
    z_ori = np.where(win[:, None, :], z_ori, -np.inf)
    z_cmp = softmax_scale * np.einsum("ihd,cd->ihc", q, cmp_kv)
    z_cmp = np.where(sel[:, None, :], z_cmp, -np.inf)
    parts = [z_ori, z_cmp]
    if sinks is not None:
        parts.append(np.broadcast_to(np.asarray(sinks, np.float64)[None, :, None], (Tq, H, 1)))
    z = np.concatenate(parts, axis=2)
    lse = logsumexp(z, axis=2)
    P = np.exp(z - lse[:, :, None])
    out = P[:, :, :Tkv] @ kv + P[:, :, Tkv:Tkv + Tc] @ cmp_kv
    return dict(out=out, lse=lse, sel=sel, cmp_kv=cmp_kv, vis=vis)
