"""Pins of the backward oracle (oracle.sparse_mla_bwd) against independent definitions.

* torch autograd (float64) through a dense masked formulation of the forward
  written here from the definition (every (query, key) pair masked in or out, the
  sink as one more logit with a zero value) -- the gradients of q, the latent rows,
  the compressed rows and the sinks, and the head-averaged probabilities;
* torch's own scaled_dot_product_attention backward for plain causal attention;
* central finite differences of a scalar loss for the sink gradient;
* the probability sum rule: window + compressed slots + the sink share = 1.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle


def _pack(rng, lengths, H, d, r=4):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(cu[-1])
    q = rng.standard_normal((T, H, d))
    kv = rng.standard_normal((T, d))
    tabs = oracle.build_indices(cu, cu, 0, T, r, 1000, 0)
    return cu, T, q, kv, tabs


def _dense_grads(q, kv, cmp_kv, sel, win, sinks, scale, dout):
    """Autograd of the masked dense forward.  sel [T, Tc] / win [T, T] are boolean masks."""
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(kv, requires_grad=True)
    ct = torch.tensor(cmp_kv, requires_grad=True) if cmp_kv is not None else None
    st = torch.tensor(sinks, requires_grad=True) if sinks is not None else None
    T, H, _ = q.shape
    keys = kt if ct is None else torch.cat([kt, ct], dim=0)                     # [T + Tc, d]
    mask = torch.tensor(win if ct is None else np.concatenate([win, sel], axis=1))  # [T, T + Tc]
    z = scale * torch.einsum("thd,kd->thk", qt, keys)
    z = z.masked_fill(~mask[:, None, :], float("-inf"))
    if st is not None:
        z = torch.cat([z, st[None, :, None].expand(T, H, 1)], dim=2)
        vals = torch.cat([keys, torch.zeros((1, keys.shape[1]), dtype=keys.dtype)], dim=0)
    else:
        vals = keys
    p = torch.softmax(z, dim=2)
    out = torch.einsum("thk,kd->thd", p, vals)
    loss = (out * torch.tensor(dout)).sum()
    grads = torch.autograd.grad(loss, [x for x in (qt, kt, ct, st) if x is not None])
    names = [n for n, x in zip(("dq", "d_ori_kv", "d_cmp_kv", "d_sinks"), (qt, kt, ct, st)) if x is not None]
    res = dict(zip(names, [g.numpy() for g in grads]))
    res["p"] = p.detach().numpy()
    return res


def _window_mask(cu, T, wl):
    seg = np.searchsorted(cu, np.arange(T), side="right") - 1
    t = np.arange(T)
    return (seg[:, None] == seg[None, :]) & (t[None, :] <= t[:, None]) & (t[None, :] >= t[:, None] - wl)


@pytest.mark.parametrize("seed,mode", [(0, "select"), (1, "select"), (2, "all"), (3, "window"), (4, "select")])
def test_bwd_matches_autograd_of_dense_forward(seed, mode):
    rng = np.random.default_rng(900 + seed)
    lengths = [int(v) for v in rng.integers(3, 40, size=3)]
    H, d, r, wl, topk = 3, 8, 4, 6, 3
    cu, T, q, kv, tabs = _pack(rng, lengths, H, d, r)
    tabs = oracle.build_indices(cu, cu, 0, T, r, wl, 0)
    cmp_kv = None if mode == "window" else oracle.compress(kv, cu, r)
    Tc = 0 if cmp_kv is None else len(cmp_kv)
    sinks = rng.standard_normal(H)
    scale = 0.4
    dout = rng.standard_normal((T, H, d))
    sel = np.zeros((T, Tc), dtype=bool)
    cmp_idx = None
    if mode == "select":
        cmp_idx = np.full((T, topk), -1, dtype=np.int64)
        for i in range(T):
            lo, nv = int(tabs["q_cmp_lo"][i]), int(tabs["q_cmp_nvis"][i])
            if nv:
                pick = np.sort(rng.choice(nv, size=min(nv, topk), replace=False)) + lo
                cmp_idx[i, :len(pick)] = pick
                sel[i, pick] = True
    elif mode == "all":
        for i in range(T):
            lo, nv = int(tabs["q_cmp_lo"][i]), int(tabs["q_cmp_nvis"][i])
            sel[i, lo:lo + nv] = True
    win = _window_mask(cu, T, wl)
    ref = _dense_grads(q, kv, cmp_kv, sel, win, sinks, scale, dout)
    slots = topk if mode == "select" else (max(1, int(tabs["q_cmp_nvis"].max())) if mode == "all" else 0)
    got = oracle.sparse_mla_bwd(q, kv, cmp_kv, cmp_idx, tabs, sinks, scale, wl, 0, cu, 0, dout,
                                cmp_slots=slots, attend_all_visible=(mode == "all"))
    np.testing.assert_allclose(got["dq"], ref["dq"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["d_ori_kv"], ref["d_ori_kv"], rtol=1e-10, atol=1e-12)
    if cmp_kv is not None:
        np.testing.assert_allclose(got["d_cmp_kv"], ref["d_cmp_kv"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["d_sinks"], ref["d_sinks"], rtol=1e-10, atol=1e-12)
    # head-averaged probabilities at the window slots and the compressed slots
    pm = ref["p"].mean(axis=1)                      # [T, T + Tc (+ 1)]
    for i in range(T):
        w = tabs["win_idx"][i]
        for k, row in enumerate(w):
            exp = pm[i, row] if row >= 0 else 0.0
            assert abs(got["ori_l1"][i, k] - exp) < 1e-12
        if mode == "select":
            for j, c in enumerate(cmp_idx[i]):
                exp = pm[i, T + c] if c >= 0 else 0.0
                assert abs(got["cmp_l1"][i, j] - exp) < 1e-12
        elif mode == "all":
            lo, nv = int(tabs["q_cmp_lo"][i]), int(tabs["q_cmp_nvis"][i])
            for j in range(slots):
                exp = pm[i, T + lo + j] if j < nv else 0.0
                assert abs(got["cmp_l1"][i, j] - exp) < 1e-12


@pytest.mark.parametrize("seed", range(3))
def test_bwd_causal_window_matches_torch_sdpa_backward(seed):
    rng = np.random.default_rng(950 + seed)
    L = int(rng.integers(5, 40))
    H, d, scale = 2, 16, 0.3
    cu = np.array([0, L], dtype=np.int64)
    q = rng.standard_normal((L, H, d))
    kv = rng.standard_normal((L, d))
    dout = rng.standard_normal((L, H, d))
    tabs = oracle.build_indices(cu, cu, 0, L, 4, 1000, 0)
    got = oracle.sparse_mla_bwd(q, kv, None, None, tabs, None, scale, 1000, 0, cu, 0, dout)
    qt = torch.tensor(q).permute(1, 0, 2).requires_grad_(True)
    kt = torch.tensor(kv, requires_grad=True)
    kk = kt[None].expand(H, -1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kk, kk, is_causal=True, scale=scale)
    gq, gk = torch.autograd.grad((out * torch.tensor(dout).permute(1, 0, 2)).sum(), [qt, kt])
    np.testing.assert_allclose(got["dq"], gq.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["d_ori_kv"], gk.numpy(), rtol=1e-10, atol=1e-12)


def test_bwd_sink_gradient_matches_finite_differences():
    rng = np.random.default_rng(977)
    lengths = [9, 14]
    H, d, wl, scale = 2, 6, 4, 0.5
    cu, T, q, kv, _ = _pack(rng, lengths, H, d)
    tabs = oracle.build_indices(cu, cu, 0, T, 4, wl, 0)
    sinks = rng.standard_normal(H)
    dout = rng.standard_normal((T, H, d))

    def loss(s):
        out, _ = oracle.sparse_mla_fwd(q, kv, None, None, tabs, s, scale, wl, 0, cu, 0)
        return float((out * dout).sum())

    got = oracle.sparse_mla_bwd(q, kv, None, None, tabs, sinks, scale, wl, 0, cu, 0, dout)["d_sinks"]
    eps = 1e-6
    for h in range(H):
        e = np.zeros(H)
        e[h] = eps
        fd = (loss(sinks + e) - loss(sinks - e)) / (2 * eps)
        assert abs(got[h] - fd) < 1e-7 * max(1.0, abs(fd))


def test_bwd_probability_sum_rule():
    rng = np.random.default_rng(990)
    lengths = [17, 33, 8]
    H, d, wl, topk = 4, 8, 9, 4
    cu, T, q, kv, _ = _pack(rng, lengths, H, d)
    tabs = oracle.build_indices(cu, cu, 0, T, 4, wl, 0)
    cmp_kv = oracle.compress(kv, cu, 4)
    cmp_idx = np.full((T, topk), -1, dtype=np.int64)
    for i in range(T):
        lo, nv = int(tabs["q_cmp_lo"][i]), int(tabs["q_cmp_nvis"][i])
        k = min(nv, topk)
        cmp_idx[i, :k] = lo + np.arange(k)
    sinks = rng.standard_normal(H)
    dout = rng.standard_normal((T, H, d))
    got = oracle.sparse_mla_bwd(q, kv, cmp_kv, cmp_idx, tabs, sinks, 0.35, wl, 0, cu, 0, dout, cmp_slots=topk)
    _, lse = oracle.sparse_mla_fwd(q, kv, cmp_kv, cmp_idx, tabs, sinks, 0.35, wl, 0, cu, 0)
    sink_share = np.exp(sinks[None, :] - lse).mean(axis=1)
    total = got["ori_l1"].sum(axis=1) + got["cmp_l1"].sum(axis=1) + sink_share
    np.testing.assert_allclose(total, 1.0, rtol=0, atol=1e-12)
