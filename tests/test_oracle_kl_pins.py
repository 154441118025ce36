"""Pins of the indexer KL-loss oracle (oracle.indexer_kl_grad) against independent definitions.

* torch autograd (float64) of the loss written here with torch's own KL divergence
  (``F.kl_div`` on ``log_softmax``) over each query's selected rows: the gradients of
  the indexer query, the head weights and the compressed keys, and the per-query loss;
* central finite differences of the oracle's own loss for the head weights;
* special cases: a target equal to the indexer's distribution (zero loss and zero
  gradients), selection rows with holes and queries with nothing selected, and a
  score exactly at the ReLU kink (gradient 0 there, as torch's ReLU).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _case(seed, lengths, H=4, dI=8, r=4, topk=3, holes=False):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(cu[-1])
    tabs = oracle.build_indices(cu, cu, 0, T, r, 1000, 0)
    k_tok = rng.standard_normal((T, dI))
    k_cmp = oracle.compress(k_tok, cu, r)
    q = rng.standard_normal((T, H, dI))
    w = rng.standard_normal((T, H))
    idx = np.full((T, topk), -1, dtype=np.int64)
    for i in range(T):
        lo, nv = int(tabs["q_cmp_lo"][i]), int(tabs["q_cmp_nvis"][i])
        if nv:
            pick = np.sort(rng.choice(nv, size=min(nv, topk), replace=False)) + lo
            if holes and len(pick) > 1 and i % 3 == 0:
                idx[i, 0] = pick[0]
                idx[i, 2 if topk > 2 else 1] = pick[1]      # a hole at slot 1
            else:
                idx[i, :len(pick)] = pick
    p = rng.random((T, topk)) * (idx >= 0)
    return cu, T, tabs, q, w, k_cmp, idx, p


def _torch_grads(q, w, k_cmp, idx, p, scale):
    qt = torch.tensor(q, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    kt = torch.tensor(k_cmp, requires_grad=True)
    total = torch.zeros((), dtype=torch.float64)
    losses = []
    for i in range(len(q)):
        rows = [int(c) for c in idx[i] if c >= 0]
        if not rows:
            losses.append(0.0)
            continue
        target = torch.tensor(p[i][np.asarray(idx[i]) >= 0])   # the target at each selected slot
        if float(target.sum()) <= 0:
            losses.append(0.0)
            continue
        target = target / target.sum()
        K = kt[rows]                                            # [n, dI]
        scores = (wt[i][:, None] * torch.relu(qt[i] @ K.T)).sum(0)  # [n]
        kl = F.kl_div(torch.log_softmax(scores, 0), target, reduction="sum")
        losses.append(float(kl.detach()))
        total = total + scale * kl
    gq, gw, gk = torch.autograd.grad(total, [qt, wt, kt], allow_unused=True)
    z = lambda g, like: np.zeros(like.shape) if g is None else g.numpy()
    return z(gq, q), z(gw, w), z(gk, k_cmp), np.array(losses)


@pytest.mark.parametrize("seed,holes", [(0, False), (1, True), (2, False), (3, True)])
def test_kl_grad_matches_autograd(seed, holes):
    lengths = [int(v) for v in np.random.default_rng(700 + seed).integers(2, 40, size=3)]
    cu, T, tabs, q, w, k_cmp, idx, p = _case(800 + seed, lengths, holes=holes)
    # the oracle reads p per compacted slot: move each row's valid targets to the front
    pc = np.zeros_like(p)
    for i in range(T):
        v = p[i][idx[i] >= 0]
        pc[i, :len(v)] = v
    scale = 0.37
    got = oracle.indexer_kl_grad(q, w, k_cmp, idx, pc, tabs, scale)
    gq, gw, gk, loss = _torch_grads(q, w, k_cmp, idx, p, scale)
    np.testing.assert_allclose(got["d_q"], gq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["d_w"], gw, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["d_k"], gk, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["loss"], loss, rtol=1e-10, atol=1e-13)
    assert (got["loss"] >= -1e-14).all()


def test_kl_grad_weights_match_finite_differences():
    cu, T, tabs, q, w, k_cmp, idx, p = _case(901, [23, 17])
    scale = 1.3

    def total(wv):
        return scale * oracle.indexer_kl_grad(q, wv, k_cmp, idx, p, tabs, 1.0)["loss"].sum()

    got = oracle.indexer_kl_grad(q, w, k_cmp, idx, p, tabs, scale)["d_w"]
    eps = 1e-6
    for i in (5, 11, 30):
        for h in range(w.shape[1]):
            e = np.zeros_like(w)
            e[i, h] = eps
            fd = (total(w + e) - total(w - e)) / (2 * eps)
            assert abs(got[i, h] - fd) < 1e-6 * max(1.0, abs(fd))


def test_kl_grad_vanishes_when_target_is_the_indexer_distribution():
    cu, T, tabs, q, w, k_cmp, idx, _ = _case(902, [30, 12])
    p = np.zeros(idx.shape)
    for i in range(T):
        rows = [int(c) for c in idx[i] if c >= 0]
        if rows:
            s = oracle.indexer_scores(q[i], w[i], k_cmp[rows])
            e = np.exp(s - s.max())
            p[i, :len(rows)] = 3.5 * e / e.sum()        # any positive multiple
    got = oracle.indexer_kl_grad(q, w, k_cmp, idx, p, tabs, 2.0)
    for key in ("d_q", "d_w", "d_k", "loss"):
        assert np.abs(got[key]).max() < 1e-12, key


def test_kl_grad_empty_selections_and_zero_targets():
    cu, T, tabs, q, w, k_cmp, idx, p = _case(903, [9, 3, 14])
    idx[4] = -1                  # nothing selected
    p[6] = 0.0                   # a target that sums to zero
    got = oracle.indexer_kl_grad(q, w, k_cmp, idx, p, tabs, 1.0)
    for i in (4, 6):
        assert not got["d_q"][i].any() and not got["d_w"][i].any() and got["loss"][i] == 0.0
    # the first query of each segment sees no compressed row at all
    for b in range(len(cu) - 1):
        assert not got["d_q"][cu[b]].any()


def test_kl_grad_relu_kink_has_zero_derivative():
    # one query, two keys; head 0's score against key 0 is exactly 0
    tabs = oracle.build_indices(np.array([0, 8]), np.array([0, 8]), 0, 8, 4, 1000, 0)
    k_cmp = np.array([[1.0, 0.0], [0.5, 2.0]])
    q = np.zeros((8, 2, 2))
    q[7] = [[0.0, 1.0], [1.0, 1.0]]           # <q_0, k_0> = 0
    w = np.ones((8, 2))
    idx = np.full((8, 2), -1)
    idx[7] = [0, 1]
    p = np.zeros((8, 2))
    p[7] = [0.9, 0.1]
    got = oracle.indexer_kl_grad(q, w, k_cmp, idx, p, tabs, 1.0)
    gq, gw, gk, _ = _torch_grads(q, w, k_cmp, idx, p, 1.0)
    np.testing.assert_allclose(got["d_q"], gq, atol=1e-14)
    np.testing.assert_allclose(got["d_k"], gk, atol=1e-14)
    np.testing.assert_allclose(got["d_w"], gw, atol=1e-14)
