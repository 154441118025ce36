"""Pins of the learned gated compressor oracle (oracle.compress_learned).

Each case reduces the learned pooling to something fixed independently of it:

* zero gate weights and position table: the softmax is uniform, so the result is
  the (separately pinned) mean pooling of the projected rows, and with overlap the
  average of the previous group's first-half mean and the group's own second-half
  mean (the second half alone for a segment's first group);
* a position table of log(1), .., log(r) and zero gates: closed-form weights m+1 / 10;
* one very large position-table entry: hard selection of that position's value
  (in the previous group's half or the group's own half), and for a segment's
  first group, where the previous half is masked, the mean of its own half;
* gates equal to a large multiple of the kv projection: the softmax-weighted sum
  tends to the per-channel maximum over the candidate positions (the minimum for a
  large negative multiple);
* packing: a pack equals its segments run one by one; tail rows are never read.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle


def _case(seed, lengths, D=24, hd=6, r=4, overlap=True):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(cu[-1])
    C = 2 * hd if overlap else hd
    x = rng.standard_normal((T, D))
    wkv = rng.standard_normal((C, D)) / np.sqrt(D)
    wgate = rng.standard_normal((C, D)) / np.sqrt(D)
    ape = rng.standard_normal((r, C))
    return cu, x, wkv, wgate, ape


def _groups(cu, r):
    """(segment start, local group index) of every compressed row, in order."""
    out = []
    for b in range(len(cu) - 1):
        for j in range((int(cu[b + 1]) - int(cu[b])) // r):
            out.append((int(cu[b]), j))
    return out


LENGTHS = [9, 3, 22, 17, 4]


def test_uniform_gates_reduce_to_mean_pooling():
    cu, x, wkv, _, _ = _case(1, LENGTHS, overlap=False)
    got = oracle.compress_learned(x, wkv, np.zeros_like(wkv), np.zeros((4, wkv.shape[0])), cu, 4, False)
    ref = oracle.compress(x @ wkv.T, cu, 4)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


def test_uniform_gates_with_overlap_average_two_half_means():
    hd = 6
    cu, x, wkv, _, _ = _case(2, LENGTHS, hd=hd, overlap=True)
    got = oracle.compress_learned(x, wkv, np.zeros_like(wkv), np.zeros((4, 2 * hd)), cu, 4, True)
    lo = oracle.compress(x @ wkv[:hd].T, cu, 4)      # first-half channels, per group
    hi = oracle.compress(x @ wkv[hd:].T, cu, 4)      # second-half channels
    for n, (s, j) in enumerate(_groups(cu, 4)):
        want = hi[n] if j == 0 else 0.5 * (lo[n - 1] + hi[n])
        np.testing.assert_allclose(got[n], want, rtol=1e-13, atol=1e-14)


def test_position_table_gives_closed_form_weights():
    cu, x, wkv, _, _ = _case(3, LENGTHS, overlap=False)
    ape = np.log(np.arange(1, 5, dtype=np.float64))[:, None] * np.ones((1, wkv.shape[0]))
    got = oracle.compress_learned(x, wkv, np.zeros_like(wkv), ape, cu, 4, False)
    wts = np.array([0.1, 0.2, 0.3, 0.4])
    for n, (s, j) in enumerate(_groups(cu, 4)):
        rows = x[s + 4 * j: s + 4 * j + 4]
        np.testing.assert_allclose(got[n], (wts @ rows) @ wkv.T, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("m0,half", [(0, "lo"), (3, "lo"), (1, "hi"), (2, "hi")])
def test_large_position_entry_selects_one_row(m0, half):
    hd = 6
    cu, x, wkv, _, _ = _case(4, LENGTHS, hd=hd, overlap=True)
    ape = np.zeros((4, 2 * hd))
    if half == "lo":
        ape[m0, :hd] = 80.0
    else:
        ape[m0, hd:] = 80.0
    got = oracle.compress_learned(x, wkv, np.zeros_like(wkv), ape, cu, 4, True)
    for n, (s, j) in enumerate(_groups(cu, 4)):
        if half == "hi":
            want = x[s + 4 * j + m0] @ wkv[hd:].T
        elif j > 0:
            want = x[s + 4 * (j - 1) + m0] @ wkv[:hd].T
        else:  # the previous half is masked: uniform over the group's own half
            want = x[s + 4 * j: s + 4 * j + 4].mean(axis=0) @ wkv[hd:].T
        np.testing.assert_allclose(got[n], want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("overlap", [False, True])
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_gates_tied_to_kv_tend_to_the_extreme(overlap, sign):
    hd = 6
    cu, x, wkv, _, _ = _case(5, LENGTHS, hd=hd, overlap=overlap)
    C = wkv.shape[0]
    got = oracle.compress_learned(x, wkv, sign * 1e5 * wkv, np.zeros((4, C)), cu, 4, overlap)
    kv = x @ wkv.T
    pick = np.max if sign > 0 else np.min
    for n, (s, j) in enumerate(_groups(cu, 4)):
        own = kv[s + 4 * j: s + 4 * j + 4]
        if not overlap:
            cand = own
        elif j == 0:
            cand = own[:, hd:]
        else:
            cand = np.concatenate([kv[s + 4 * (j - 1): s + 4 * j, :hd], own[:, hd:]], axis=0)
        np.testing.assert_allclose(got[n], pick(cand, axis=0), rtol=1e-9, atol=1e-12)


def test_pack_equals_segments_alone_and_tails_are_unread():
    cu, x, wkv, wgate, ape = _case(6, LENGTHS, overlap=True)
    got = oracle.compress_learned(x, wkv, wgate, ape, cu, 4, True)
    parts = []
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        parts.append(oracle.compress_learned(x[s:e], wkv, wgate, ape, np.array([0, e - s]), 4, True))
    np.testing.assert_allclose(got, np.concatenate(parts), rtol=1e-13, atol=1e-14)
    x2 = x.copy()
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        tail = (e - s) % 4
        if tail:
            x2[e - tail:e] = 1e3            # rows past the last complete group
    np.testing.assert_array_equal(oracle.compress_learned(x2, wkv, wgate, ape, cu, 4, True), got)
    assert got.shape == (sum(n // 4 for n in LENGTHS), 6)
