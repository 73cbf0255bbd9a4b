"""Pins for the oracle's sparse branch and Top-K selection (CPU only).

The window and Top-K forms are checked against torch's CPU
scaled_dot_product_attention in float64 with the {-inf, 0} mask written
out from its definition, against exact high-precision brute force, and
against the special cases that reduce to dense attention or to V.
"""

import decimal
from decimal import Decimal

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

import oracle as O


def _sdpa(q, k, v, allowed=None, scale=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float64))[None, None]
    mask = None if allowed is None else torch.from_numpy(allowed)[None, None]
    return Fnn.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask,
                                            scale=scale)[0, 0].numpy()


def _window_mask(N, r):
    i = np.arange(N)
    return np.abs(i[:, None] - i[None, :]) <= r


def _qkv(N, d, seed, dv=None):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, d)), rng.standard_normal((N, d)),
            rng.standard_normal((N, dv or d)))


def test_window_radius_zero_returns_v():
    q, k, v = _qkv(37, 8, 1)
    out = O.sparse_attention(q, k, v, lambda p: O.swa_keys(p, 37, 0), 0.3)
    np.testing.assert_array_equal(out, v)


@pytest.mark.parametrize("N,r", [(50, 49), (50, 200), (1, 0)])
def test_full_window_is_dense_attention(N, r):
    q, k, v = _qkv(N, 16, 2)
    out = O.sparse_attention(q, k, v, lambda p: O.swa_keys(p, N, r), 0.25)
    np.testing.assert_allclose(out, _sdpa(q, k, v, scale=0.25), rtol=0, atol=1e-12)


@pytest.mark.parametrize("N,r", [(64, 5), (100, 17), (33, 1)])
def test_window_matches_masked_dense(N, r):
    q, k, v = _qkv(N, 8, 3)
    out = O.sparse_attention(q, k, v, lambda p: O.swa_keys(p, N, r), 1 / np.sqrt(8))
    np.testing.assert_allclose(out, _sdpa(q, k, v, _window_mask(N, r)), rtol=0, atol=1e-12)


def test_window_matches_high_precision_brute_force():
    # softmax attention written out with 40-digit decimals (exp correctly rounded)
    decimal.getcontext().prec = 40
    N, d, r, scale = 7, 3, 2, 0.5
    q, k, v = _qkv(N, d, 4)
    out = O.sparse_attention(q, k, v, lambda p: O.swa_keys(p, N, r), scale)
    D = lambda a: Decimal(float(a))
    for i in range(N):
        keys = [j for j in range(N) if abs(i - j) <= r]
        logit = [D(scale) * sum(D(q[i, c]) * D(k[j, c]) for c in range(d)) for j in keys]
        w = [x.exp() for x in logit]
        tot = sum(w)
        for c in range(d):
            ref = sum(wj * D(v[j, c]) for wj, j in zip(w, keys)) / tot
            assert abs(float(ref) - out[i, c]) < 1e-13


def test_rows_subset_and_pair_counts():
    N, r = 90, 11
    q, k, v = _qkv(N, 4, 5)
    full = O.sparse_attention(q, k, v, lambda p: O.swa_keys(p, N, r), 0.5)
    part = O.sparse_attention(q, k, v, lambda p: O.swa_keys(p, N, r), 0.5, rows=[0, 45, 89])
    np.testing.assert_array_equal(part, full[[0, 45, 89]])
    for NN, rr in ((90, 11), (31200, 1601), (10, 30), (75600, 3880)):
        if NN <= 2000:
            assert O.swa_pair_count(NN, rr) == int(_window_mask(NN, rr).sum())
    # 90 % sparsity radii of the 480p and 720p-like lengths (closed form)
    assert O.swa_pair_count(31200, 1601) >= 0.1 * 31200 ** 2 > O.swa_pair_count(31200, 1600)
    assert O.swa_pair_count(75600, 3880) >= 0.1 * 75600 ** 2 > O.swa_pair_count(75600, 3879)


# ---- Top-K --------------------------------------------------------------

def test_block_means_even_and_tail():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((128, 5))
    np.testing.assert_allclose(O.block_means(x, 32), x.reshape(4, 32, 5).mean(axis=1), atol=1e-15)
    y = rng.standard_normal((100, 3))
    m = O.block_means(y, 32)
    assert m.shape == (4, 3)
    np.testing.assert_allclose(m[3], y[96:].mean(axis=0), atol=1e-15)


def _brute_topk(qbar, kbar, k):
    out = []
    for a in range(qbar.shape[0]):
        sc = [(-float(np.dot(qbar[a], kbar[b])), b) for b in range(kbar.shape[0])]
        out.append(sorted(b for _, b in sorted(sc)[:k]))
    return np.array(out)


@pytest.mark.parametrize("nb,k", [(8, 2), (13, 5), (16, 16), (9, 1)])
def test_topk_matches_brute_force(nb, k):
    rng = np.random.default_rng(nb * 10 + k)
    qbar, kbar = rng.standard_normal((nb, 6)), rng.standard_normal((nb, 6))
    np.testing.assert_array_equal(O.topk_blocks(qbar, kbar, k), _brute_topk(qbar, kbar, k))


def test_topk_ties_prefer_lower_index_and_planted_block():
    qbar = np.ones((3, 2))
    kbar = np.array([[1.0, 0], [0, 1.0], [0.5, 0.5], [1.0, 0.0], [2.0, 2.0]])
    # scores 1, 1, 1, 1, 4: block 4 wins, then the lowest-index ties
    np.testing.assert_array_equal(O.topk_blocks(qbar, kbar, 3), [[0, 1, 4]] * 3)
    rng = np.random.default_rng(8)
    qb, kb = np.abs(rng.standard_normal((20, 4))), rng.standard_normal((20, 4))
    kb[13] = 50.0  # aligned with every (positive) query mean
    assert all(13 in row for row in O.topk_blocks(qb, kb, 1))
    assert O.topk_gap(qb, kb, 20)[0] == np.inf


def test_topk_all_blocks_is_dense():
    N, bs, d = 70, 16, 8
    q, k, v = _qkv(N, d, 9)
    out, idx = O.sparse_attention_head(O.HEAD_TOPK, q, k, v, r=0, bs=bs, k=5, scale=1 / np.sqrt(d))
    np.testing.assert_array_equal(idx, np.tile(np.arange(5), (5, 1)))
    np.testing.assert_allclose(out, _sdpa(q, k, v), rtol=0, atol=1e-12)


def test_topk_matches_masked_dense():
    N, bs, d, k = 100, 16, 8, 3
    q, k_, v = _qkv(N, d, 10)
    out, idx = O.sparse_attention_head(O.HEAD_TOPK, q, k_, v, r=0, bs=bs, k=k, scale=1 / np.sqrt(d))
    allowed = np.zeros((N, N), bool)
    for p in range(N):
        for kb in idx[p // bs]:
            allowed[p, kb * bs:min(N, (kb + 1) * bs)] = True
    np.testing.assert_allclose(out, _sdpa(q, k_, v, allowed), rtol=0, atol=1e-12)
    assert O.topk_pair_count(idx, bs, N) == int(allowed.sum())


def test_topk_gap_finite_values():
    """The gap between the k-th and (k+1)-th best block scores ([I] 1.2 keeps
    the k best; a smaller gap means the choice hangs on rounding), checked on
    hand-built score rows: qbar = 1 and kbar = diag(values) make the scores of
    row 0 the listed values exactly."""
    vals = np.array([5.0, 3.0, 9.0, 3.5, 1.0])
    qbar = np.ones((1, 5))
    kbar = np.diag(vals)
    # descending 9, 5, 3.5, 3, 1: k = 2 compares 5 with 3.5 -> 1.5 / 5
    assert O.topk_gap(qbar, kbar, 2)[0] == 0.3
    # k = 1 compares 9 with 5 -> 4 / 9; k = 4 compares 3 with 1 -> 2 / 3
    assert O.topk_gap(qbar, kbar, 1)[0] == 4.0 / 9.0
    assert O.topk_gap(qbar, kbar, 4)[0] == 2.0 / 3.0
    # negative scores: the larger magnitude scales the gap
    neg = np.diag(np.array([-1.0, -4.0, -2.0]))
    assert O.topk_gap(np.ones((1, 3)), neg, 1)[0] == 0.5      # -1 vs -2 -> 1 / 2
    assert O.topk_gap(np.ones((1, 3)), neg, 2)[0] == 0.5      # -2 vs -4 -> 2 / 4
    # an exact tie at the boundary gives 0, whatever the other scores
    tie = np.diag(np.array([7.0, 2.0, 7.0, 2.0]))
    assert O.topk_gap(np.ones((1, 4)), tie, 1)[0] == 0.0
    assert O.topk_gap(np.ones((1, 4)), tie, 3)[0] == 0.0
    # several rows at once (row r scales the scores by r + 1: same gaps)
    q3 = np.array([[1.0] * 5, [2.0] * 5, [3.0] * 5])
    np.testing.assert_array_equal(O.topk_gap(q3, kbar, 2), [0.3, 0.3, 0.3])


def test_topk_gap_matches_exact_rational_brute_force():
    """Random small integer means: every score is an exact integer, so the
    gap can be formed in exact rationals from a Python sort."""
    from fractions import Fraction
    rng = np.random.default_rng(31)
    qbar = rng.integers(-4, 5, size=(9, 3)).astype(np.float64)
    kbar = rng.integers(-4, 5, size=(11, 3)).astype(np.float64)
    for k in (1, 3, 5, 10):
        got = O.topk_gap(qbar, kbar, k)
        for a in range(qbar.shape[0]):
            sc = sorted((int(np.dot(qbar[a], kbar[b])) for b in range(kbar.shape[0])), reverse=True)
            hi, lo = sc[k - 1], sc[k]
            den = max(abs(hi), abs(lo))
            ref = Fraction(hi - lo, den) if den else Fraction(0)
            assert got[a] == float(ref), (k, a, got[a], ref)
