"""Pins for the oracle's token orders and storage rounding (CPU only)."""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _spatial_major_by_sorting(F, Hg, Wg):
    # Independent construction: list every token with its (f, y, x)
    # coordinates, then sort by (y, x, f) -- site-major, time fastest.
    toks = []
    for n in range(F * Hg * Wg):
        f, rem = divmod(n, Hg * Wg)
        y, x = divmod(rem, Wg)
        toks.append(((y, x, f), n))
    return np.array([n for _, n in sorted(toks)], dtype=np.int64)


@pytest.mark.parametrize("grid", [(4, 8, 8), (3, 5, 7), (1, 4, 6), (7, 1, 1), (20, 30, 52)])
def test_st_permutation_matches_sort_construction(grid):
    F, Hg, Wg = grid
    pi = O.st_permutation(F, Hg, Wg)
    if F * Hg * Wg <= 5000:
        np.testing.assert_array_equal(pi, _spatial_major_by_sorting(F, Hg, Wg))
    assert np.array_equal(np.sort(pi), np.arange(F * Hg * Wg))  # bijection
    # frames of one site are contiguous and ascending
    assert np.all(np.diff(pi.reshape(Hg * Wg, F), axis=1) == Hg * Wg)


def test_single_frame_is_identity():
    np.testing.assert_array_equal(O.st_permutation(1, 5, 9), np.arange(45))


def test_golden_tiny_temporal_order():
    # tests/golden/tiny_temporal_order.txt: first 24 working positions of a
    # temporal head on the 4 x 8 x 8 grid, derived by hand from the
    # re-ordering of the ijyty.com article, section 1.1.
    vals = [int(t) for t in open(os.path.join(GOLDEN, "tiny_temporal_order.txt"))
            .read().split("\n", 3)[3].split()]
    np.testing.assert_array_equal(O.st_permutation(4, 8, 8)[:len(vals)], vals)


def test_head_order_kinds():
    F, Hg, Wg = 3, 4, 5
    np.testing.assert_array_equal(O.head_order(O.HEAD_SPATIAL, F, Hg, Wg), np.arange(60))
    np.testing.assert_array_equal(O.head_order(O.HEAD_TOPK, F, Hg, Wg), np.arange(60))
    np.testing.assert_array_equal(O.head_order(O.HEAD_TEMPORAL, F, Hg, Wg),
                                  O.st_permutation(F, Hg, Wg))


def test_to_working_gathers_rows():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 12, 3, 4))
    orders = [np.arange(12), O.st_permutation(3, 2, 2), np.arange(12)[::-1].copy()]
    w = O.to_working(x, orders)
    for b in range(2):
        for h in range(3):
            for p in range(12):
                np.testing.assert_array_equal(w[b, h, p], x[b, orders[h][p], h])


# ---- bf16 rounding -------------------------------------------------------

def test_round_to_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(2)
    a = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(5000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 3.0e38, -3.3e38], np.float32),
    ])
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_to_bf16(a.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def _bf16_exact_round(x: float) -> float:
    # Brute force with exact rationals: the two bf16 neighbours of x are
    # consecutive multiples of the spacing; pick the nearer, ties to the
    # even multiple.
    fx = Fraction(x)
    m, e = np.frexp(abs(x))
    sp = Fraction(2) ** max(int(e) - 8, -133)
    lo = (fx / sp).__floor__()
    cand = [(abs(fx - lo * sp), lo % 2, lo), (abs(fx - (lo + 1) * sp), (lo + 1) % 2, lo + 1)]
    cand.sort(key=lambda c: (c[0], c[1]))
    return float(cand[0][2] * sp)


def test_round_to_bf16_exact_on_float64_values():
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.standard_normal(2000), rng.standard_normal(200) * 1e-39])
    # exact ties between bf16 neighbours: 1 + (2k+1) * 2^-8
    ties = 1.0 + (2 * np.arange(20) + 1) * 2.0 ** -8
    xs = np.concatenate([xs, ties, -ties])
    got = O.round_to_bf16(xs)
    ref = np.array([_bf16_exact_round(float(v)) for v in xs])
    np.testing.assert_array_equal(got, ref)


def test_round_to_io_f32():
    x = np.array([1.0 + 2.0 ** -30, np.pi])
    np.testing.assert_array_equal(O.round_to_io(x, "f32"), x.astype(np.float32).astype(np.float64))
