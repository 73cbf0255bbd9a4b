"""Pins for the oracle's 3D rotary position encoding (CPU only)."""

import numpy as np
import pytest

import oracle as O


def _rope_complex(x, F, Hg, Wg, dims, base):
    # Independent formulation: each pair (2i, 2i+1) of an axis segment is the
    # complex number a + ib, multiplied by exp(i * pos * base^(-2i/D)).
    B, N, H, d = x.shape
    out = np.empty_like(x)
    off = 0
    n = np.arange(N)
    coords = [n // (Hg * Wg), (n // Wg) % Hg, n % Wg]
    for axis, D in enumerate(dims):
        seg = x[..., off:off + D]
        z = seg[..., 0::2] + 1j * seg[..., 1::2]
        freqs = base ** (-np.arange(0, D, 2) / D)
        rot = np.exp(1j * coords[axis][:, None] * freqs[None, :])  # [N, D/2]
        z = z * rot[None, :, None, :]
        out[..., off:off + D:2] = z.real
        out[..., off + 1:off + D:2] = z.imag
        off += D
    return out


@pytest.mark.parametrize("grid,dims", [((3, 4, 5), (4, 6, 6)), ((2, 3, 3), (44, 42, 42))])
def test_rope_matches_complex_form(grid, dims):
    rng = np.random.default_rng(5)
    F, Hg, Wg = grid
    x = rng.standard_normal((2, F * Hg * Wg, 3, sum(dims)))
    np.testing.assert_allclose(O.rope_3d(x, F, Hg, Wg, dims, 10000.0),
                               _rope_complex(x, F, Hg, Wg, dims, 10000.0), rtol=0, atol=1e-12)


def test_rope_identity_at_origin_and_norm_preserving():
    rng = np.random.default_rng(6)
    F, Hg, Wg, dims = 3, 4, 5, (4, 6, 6)
    x = rng.standard_normal((1, 60, 2, 16))
    y = O.rope_3d(x, F, Hg, Wg, dims, 10000.0)
    np.testing.assert_array_equal(y[:, 0], x[:, 0])          # token 0 is position (0,0,0)
    pair_norm = lambda t: t[..., 0::2] ** 2 + t[..., 1::2] ** 2
    np.testing.assert_allclose(pair_norm(y), pair_norm(x), rtol=1e-12)
    # the first pair of each axis segment turns by exactly pos radians
    n = 1 * 20 + 2 * 5 + 3  # (f, y, x) = (1, 2, 3)
    for off, pos in ((0, 1), (4, 2), (10, 3)):
        a, b = x[0, n, 0, off], x[0, n, 0, off + 1]
        np.testing.assert_allclose(y[0, n, 0, off], a * np.cos(pos) - b * np.sin(pos), atol=1e-14)


def test_rope_scores_depend_on_offset_only():
    # <R(p) q, R(p') k> is unchanged when both positions move by one frame.
    rng = np.random.default_rng(7)
    F, Hg, Wg, dims = 4, 3, 3, (4, 6, 6)
    x = rng.standard_normal((1, 36, 1, 16))
    q, k = x[0, 2, 0], x[0, 7, 0]
    def score(nq, nk):
        t = np.zeros_like(x)
        t[0, nq, 0] = q
        t[0, nk, 0] = k
        r = O.rope_3d(t, F, Hg, Wg, dims, 10000.0)
        return r[0, nq, 0] @ r[0, nk, 0]
    np.testing.assert_allclose(score(2, 7), score(2 + 9, 7 + 9), atol=1e-12)
    np.testing.assert_allclose(score(2, 7), score(2 + 18, 7 + 18), atol=1e-12)


def test_rope_rejects_bad_dims():
    with pytest.raises(ValueError):
        O.rope_3d(np.zeros((1, 4, 1, 8)), 1, 2, 2, (2, 2, 2), 10000.0)
