"""Pins of the window calibration oracle ([I] 1.1), CPU only: the errors
against an independent computation (torch fp64 SDPA with the window mask
and without), the dense window's zero error, and the greedy rule."""

import numpy as np
import torch

import oracle as O


def _inputs(seed=0, B=2, grid=(3, 4, 5), H=3, d=8):
    rng = np.random.default_rng(seed)
    N = int(np.prod(grid))
    # a local component so that errors fall with the window
    pos = np.arange(N)[None, :, None, None] / N
    q = rng.standard_normal((B, N, H, d)) + 3 * np.sin(6 * pos + np.arange(d))
    k = rng.standard_normal((B, N, H, d)) + 3 * np.sin(6 * pos + np.arange(d))
    v = rng.standard_normal((B, N, H, d))
    return q, k, v


def test_errors_match_masked_sdpa_and_dense_is_exact():
    q, k, v = _inputs()
    grid = (3, 4, 5)
    B, N, H, d = q.shape
    radii = [0, 2, 7, 20, N - 1]
    err, _ = O.calibrate_windows(q, k, v, grid=grid, head_kinds=[0, 1, 2], radii=radii, tau=0.5)
    assert np.all(err[-1] <= 1e-28)                  # the dense window is dense attention
    for h, kind in enumerate([0, 1, 2]):
        order = O.head_order(kind, *grid)
        for b in range(B):
            qt, kt, vt = (torch.tensor(t[b, order, h])[None, None] for t in (q, k, v))
            od = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0].numpy()
            for i, r in enumerate(radii):
                idx = np.arange(N)
                mask = torch.tensor(np.abs(idx[:, None] - idx[None, :]) <= r)
                ow = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)[0, 0].numpy()
                ref = np.sum((ow - od) ** 2) / np.sum(od ** 2)
                assert abs(err[i, b, h] - ref) <= 1e-12 * max(1.0, ref)


def test_greedy_choice_is_smallest_radius_meeting_the_bound():
    q, k, v = _inputs(seed=1)
    N = q.shape[1]
    radii = [1, 3, 6, 12, 30]
    for tau in (0.0, 0.05, 0.3, 1.0, 5.0):
        err, choice = O.calibrate_windows(q, k, v, grid=(3, 4, 5), head_kinds=[0, 1, 2], radii=radii,
                                          tau=tau)
        for h in range(3):
            ok = [i for i in range(len(radii)) if err[i, :, h].max() <= tau]
            assert choice[h] == (radii[ok[0]] if ok else N - 1)
    # the bound is on the worst sample: raising one sample's error past tau
    # moves the choice
    err, choice = O.calibrate_windows(q, k, v, grid=(3, 4, 5), head_kinds=[0, 1, 2], radii=radii, tau=0.3)
    h = 0
    i = radii.index(choice[h]) if choice[h] in radii else None
    if i is not None:
        assert err[i, :, h].max() <= 0.3 and (i == 0 or err[i - 1, :, h].max() > 0.3)
