"""Pins of the backward oracle (oracle/salad_backward.py), CPU only.

The backward is the derivative of the forward oracle, so it is pinned
against the forward itself by central finite differences: for the scalar
L = sum(dout * out), the change of L along a random direction E of one input
must equal <dL/dinput, E>.  The forward runs with no storage rounding
("f64") so that it is a smooth function of its inputs; the checks assert
that the perturbation crosses no ReLU kink, Top-K selection change or drop
threshold.  A second, independent pin: with W_p = 0 the sparse branch's
gradients equal torch's autograd of masked SDPA in fp64 per head."""

import numpy as np
import pytest
import torch

import oracle as O

EPS = 1e-5


def _problem(rope, seed=0, B=2, grid=(2, 3, 4), H=3, d=8):
    rng = np.random.default_rng(seed)
    N = int(np.prod(grid))
    C = H * d
    q = rng.standard_normal((B, N, H, d))
    k = rng.standard_normal((B, N, H, d))
    v = rng.standard_normal((B, N, H, d))
    x = rng.standard_normal((B, N, C)) + rng.standard_normal((B, 1, 1))
    wp = rng.standard_normal((d, d)) * 0.3
    gw = rng.standard_normal(C) * 0.3
    G = rng.standard_normal((B, N, H, d))
    kw = dict(grid=grid, head_kinds=[0, 1, 2], window_radius=3, block=8, topk=2, io_dtype="f64",
              rope=rope, rope_dims=(4, 2, 2), rope_base=100.0)
    return dict(q=q, k=k, v=v, x=x, w_p=wp, gate_w=gw, gate_b=0.1), G, kw


def _loss(inp, G, kw, **extra):
    f = O.attn_forward(inp["q"], inp["k"], inp["v"], inp["x"], inp["w_p"], inp["gate_w"],
                       inp["gate_b"], **kw, **extra)
    return float(np.sum(G * f["out"])), f


def _check_fd(inp, G, kw, names=("q", "k", "v", "x", "w_p", "gate_w", "gate_b"), seed=1, **extra):
    grads = O.attn_backward(inp["q"], inp["k"], inp["v"], inp["x"], inp["w_p"], inp["gate_w"],
                            inp["gate_b"], G, **kw, **extra)
    key = {"q": "dq", "k": "dk", "v": "dv", "x": "dx", "w_p": "dw_p", "gate_w": "dgate_w",
           "gate_b": "dgate_b"}
    _, base = _loss(inp, G, kw, **extra)
    rng = np.random.default_rng(seed)
    for n in names:
        E = rng.standard_normal(np.shape(inp[n]))
        plus, minus = dict(inp), dict(inp)
        plus[n] = inp[n] + EPS * E
        minus[n] = inp[n] - EPS * E
        lp, fp = _loss(plus, G, kw, **extra)
        lm, fm = _loss(minus, G, kw, **extra)
        # the perturbation crosses none of the kinks the derivative ignores
        for f_ in (fp, fm):
            for key_ in base["idx"]:
                assert np.array_equal(f_["idx"][key_], base["idx"][key_])
            for t in ("q_used", "k_used"):
                assert np.array_equal(f_[t] > 0, base[t] > 0)
        fd = (lp - lm) / (2 * EPS)
        an = float(np.sum(np.asarray(grads[key[n]]) * E))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), f"{n}: finite difference {fd!r} vs {an!r}"
    return grads


@pytest.mark.parametrize("rope", [False, True])
def test_backward_matches_finite_differences(rope):
    inp, G, kw = _problem(rope)
    _check_fd(inp, G, kw)


def test_backward_with_one_sample_dropped():
    inp, G, kw = _problem(False, seed=3)
    s = np.array([O.gate(inp["x"][b], inp["gate_w"], inp["gate_b"]) for b in range(2)])
    assert abs(s[0] - s[1]) > 1e-3
    tau = float(s.mean())
    g = _check_fd(inp, G, kw, drop_tau=tau)
    lo = int(np.argmin(s))
    assert g["ds"][lo] == 0.0 and np.all(g["dx"][lo] == 0.0)
    assert g["ds"][1 - lo] != 0.0


def test_gate_override_reports_ds():
    inp, G, kw = _problem(True, seed=4)
    s0 = np.array([0.3, 0.7])
    g = _check_fd(inp, G, kw, names=("q", "k", "v", "w_p"), s_override=s0)
    assert np.all(g["dx"] == 0.0) and np.all(g["dgate_w"] == 0.0) and g["dgate_b"] == 0.0
    for b in range(2):
        e = np.zeros(2)
        e[b] = EPS
        lp, _ = _loss(inp, G, kw, s_override=s0 + e)
        lm, _ = _loss(inp, G, kw, s_override=s0 - e)
        fd = (lp - lm) / (2 * EPS)
        assert abs(fd - g["ds"][b]) <= 1e-6 * max(1.0, abs(fd))


def test_rope_transpose_inverts_rotation():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 24, 2, 8))
    r = O.rope_3d(x, 2, 3, 4, (4, 2, 2), 100.0)
    np.testing.assert_allclose(O.rope_3d_transpose(r, 2, 3, 4, (4, 2, 2), 100.0), x, atol=1e-13)


def test_sparse_gradients_match_torch_autograd_with_zero_projection():
    """W_p = 0 removes the linear branch's output: dQ, dK, dV are those of
    masked softmax attention, per head, from torch's autograd."""
    inp, G, kw = _problem(False, seed=6)
    inp["w_p"] = np.zeros_like(inp["w_p"])
    g = O.attn_backward(inp["q"], inp["k"], inp["v"], inp["x"], inp["w_p"], inp["gate_w"],
                        inp["gate_b"], G, **kw)
    f = O.attn_forward(inp["q"], inp["k"], inp["v"], inp["x"], inp["w_p"], inp["gate_w"],
                       inp["gate_b"], **kw)
    B, N, H, d = inp["q"].shape
    for b in range(B):
        for h in range(H):
            order = f["orders"][h]
            kind = kw["head_kinds"][h]
            mask = np.zeros((N, N), dtype=bool)
            if kind == 2:
                idx = f["idx"][(b, h)]
                for p in range(N):
                    mask[p, O.topk_keys(p, idx, kw["block"], N)] = True
            else:
                for p in range(N):
                    mask[p, O.swa_keys(p, N, kw["window_radius"])] = True
            qt, kt, vt = (torch.tensor(t[b, order, h], requires_grad=True)
                          for t in (inp["q"], inp["k"], inp["v"]))
            o = torch.nn.functional.scaled_dot_product_attention(
                qt[None, None], kt[None, None], vt[None, None], attn_mask=torch.tensor(mask))[0, 0]
            o.backward(torch.tensor(G[b, order, h]))
            np.testing.assert_allclose(g["dq"][b, order, h], qt.grad.numpy(), atol=1e-12)
            np.testing.assert_allclose(g["dk"][b, order, h], kt.grad.numpy(), atol=1e-12)
            np.testing.assert_allclose(g["dv"][b, order, h], vt.grad.numpy(), atol=1e-12)
    # W_p = 0: the gate's output does not reach the layer, so no gradient reaches it
    assert np.all(g["ds"] == 0.0) and np.all(g["dx"] == 0.0)


@pytest.mark.parametrize("rope,drop", [(False, False), (True, False), (True, True)])
def test_rows_mode_equals_full_backward(rope, drop):
    """The rows form (used at full workload sizes) gives the full form's
    rows and whole-layer gradients."""
    inp, G, kw = _problem(rope, seed=8)
    extra = {}
    if drop:
        s = np.array([O.gate(inp["x"][b], inp["gate_w"], inp["gate_b"]) for b in range(2)])
        extra["drop_tau"] = float(s.mean())
    args = [inp[n] for n in ("q", "k", "v", "x", "w_p", "gate_w")] + [inp["gate_b"], G]
    full = O.attn_backward(*args, **kw, **extra)
    rng = np.random.default_rng(9)
    B, N, H, _ = inp["q"].shape
    rows = sorted({(int(rng.integers(B)), int(rng.integers(N)), int(rng.integers(H))) for _ in range(12)}
                  | {(0, 0, 2), (1, N - 1, 1), (0, 7, 0)})
    part = O.attn_backward_rows(*args, rows_q=rows, rows_kv=rows, **kw, **extra)
    for key in rows:
        b, n, h = key
        np.testing.assert_allclose(part["dq"][key], full["dq"][b, n, h], atol=1e-12)
        np.testing.assert_allclose(part["dk"][key], full["dk"][b, n, h], atol=1e-12)
        np.testing.assert_allclose(part["dv"][key], full["dv"][b, n, h], atol=1e-12)
    for name in ("dw_p", "dgate_w", "ds"):
        np.testing.assert_allclose(part[name], full[name], atol=1e-12)
    assert abs(part["dgate_b"] - full["dgate_b"]) <= 1e-12
