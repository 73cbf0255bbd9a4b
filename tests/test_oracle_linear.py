"""Pins for the oracle's linear branch, gate, combine and whole layer (CPU only)."""

import decimal
from decimal import Decimal
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

import oracle as O


def _brute_linear(q, k, v, eps):
    # Defining O(N^2) expansion: O_i = sum_j (phi(q_i).phi(k_j)) v_j / (sum_j phi(q_i).phi(k_j) + eps)
    pq, pk = np.maximum(q, 0), np.maximum(k, 0)
    out = np.zeros((q.shape[0], v.shape[1]))
    for i in range(q.shape[0]):
        num = np.zeros(v.shape[1])
        den = 0.0
        for j in range(k.shape[0]):
            a = float(pq[i] @ pk[j])
            num += a * v[j]
            den += a
        out[i] = num / (den + eps)
    return out


def test_linear_closed_form_equals_quadratic_expansion():
    rng = np.random.default_rng(11)
    q, k, v = rng.standard_normal((40, 6)), rng.standard_normal((40, 6)), rng.standard_normal((40, 5))
    H, Z = O.linear_state(k, v)
    np.testing.assert_allclose(O.linear_apply(q, H, Z, 1e-6), _brute_linear(q, k, v, 1e-6),
                               rtol=1e-11, atol=1e-12)


def test_linear_exact_rational():
    # small integers: the ReLU linear attention is rational, so Fractions are exact
    rng = np.random.default_rng(12)
    q = rng.integers(-3, 4, (5, 3)).astype(float)
    k = rng.integers(-3, 4, (6, 3)).astype(float)
    v = rng.integers(-5, 6, (6, 2)).astype(float)
    q[0] = [1, 2, 3]
    eps = Fraction(1, 10 ** 6)
    H, Z = O.linear_state(k, v)
    out = O.linear_apply(q, H, Z, float(eps))
    for i in range(5):
        pq = [Fraction(max(int(t), 0)) for t in q[i]]
        a = [sum(pq[c] * max(int(k[j, c]), 0) for c in range(3)) for j in range(6)]
        den = sum(a) + eps
        for c in range(2):
            ref = sum(a[j] * int(v[j, c]) for j in range(6)) / den
            assert abs(float(ref) - out[i, c]) <= 1e-15 * max(1.0, abs(float(ref)))


def test_linear_state_permutation_invariant_and_ones():
    rng = np.random.default_rng(13)
    k, v, q = rng.standard_normal((50, 4)), rng.standard_normal((50, 4)), rng.standard_normal((9, 4))
    perm = rng.permutation(50)
    H1, Z1 = O.linear_state(k, v)
    H2, Z2 = O.linear_state(k[perm], v[perm])
    np.testing.assert_allclose(H1, H2, atol=1e-12)
    np.testing.assert_allclose(Z1, Z2, atol=1e-12)
    H, Z = O.linear_state(k, np.ones((50, 3)))
    pz = np.maximum(q, 0) @ Z
    np.testing.assert_allclose(O.linear_apply(q, H, Z, 1e-6),
                               np.repeat((pz / (pz + 1e-6))[:, None], 3, 1), atol=1e-14)
    # a query with no positive feature gives zero output
    assert np.all(O.linear_apply(-np.abs(q), H, Z, 1e-6) == 0)


def test_gate_values():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((30, 8))
    assert O.gate(x, np.zeros(8), 0.0) == 0.5
    w, b = rng.standard_normal(8) * 0.1, 0.3
    decimal.getcontext().prec = 40
    m = [sum(Decimal(float(x[n, c])) for n in range(30)) / 30 for c in range(8)]
    t = sum(Decimal(float(w[c])) * m[c] for c in range(8)) + Decimal(b)
    ref = 1 / (1 + (-t).exp())
    assert abs(O.gate(x, w, b) - float(ref)) < 1e-15


def test_combine_special_cases():
    rng = np.random.default_rng(15)
    o_s, o_l, wp = rng.standard_normal((6, 4)), rng.standard_normal((6, 4)), rng.standard_normal((4, 4))
    np.testing.assert_array_equal(O.combine(o_s, o_l, np.zeros((4, 4)), 0.7), o_s)
    np.testing.assert_array_equal(O.combine(o_s, o_l, wp, 0.0), o_s)
    np.testing.assert_allclose(O.combine(o_s, o_l, np.eye(4), 1.0), o_s + o_l, atol=1e-15)
    # row vector times matrix: a W_p that maps channel 0 to channel 1 only
    e = np.zeros((4, 4))
    e[0, 1] = 1.0
    np.testing.assert_allclose(O.combine(0 * o_s, o_l, e, 1.0)[:, 1], o_l[:, 0], atol=0)


# ---- whole layer ---------------------------------------------------------

def _layer_inputs(B, grid, H, d, seed):
    rng = np.random.default_rng(seed)
    N = grid[0] * grid[1] * grid[2]
    return (rng.standard_normal((B, N, H, d)), rng.standard_normal((B, N, H, d)),
            rng.standard_normal((B, N, H, d)), rng.standard_normal((B, N, H * d)),
            rng.standard_normal((d, d)) * 0.3, rng.standard_normal(H * d) * 0.05)


def test_layer_dense_window_zero_projection_is_dense_attention():
    grid, H, d = (3, 4, 4), 3, 8
    q, k, v, x, wp, gw = _layer_inputs(2, grid, H, d, 21)
    N = 48
    res = O.attn_forward(q, k, v, x, np.zeros((d, d)), gw, 0.1, grid=grid,
                         head_kinds=[0, 1, 2], window_radius=N, block=16, topk=3,
                         io_dtype="f32")
    for b in range(2):
        for h in range(H):
            ref = Fnn.scaled_dot_product_attention(
                *(torch.from_numpy(np.ascontiguousarray(t[b, :, h]))[None, None] for t in (q, k, v))
            )[0, 0].numpy()
            np.testing.assert_allclose(res["out"][b, :, h], ref, atol=1e-12)


def test_layer_combine_and_gate_override():
    grid, H, d = (2, 3, 4), 2, 4
    q, k, v, x, wp, gw = _layer_inputs(1, grid, H, d, 22)
    kw = dict(grid=grid, head_kinds=[0, 1], window_radius=3, block=8, topk=1, io_dtype="f32")
    res = O.attn_forward(q, k, v, x, wp, gw, -0.2, **kw)
    s = O.gate(x[0], gw, -0.2)
    assert res["s"][0] == s
    np.testing.assert_allclose(res["out"], res["o_s"] + s * (res["o_l"] @ wp), atol=1e-14)
    zero = O.attn_forward(q, k, v, x, wp, gw, -0.2, s_override=[0.0], **kw)
    np.testing.assert_array_equal(zero["out"], zero["o_s"])
    # the rows form agrees with the full form
    rows = [(0, 0, 0), (0, 17, 1), (0, 23, 0)]
    part = O.attn_forward(q, k, v, x, wp, gw, -0.2, rows=rows, **kw)
    for key in rows:
        np.testing.assert_allclose(part[key], res["out"][key], atol=1e-14)


def test_layer_branch_dropping():
    """[G] 2 C: a sample whose gate value is below the threshold keeps only
    the sparse branch.  Pinned against the zero-projection layer (which has
    no linear term by construction) and against the undropped layer."""
    grid, H, d = (2, 3, 4), 2, 4
    q, k, v, x, wp, gw = _layer_inputs(2, grid, H, d, 23)
    x[1] += 3.0                                  # a second, different gate value
    kw = dict(grid=grid, head_kinds=[0, 1], window_radius=3, block=8, topk=1, io_dtype="f32")
    full = O.attn_forward(q, k, v, x, wp, gw, 0.1, **kw)
    sparse_only = O.attn_forward(q, k, v, x, np.zeros_like(wp), gw, 0.1, **kw)
    s0, s1 = full["s"]
    assert s0 != s1
    lo, hi = (0, 1) if s0 < s1 else (1, 0)
    tau = 0.5 * (s0 + s1)
    mixed = O.attn_forward(q, k, v, x, wp, gw, 0.1, drop_tau=tau, **kw)
    np.testing.assert_array_equal(mixed["out"][lo], sparse_only["out"][lo])
    np.testing.assert_array_equal(mixed["out"][hi], full["out"][hi])
    np.testing.assert_array_equal(mixed["s"], full["s"])          # s reports the gate value
    for t, ref in ((0.0, full), (1.0, sparse_only)):
        np.testing.assert_array_equal(O.attn_forward(q, k, v, x, wp, gw, 0.1, drop_tau=t, **kw)["out"],
                                      ref["out"])
    # a gate value equal to the threshold is kept (strict comparison)
    eq = O.attn_forward(q, k, v, x, wp, gw, 0.1, drop_tau=full["s"][lo], **kw)
    np.testing.assert_array_equal(eq["out"][lo], full["out"][lo])
    # the rows form agrees
    rows = [(lo, 0, 0), (lo, 17, 1), (hi, 5, 0)]
    part = O.attn_forward(q, k, v, x, wp, gw, 0.1, drop_tau=tau, rows=rows, **kw)
    for key in rows:
        np.testing.assert_allclose(part[key], mixed["out"][key], atol=1e-14)


def test_layer_full_width_projection_and_output_projection():
    """[C, C] reading of the static projection and the W^O step: a
    block-diagonal W_p with equal blocks is the per-head reading; one
    off-diagonal block moves head 0's linear output into head 1's columns
    (head-major concatenation); W_p = 0 leaves O_s; W^O = I changes nothing
    and a permutation W^O permutes the output columns."""
    grid, H, d = (2, 3, 4), 3, 4
    C = H * d
    q, k, v, x, wp, gw = _layer_inputs(1, grid, H, d, 24)
    kw = dict(grid=grid, head_kinds=[0, 1, 2], window_radius=3, block=8, topk=2, io_dtype="f32")
    head = O.attn_forward(q, k, v, x, wp, gw, 0.1, **kw)
    full = O.attn_forward(q, k, v, x, np.kron(np.eye(H), wp), gw, 0.1, proj="full", **kw)
    np.testing.assert_allclose(full["out"], head["out"], atol=1e-13)
    s = head["s"][0]
    off = np.zeros((C, C))
    off[0:d, d:2 * d] = wp                        # head 0's O_l -> head 1's columns
    cross = O.attn_forward(q, k, v, x, off, gw, 0.1, proj="full", **kw)
    np.testing.assert_allclose(cross["out"][0, :, 1],
                               head["o_s"][0, :, 1] + s * (head["o_l"][0, :, 0] @ wp), atol=1e-13)
    np.testing.assert_array_equal(cross["out"][0, :, 0], head["o_s"][0, :, 0])
    zero = O.attn_forward(q, k, v, x, np.zeros((C, C)), gw, 0.1, proj="full", **kw)
    np.testing.assert_array_equal(zero["out"], zero["o_s"])
    ident = O.attn_forward(q, k, v, x, wp, gw, 0.1, w_o=np.eye(C), **kw)
    np.testing.assert_array_equal(ident["out"], head["out"])
    perm = np.random.default_rng(5).permutation(C)
    P = np.eye(C)[:, perm]                        # column c of the result = column perm[c]
    moved = O.attn_forward(q, k, v, x, wp, gw, 0.1, w_o=P, **kw)
    np.testing.assert_array_equal(moved["out"][0].reshape(-1, C), head["out"][0].reshape(-1, C)[:, perm])
    # rows form with both cross-head steps
    w_o = np.random.default_rng(6).standard_normal((C, C)) * 0.2
    both = O.attn_forward(q, k, v, x, off + np.kron(np.eye(H), wp), gw, 0.1, proj="full", w_o=w_o, **kw)
    rows = [(0, 0, 0), (0, 13, 2), (0, 23, 1)]
    part = O.attn_forward(q, k, v, x, off + np.kron(np.eye(H), wp), gw, 0.1, proj="full", w_o=w_o,
                          rows=rows, **kw)
    for key in rows:
        np.testing.assert_allclose(part[key], both["out"][key], atol=1e-13)


def test_layer_temporal_head_is_window_on_regrouped_sequence():
    # a temporal head's output for token n equals a plain window attention on
    # the regrouped sequence, read back at n's working position
    grid, H, d = (3, 2, 3), 1, 4
    q, k, v, x, wp, gw = _layer_inputs(1, grid, H, d, 23)
    res = O.attn_forward(q, k, v, x, wp, gw, 0.0, grid=grid, head_kinds=[1], window_radius=2,
                         block=4, topk=1, io_dtype="f32")
    pi = O.st_permutation(*grid)
    qw, kw, vw = (t[0, pi, 0] for t in (q, k, v))
    N = 18
    allowed = np.abs(np.arange(N)[:, None] - np.arange(N)[None, :]) <= 2
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    ref_w = Fnn.scaled_dot_product_attention(t(qw), t(kw), t(vw),
                                             attn_mask=torch.from_numpy(allowed)[None, None])[0, 0].numpy()
    np.testing.assert_allclose(res["o_s"][0, pi, 0], ref_w, atol=1e-12)


def test_layer_dense_window_spatial_equals_temporal():
    # with a window covering everything, the token order cannot matter
    grid, H, d = (3, 2, 4), 2, 4
    q, k, v, x, wp, gw = _layer_inputs(1, grid, H, d, 24)
    q[:, :, 1], k[:, :, 1], v[:, :, 1] = q[:, :, 0], k[:, :, 0], v[:, :, 0]
    res = O.attn_forward(q, k, v, x, wp, gw, 0.0, grid=grid, head_kinds=[0, 1],
                         window_radius=100, block=8, topk=1, io_dtype="f32")
    np.testing.assert_allclose(res["out"][:, :, 0], res["out"][:, :, 1], atol=1e-12)


def test_layer_rope_is_rounded_to_storage():
    grid, H, d = (2, 2, 3), 1, 12
    q, k, v, x, wp, gw = _layer_inputs(1, grid, H, d, 25)
    res = O.attn_forward(q, k, v, x, wp, gw, 0.0, grid=grid, head_kinds=[0], window_radius=2,
                         block=4, topk=1, io_dtype="bf16", rope=True, rope_dims=(4, 4, 4))
    ref = O.round_to_bf16(O.rope_3d(q, *grid, (4, 4, 4), 10000.0))
    np.testing.assert_array_equal(res["q_used"], ref)
