"""Whole-layer parity (salad_attn_forward) against the oracle: the tiny fp32
workload, small bf16 cases with ragged tails, and the method's degenerate
cases (window 0, full window, all blocks kept, gate 0, zero projection)."""

import numpy as np
import pytest
import torch

import oracle as O
import sparse_linear_hybrid_st_amd as S
from sparse_linear_hybrid_st_amd import configs as C
from sparse_linear_hybrid_st_amd import inputs as I
from tests.gpu_util import assert_close, check_selection, host64, oracle_kwargs, run_forward

pytestmark = pytest.mark.gpu


def _oracle(w, inp, s_override=None):
    return O.attn_forward(*(I.as_f64(inp[n]) for n in ("q", "k", "v", "x", "w_p", "gate_w")),
                          inp["gate_b"], s_override=s_override, **oracle_kwargs(w))


def _check_layer(w, inp, s_override=None, what=""):
    out, s, idx = run_forward(w, inp, s_override)
    ref = _oracle(w, inp, s_override)
    if s_override is None:
        np.testing.assert_allclose(s, ref["s"], atol=1e-6, rtol=0)
    for (b, h), ridx in ref["idx"].items():
        q = ref["q_used"][b, :, h]
        k = ref["k_used"][b, :, h]
        # rows that differ must be near-ties and still a valid top-k (asserted inside)
        check_selection(idx[b, h], O.block_means(q, w.block), O.block_means(k, w.block),
                        w.topk, f"{what} b{b} h{h}")
    mx, mn = assert_close(host64(out), ref["out"], w.io_dtype, f"{what}: out")
    print(f"{what}: out max {mx:.3g} mean {mn:.3g}")
    return out, ref


@pytest.mark.parametrize("topk", [False, True])
def test_tiny_f32_layer(topk):
    w = C.tiny_f32(topk)
    _check_layer(w, I.make_inputs(w), what=w.name)


def test_tiny_f32_zero_projection_and_gate_zero_equal_sparse_only():
    w = C.tiny_f32()
    inp = I.make_inputs(w)
    zero_wp = I.make_inputs(w, wp_zero=True)
    out0, ref0 = _check_layer(w, zero_wp, what="tiny W_p=0")
    outg, refg = _check_layer(w, inp, s_override=[0.0], what="tiny s=0")
    # both reduce to the sparse branch alone: bitwise equal on the device
    assert torch.equal(out0, outg)
    np.testing.assert_allclose(host64(outg), refg["o_s"], atol=1e-4, rtol=0)


SMALL = [
    C.small("ragged-mixed", (5, 6, 7), 4, 128, "bf16", [0, 1, 2, 2], 37, 64, 2),
    C.small("window-multi-tile", (6, 16, 24), 2, 128, "bf16", [1, 0], 300, 64, 1, seed=9),
    C.small("topk-batch2", (4, 12, 20), 3, 128, "bf16", [2, 2, 2], 0, 64, 4, batch=2),
    C.small("rope-cfg", (3, 4, 10), 4, 128, "bf16", [0, 1, 2, 2], 20, 64, 1, batch=2, rope=True,
            rope_dims=(44, 42, 42), x_sample_shift=True),
    C.small("single-frame", (1, 9, 11), 2, 128, "bf16", [0, 1], 13, 64, 1),
    C.small("short", (1, 1, 37), 1, 128, "bf16", [1], 5, 64, 1),
    C.small("f32-d128-mixed", (2, 5, 9), 3, 128, "f32", [0, 1, 2], 11, 16, 2, batch=2),
    # one token: every window and every Top-K selection is that token
    C.small("one-token", (1, 1, 1), 2, 128, "bf16", [0, 2], 3, 64, 1),
    # more than 64 heads: the head masks' later words; 256 is the maximum
    C.small("70-heads", (1, 4, 20), 70, 128, "bf16", [h % 3 for h in range(70)], 9, 64, 1),
    C.small("256-heads", (1, 2, 8), 256, 128, "bf16", [h % 3 for h in range(256)], 5, 64, 1, batch=2),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_layers(w):
    _check_layer(w, I.make_inputs(w), what=w.name)


def test_degenerate_window_zero_returns_v():
    # r = 0 keeps only the diagonal: O_s = V, and W_p = 0 leaves out = V exactly
    w = C.small("r0", (2, 8, 9), 2, 128, "bf16", [0, 1], 0, 64, 1)
    inp = I.make_inputs(w, wp_zero=True)
    out, _, _ = run_forward(w, inp)
    assert torch.equal(out, inp["v"])


def test_degenerate_full_window_and_all_blocks_are_dense():
    # a window covering the sequence and k = all blocks both give dense attention
    w = C.small("dense", (2, 6, 11), 3, 128, "bf16", [0, 1, 2], 10_000, 64, 3)
    inp = I.make_inputs(w, wp_zero=True)
    out, _, idx = run_forward(w, inp)
    q, k, v = (I.as_f64(inp[n]) for n in ("q", "k", "v"))
    for h in range(3):
        ref = torch.nn.functional.scaled_dot_product_attention(
            *(torch.from_numpy(np.ascontiguousarray(t[0, :, h]))[None, None] for t in (q, k, v)))[0, 0]
        assert_close(host64(out)[0, :, h], ref.numpy(), "bf16", f"dense head {h}")
    assert np.array_equal(idx[0, 2], np.tile(np.arange(3), (3, 1)))


def test_forward_is_deterministic():
    w = SMALL[0]
    inp = I.make_inputs(w)
    a, sa, ia = run_forward(w, inp)
    b, sb, ib = run_forward(w, inp)
    assert torch.equal(a, b) and np.array_equal(sa, sb) and np.array_equal(ia, ib)


# ---- post-tuning branch dropping ([G] 2 C) ---------------------------------

DROP_CASES = [
    C.small("drop-bf16", (4, 6, 10), 4, 128, "bf16", [0, 1, 2, 2], 25, 64, 2, batch=2,
            x_sample_shift=True),
    C.small("drop-f32", (3, 4, 8), 3, 64, "f32", [0, 1, 2], 9, 16, 2, batch=2,
            x_sample_shift=True, qk_channel_scale=False),
]


@pytest.mark.parametrize("w", DROP_CASES, ids=[w.name for w in DROP_CASES])
def test_branch_dropping(w):
    """A sample whose gate value is below the threshold keeps only the
    sparse branch; the other sample is untouched.  Against the oracle, and
    bitwise against the same layer with the dropped sample's gate forced
    to 0 (no linear term) and the kept sample's gate left alone."""
    inp = I.make_inputs(w)
    full, s, _ = run_forward(w, inp)
    assert s[0] != s[1]
    lo, hi = (0, 1) if s[0] < s[1] else (1, 0)
    tau = float(0.5 * (s[0] + s[1]))
    out, s_d, _ = run_forward(w, inp, branch_drop_tau=tau)
    np.testing.assert_array_equal(s_d, s)                      # s_out reports the gate value
    assert torch.equal(out[hi], full[hi]), "kept sample changed"
    forced = [float(v) for v in s]
    forced[lo] = 0.0
    ref0, _, _ = run_forward(w, inp, s_override=forced)
    assert torch.equal(out[lo], ref0[lo]), "dropped sample is not the sparse branch alone"
    ref = O.attn_forward(*(I.as_f64(inp[n]) for n in ("q", "k", "v", "x", "w_p", "gate_w")),
                         inp["gate_b"], drop_tau=tau, **oracle_kwargs(w))
    mx, mn = assert_close(host64(out), ref["out"], w.io_dtype, f"{w.name}: dropped layer")
    print(f"{w.name}: tau {tau:.4f} (s = {s}), out max {mx:.3g} mean {mn:.3g}")
    # every sample dropped
    out_all, _, _ = run_forward(w, inp, branch_drop_tau=1.0)
    ref_all, _, _ = run_forward(w, inp, s_override=[0.0, 0.0])
    assert torch.equal(out_all, ref_all)


def test_window_radius_past_the_sequence_equals_dense_radius():
    """r = INT32_MAX keeps the same keys as r = N - 1 (the library clamps the
    radius before any window arithmetic): bitwise equal outputs."""
    w = C.small("r-huge", (2, 6, 11), 3, 128, "bf16", [0, 1, 0], 131, 64, 1)
    inp = I.make_inputs(w)
    w.window_radius = w.N - 1
    a, _, _ = run_forward(w, inp)
    w.window_radius = 2 ** 31 - 1
    b, _, _ = run_forward(w, inp)
    assert torch.equal(a, b)


GUARD = [
    C.small("guard-mixed", (5, 6, 7), 4, 128, "bf16", [0, 1, 2, 2], 37, 64, 2, batch=2),
    C.small("guard-f32", (3, 4, 8), 3, 64, "f32", [0, 1, 2], 9, 16, 2, batch=2, qk_channel_scale=False),
]


@pytest.mark.parametrize("w", GUARD, ids=[w.name for w in GUARD])
def test_outputs_stay_inside_their_buffers(w):
    """Guard bands: out, s_out, idx_out and lse_out are views into larger
    buffers filled with a sentinel; after the forward every guard element is
    unchanged and the outputs equal those of a plain call."""
    p = S.problem_from_workload(w)
    inp = I.make_inputs(w)
    q, k, v, x, wp, gw = (inp[n].cuda() for n in ("q", "k", "v", "x", "w_p", "gate_w"))
    pad = 256                                     # elements on each side (keeps 16-byte alignment)

    def guarded(shape, dtype, fill):
        n = int(np.prod(shape))
        big = torch.full((pad + n + pad,), fill, dtype=dtype, device="cuda")
        return big, big[pad:pad + n].view(shape)

    o_big, out = guarded(tuple(q.shape), q.dtype, -7.0)
    s_big, s_out = guarded((w.batch,), torch.float32, -7.0)
    i_big, idx = guarded((w.batch, w.n_heads, p.n_blocks, w.topk), torch.int32, -7)
    l_big = lse = None
    if w.io_dtype == "bf16":
        l_big, lse = guarded((w.batch, w.n_heads, w.N), torch.float32, -7.0)
    S.salad_attn_forward(p, q, k, v, x, wp, gw, inp["gate_b"], out, S.workspace(p), s_out=s_out,
                         idx_out=idx, lse_out=lse)
    torch.cuda.synchronize()
    for big, name in ((o_big, "out"), (s_big, "s_out"), (i_big, "idx_out"), (l_big, "lse_out")):
        if big is None:
            continue
        assert bool((big[:pad] == -7).all()) and bool((big[-pad:] == -7).all()), f"{name} written outside"
    ref, s_ref, _ = run_forward(w, inp)
    assert torch.equal(out.cpu(), ref) and np.array_equal(s_out.cpu().numpy(), s_ref)
