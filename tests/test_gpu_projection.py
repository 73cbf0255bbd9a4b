"""Full-width [C, C] static projection and the output projection W^O
(SALAD structured summary, method steps 4 and 7) on the device, against the
oracle's ``combine_full`` / ``output_projection`` readings.

The layer in full-width mode writes O_s and s_b * O_l (both rounded to the
storage type) and one GEMM over the B*N token rows adds (s_b O_l) W_p, so
its error budget is that of the per-head layer plus one storage rounding of
s_b * O_l before the product; the bf16 bar stays max |err| <= 2e-2,
mean <= 2e-3, the f32 bar 1e-4."""

import numpy as np
import pytest
import torch

import oracle as O
import sparse_linear_hybrid_st_amd as S
from sparse_linear_hybrid_st_amd import configs as C
from sparse_linear_hybrid_st_amd import inputs as I
from tests.gpu_util import assert_close, dev, host64, oracle_kwargs, run_forward

pytestmark = pytest.mark.gpu

FULL_CASES = [
    C.small("full-ragged-mixed", (5, 6, 7), 4, 128, "bf16", [0, 1, 2, 2], 37, 64, 2),
    C.small("full-window-multi-tile", (6, 16, 24), 2, 128, "bf16", [1, 0], 300, 64, 1, seed=9),
    C.small("full-rope-cfg", (3, 4, 10), 4, 128, "bf16", [0, 1, 2, 2], 20, 64, 1, batch=2,
            rope=True, rope_dims=(44, 42, 42), x_sample_shift=True),
    C.small("full-f32-d64", (3, 4, 8), 3, 64, "f32", [0, 1, 2], 9, 16, 2, batch=2,
            x_sample_shift=True, qk_channel_scale=False),
    C.small("full-f32-d128", (2, 5, 9), 3, 128, "f32", [0, 1, 2], 11, 16, 2, batch=2),
    # 1,056 token rows: the GEMM's 256-row bands, the last one ragged
    C.small("full-bf16-1056rows", (4, 6, 11), 4, 128, "bf16", [0, 1, 2, 2], 9, 64, 2, batch=4),
    # C = 640: the last 256-column tile is half wide (its upper waves store
    # nothing); 378 rows: two row bands, the second ragged
    C.small("full-bf16-c640-ragged", (3, 7, 9), 5, 128, "bf16", [0, 1, 2, 0, 1], 20, 64, 2, batch=2),
    # one head, C = 128: a single half-wide column tile
    C.small("full-bf16-one-head", (4, 5, 6), 1, 128, "bf16", [1], 10, 64, 1, batch=2),
]


def _args(inp):
    return [I.as_f64(inp[n]) for n in ("q", "k", "v", "x", "w_p", "gate_w")]


@pytest.mark.parametrize("w", FULL_CASES, ids=[w.name for w in FULL_CASES])
def test_full_width_layer(w):
    inp = I.make_inputs(w, proj="full")
    out, s, _ = run_forward(w, inp, proj="full")
    ref = O.attn_forward(*_args(inp), inp["gate_b"], proj="full", **oracle_kwargs(w))
    np.testing.assert_allclose(s, ref["s"], atol=1e-6, rtol=0)
    mx, mn = assert_close(host64(out), ref["out"], w.io_dtype, f"{w.name}: out")
    print(f"{w.name}: out max {mx:.3g} mean {mn:.3g}")


@pytest.mark.parametrize("w", FULL_CASES[:1] + FULL_CASES[3:4], ids=["bf16", "f32"])
def test_block_diagonal_full_width_equals_per_head(w):
    """W_p = diag(w_p, ..., w_p) in full-width mode is the per-head layer."""
    inp = I.make_inputs(w)
    head, _, _ = run_forward(w, inp)
    blk = dict(inp)
    wp = I.as_f64(inp["w_p"])
    blk["w_p"] = I.to_storage(np.kron(np.eye(w.n_heads), wp), w.io_dtype)
    full, _, _ = run_forward(w, blk, proj="full")
    ref = O.attn_forward(*_args(inp), inp["gate_b"], **oracle_kwargs(w))
    assert_close(host64(full), ref["out"], w.io_dtype, f"{w.name}: block-diagonal full")
    assert_close(host64(full), host64(head), w.io_dtype, f"{w.name}: full vs per-head")


@pytest.mark.parametrize("w", [FULL_CASES[2], FULL_CASES[3]], ids=["bf16", "f32"])
def test_full_width_gate_zero_and_dropping(w):
    """Gate 0 and a dropped sample leave O_s alone, bit for bit the same as
    the per-head layer's sparse-only output; the kept sample matches the
    oracle's full-width layer."""
    inp = I.make_inputs(w, proj="full")
    head_inp = I.make_inputs(w)
    _, s, _ = run_forward(w, inp, proj="full")
    zero_full, _, _ = run_forward(w, inp, s_override=[0.0] * w.batch, proj="full")
    zero_head, _, _ = run_forward(w, head_inp, s_override=[0.0] * w.batch)
    assert torch.equal(zero_full, zero_head)
    lo, hi = (0, 1) if s[0] < s[1] else (1, 0)
    tau = float(0.5 * (s[0] + s[1]))
    out, s_d, _ = run_forward(w, inp, branch_drop_tau=tau, proj="full")
    np.testing.assert_array_equal(s_d, s)
    assert torch.equal(out[lo], zero_head[lo]), "dropped sample is not O_s alone"
    ref = O.attn_forward(*_args(inp), inp["gate_b"], proj="full", drop_tau=tau, **oracle_kwargs(w))
    assert_close(host64(out), ref["out"], w.io_dtype, f"{w.name}: full-width, one sample dropped")


@pytest.mark.parametrize("io_dtype,grid,head_dim", [("bf16", (3, 5, 7), 128), ("f32", (3, 5, 7), 64),
                                                   ("bf16", (6, 7, 9), 128)],
                         ids=["bf16-c384", "f32-c192", "bf16-c384-756rows"])
def test_output_projection(io_dtype, grid, head_dim):
    bf16 = io_dtype == "bf16"
    w = C.small("wo", grid, 3, head_dim, io_dtype, [0, 1, 2], 9, 64 if bf16 else 16, 2, batch=2)
    p = S.problem_from_workload(w)
    x = I.make_inputs(w)["v"]                       # any [B, N, C] storage-type tensor
    w_o = I.make_w_o(w)
    out = torch.empty_like(dev(x))
    S.salad_output_projection(p, dev(x), dev(w_o), out)
    torch.cuda.synchronize()
    C_ = w.n_heads * w.head_dim
    ref = O.output_projection(I.as_f64(x).reshape(-1, C_), I.as_f64(w_o)).reshape(x.shape)
    # |ref| ~ 1: bf16 output rounding is up to 2^-8 relative
    assert_close(host64(out), ref, io_dtype, f"W^O {io_dtype}", max_abs=3e-2 if io_dtype == "bf16" else 1e-4,
                 mean_abs=4e-3 if io_dtype == "bf16" else None)


def test_layer_then_output_projection():
    """Full-width layer followed by W^O against the oracle's layer with w_o."""
    w = FULL_CASES[0]
    inp = I.make_inputs(w, proj="full")
    p = S.problem_from_workload(w, proj="full")
    d = {n: dev(inp[n]) for n in ("q", "k", "v", "x", "w_p", "gate_w")}
    w_o = I.make_w_o(w)
    mid = torch.empty_like(d["q"])
    S.salad_attn_forward(p, d["q"], d["k"], d["v"], d["x"], d["w_p"], d["gate_w"], inp["gate_b"], mid,
                         S.workspace(p))
    out = torch.empty_like(mid)
    S.salad_output_projection(p, mid, dev(w_o), out)
    torch.cuda.synchronize()
    ref = O.attn_forward(*_args(inp), inp["gate_b"], proj="full", w_o=I.as_f64(w_o), **oracle_kwargs(w))
    # W^O mixes C = 512 rounded values of size ~|O| into each output
    assert_close(host64(out), ref["out"], "bf16", "layer + W^O", max_abs=3e-2, mean_abs=4e-3)


def test_output_projection_rejects_overlap():
    w = C.small("wo-overlap", (2, 2, 2), 1, 128, "bf16", [0], 1, 64, 1)
    p = S.problem_from_workload(w)
    x = torch.zeros((1, 8, 1, 128), dtype=torch.bfloat16, device="cuda")
    w_o = torch.zeros((128, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(S.SaladError, match="overlap"):
        S.salad_output_projection(p, x, w_o, x)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_full_width_480p_window_12_heads_sampled_tokens():
    """The 480p window workload (N = 31,200, C = 1536) with the full-width
    projection, as bench.py --proj full runs it: whole token rows (every
    head) at edge and random tokens against the oracle."""
    w = C.swa_480p()
    inp = I.make_inputs(w, proj="full")
    out, s, _ = run_forward(w, inp, proj="full")
    rng = np.random.default_rng(3)
    toks = sorted({0, 1, 127, 128, w.N // 2, w.N - 1, *rng.integers(w.N, size=10).tolist()})
    rows = [(0, int(n), h) for n in toks for h in range(w.n_heads)]
    args = [inp[n].float().numpy() for n in ("q", "k", "v", "x")] + \
        [I.as_f64(inp[n]) for n in ("w_p", "gate_w")]
    ref = O.attn_forward(*args, inp["gate_b"], rows=rows, proj="full", **oracle_kwargs(w))
    got = host64(out)
    err = np.stack([np.abs(got[b, n, h] - ref[(b, n, h)]) for (b, n, h) in rows])
    print(f"full-width 480p: {len(toks)} tokens, max {err.max():.3g} mean {err.mean():.3g}, s = {s}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
