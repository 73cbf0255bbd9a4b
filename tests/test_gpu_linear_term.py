"""The fused linear branch, made visible ([S] Prerequisites > Linear
Attention; [S] method steps 4-6).

With W_p ~ N(0, 0.02) the linear term s_b * (O_l W_p) of a bf16 layer is
far below the output tolerance once N reaches a few thousand tokens, so the
ordinary layer tests cannot see a mistake in it.  Here W_p is drawn with a
larger standard deviation and the term is isolated on the device as
out(s) - out(s = 0): the same inputs, once with the computed gate and once
with the gate forced to 0 (which leaves bf16(O_s)).  The oracle's term comes
from its linear state, linear apply, gate and combine.

Bar: relative Frobenius error <= 1e-2 and max |err| <= 2e-2 * max |ref|.
The difference carries two bf16 roundings of the output (each <= 2^-9 of
|out|), so W_p's scale is chosen per case to make the term large against
them (relative Frobenius of the rounding noise alone ~1e-3).  The test also
checks that the bar is sharp enough: the oracle's term with W_p transposed,
or scaled by 1/2 or 2, is rejected by it.
"""

import numpy as np
import pytest
import torch

import oracle as O
from sparse_linear_hybrid_st_amd import configs as C
from sparse_linear_hybrid_st_amd import inputs as I
from tests.gpu_util import host64, rel_fro, run_forward

pytestmark = pytest.mark.gpu

CASES = [
    (C.small("ragged-mixed", (5, 6, 7), 4, 128, "bf16", [0, 1, 2, 2], 37, 64, 2), 1.0),
    (C.small("window-multi-tile", (6, 16, 24), 2, 128, "bf16", [1, 0], 300, 64, 1, seed=9), 2.0),
    (C.small("topk-batch2", (4, 12, 20), 3, 128, "bf16", [2, 2, 2], 0, 64, 4, batch=2), 1.0),
    (C.small("rope-cfg", (3, 4, 10), 4, 128, "bf16", [0, 1, 2, 2], 20, 64, 1, batch=2, rope=True,
             rope_dims=(44, 42, 42), x_sample_shift=True), 1.0),
    (C.swa_480p(), 8.0),
]


def oracle_linear_term(w, inp, w_p=None):
    """s_b * (O_l W_p) for every (b, n, h), token order, from the oracle's
    linear branch (RoPE'd and rounded Q, K when the workload has RoPE)."""
    q, k, v, x = (I.as_f64(inp[n]) for n in ("q", "k", "v", "x"))
    wp = I.as_f64(inp["w_p"]) if w_p is None else w_p
    gw = I.as_f64(inp["gate_w"])
    out = np.empty(q.shape)
    zero = np.zeros((w.N, w.head_dim))
    for b in range(w.batch):
        s = O.gate(x[b], gw, inp["gate_b"])
        for h in range(w.n_heads):
            qh, kh = q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1]
            if w.rope:
                qh = O.round_to_io(O.rope_3d(qh, *w.grid, w.rope_dims, w.rope_base), w.io_dtype)
                kh = O.round_to_io(O.rope_3d(kh, *w.grid, w.rope_dims, w.rope_base), w.io_dtype)
            Hm, Zv = O.linear_state(kh[0, :, 0], v[b, :, h])
            o_l = O.linear_apply(qh[0, :, 0], Hm, Zv, 1e-6)
            out[b, :, h] = O.combine(zero, o_l, wp, s)
    return out


def _passes(got, ref):
    err = np.abs(got - ref)
    return rel_fro(got, ref) <= 1e-2 and err.max() <= 2e-2 * np.abs(ref).max()


@pytest.mark.parametrize("w,wp_std", CASES, ids=[c[0].name for c in CASES])
def test_fused_linear_term_visible(w, wp_std):
    print(f"[linear-term] {w.name}: N={w.N} H={w.n_heads} W_p std {wp_std}", flush=True)
    inp = I.make_inputs(w, wp_std=wp_std)
    out, s, _ = run_forward(w, inp)
    out0, _, _ = run_forward(w, inp, s_override=[0.0] * w.batch)
    got = host64(out) - host64(out0)
    ref = oracle_linear_term(w, inp)
    fro = rel_fro(got, ref)
    mx = float(np.abs(got - ref).max() / np.abs(ref).max())
    print(f"[linear-term] {w.name}: term rms {np.sqrt((ref ** 2).mean()):.3g}, rel Frobenius {fro:.3g}, "
          f"max err / max |ref| {mx:.3g}", flush=True)
    assert fro <= 1e-2, f"{w.name}: relative Frobenius {fro:.3g} > 1e-2"
    assert mx <= 2e-2, f"{w.name}: max err {mx:.3g} of max |ref| > 2e-2"
    # the bar rejects a transposed, halved or doubled term
    wp = I.as_f64(inp["w_p"])
    assert not _passes(got, oracle_linear_term(w, inp, wp.T)), "transposed W_p not rejected"
    assert not _passes(got, 0.5 * ref) and not _passes(got, 2.0 * ref), "mis-scaled term not rejected"
    # the s = 0 call is the sparse branch alone: W_p plays no part there
    inp_z = I.make_inputs(w, wp_zero=True)
    out_z, _, _ = run_forward(w, inp_z)
    assert torch.equal(out0, out_z), "s = 0 output depends on W_p"
