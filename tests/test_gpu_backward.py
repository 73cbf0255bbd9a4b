"""Backward parity (salad_attn_backward) against the oracle's attn_backward,
on small bf16 layers with ragged tails, every head kind, RoPE, a CFG pair,
branch dropping and a fixed gate.

Tolerances.  The device computes in bf16 MFMA operands with fp32
accumulation: P and dS are rounded to bf16 (relative 2^-9) before the
products, M = H W_p and dH are rounded to bf16 for the linear branch, and
dQ, dK, dV, dX are stored in bf16 (relative 2^-9).  Each gradient is
therefore compared relative to its own scale: max |err| <= 2e-2 * max|ref|
and ||err|| <= 1e-2 * ||ref|| (Frobenius); the fp32 reductions dW_p,
dgate_w, dgate_b and ds meet the same relative bar."""

import numpy as np
import pytest
import torch

import oracle as O
import sparse_linear_hybrid_st_amd as S
from sparse_linear_hybrid_st_amd import configs as C
from sparse_linear_hybrid_st_amd import inputs as I
from tests.gpu_util import dev, host64, oracle_kwargs

pytestmark = pytest.mark.gpu

MAX_REL, FRO_REL = 2e-2, 1e-2

CASES = [
    C.small("bwd-ragged-mixed", (5, 6, 7), 4, 128, "bf16", [0, 1, 2, 2], 37, 64, 2),
    C.small("bwd-window-multi-tile", (6, 16, 24), 2, 128, "bf16", [1, 0], 300, 64, 1, seed=9),
    C.small("bwd-topk-batch2", (4, 12, 20), 3, 128, "bf16", [2, 2, 2], 0, 64, 4, batch=2),
    C.small("bwd-rope-cfg", (3, 4, 10), 4, 128, "bf16", [0, 1, 2, 2], 20, 64, 1, batch=2, rope=True,
            rope_dims=(44, 42, 42), x_sample_shift=True),
    C.small("bwd-short", (1, 1, 37), 1, 128, "bf16", [1], 5, 64, 1),
    # more than 64 heads (the head masks' later words), RoPE and two samples
    C.small("bwd-70-heads", (2, 4, 10), 70, 128, "bf16", [h % 3 for h in range(70)], 9, 64, 1, batch=2,
            rope=True, rope_dims=(44, 42, 42)),
]


def _dout(w):
    rng = np.random.default_rng(w.seed + 77)
    g = rng.standard_normal((w.batch, w.N, w.n_heads, w.head_dim)).astype(np.float32)
    return I.to_storage(g, w.io_dtype)


def run_backward(w, inp, dout, s_override=None, branch_drop_tau=0.0, saved=False, repeat=False):
    """salad_attn_backward on the device; with saved=True the forward runs
    first and its out and row normalisers are handed to the backward.  With
    repeat=True the backward runs a second time into fresh buffers (same
    workspace) and every output must equal the first call's bit for bit: a
    race between waves or a read of memory the call did not write shows up
    as a difference."""
    p = S.problem_from_workload(w, branch_drop_tau=branch_drop_tau)
    d = {n: dev(inp[n]) for n in ("q", "k", "v", "x", "w_p", "gate_w")}
    go = dev(dout)
    so = None if s_override is None else torch.tensor(s_override, dtype=torch.float32, device="cuda")
    out = lse = None
    if saved:
        out = torch.empty_like(d["q"])
        lse = torch.empty((w.batch, w.n_heads, w.N), dtype=torch.float32, device="cuda")
        S.salad_attn_forward(p, d["q"], d["k"], d["v"], d["x"], d["w_p"], d["gate_w"], inp["gate_b"], out,
                             S.workspace(p), s_override=so, lse_out=lse)
    dq, dk, dv = (torch.empty_like(d["q"]) for _ in range(3))
    dx = torch.empty_like(d["x"])
    dwp = torch.empty((w.head_dim, w.head_dim), dtype=torch.float32, device="cuda")
    dgw = torch.empty(w.n_heads * w.head_dim, dtype=torch.float32, device="cuda")
    dgb = torch.empty(1, dtype=torch.float32, device="cuda")
    ds = torch.empty(w.batch, dtype=torch.float32, device="cuda")
    bws = S.backward_workspace(p)
    S.salad_attn_backward(p, d["q"], d["k"], d["v"], d["x"], d["w_p"], d["gate_w"], inp["gate_b"], go,
                          dq, dk, dv, dwp, bws, dx=dx, dgate_w=dgw, dgate_b=dgb, ds=ds,
                          s_override=so, out_saved=out, lse_saved=lse)
    torch.cuda.synchronize()
    if repeat:
        first = {"dq": dq, "dk": dk, "dv": dv, "dx": dx, "dw_p": dwp, "dgate_w": dgw, "dgate_b": dgb, "ds": ds}
        again = {n: torch.full_like(t, float("nan")) for n, t in first.items()}
        S.salad_attn_backward(p, d["q"], d["k"], d["v"], d["x"], d["w_p"], d["gate_w"], inp["gate_b"], go,
                              again["dq"], again["dk"], again["dv"], again["dw_p"], bws, dx=again["dx"],
                              dgate_w=again["dgate_w"], dgate_b=again["dgate_b"], ds=again["ds"],
                              s_override=so, out_saved=out, lse_saved=lse)
        torch.cuda.synchronize()
        for n, t in first.items():
            if not torch.equal(t, again[n]):
                bad = (t != again[n]).reshape(t.shape[0], -1).any(dim=-1).nonzero()
                raise AssertionError(f"{w.name}: second backward call differs in {n} ({len(bad)} leading rows)")
    return {"dq": host64(dq), "dk": host64(dk), "dv": host64(dv), "dx": host64(dx), "dw_p": host64(dwp),
            "dgate_w": host64(dgw), "dgate_b": float(dgb.item()), "ds": host64(ds)}


def oracle_backward(w, inp, dout, **extra):
    return O.attn_backward(*(I.as_f64(inp[n]) for n in ("q", "k", "v", "x", "w_p", "gate_w")),
                           inp["gate_b"], I.as_f64(dout), **oracle_kwargs(w), **extra)


def assert_rel(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = np.abs(got - ref)
    fro = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    assert err.max() <= MAX_REL * scale, f"{what}: max err {err.max():.3g} vs scale {scale:.3g}"
    assert fro <= FRO_REL, f"{what}: relative Frobenius error {fro:.3g}"
    return float(err.max() / scale), fro


def _compare(w, got, ref, names=("dq", "dk", "dv", "dw_p", "dx", "dgate_w", "ds")):
    out = []
    for n in names:
        out.append((n,) + assert_rel(got[n], ref[n], f"{w.name}: {n}"))
    print(w.name, " ".join(f"{n} {m:.2g}/{f:.2g}" for n, m, f in out))


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_backward_matches_oracle(w, saved):
    inp = I.make_inputs(w)
    dout = _dout(w)
    got = run_backward(w, inp, dout, saved=saved)
    ref = oracle_backward(w, inp, dout)
    _compare(w, got, ref)
    assert abs(got["dgate_b"] - ref["dgate_b"]) <= MAX_REL * max(abs(ref["dgate_b"]), 1e-30) + 1e-7


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
def test_backward_with_dropping_and_fixed_gate(saved):
    w = CASES[3]
    inp = I.make_inputs(w)
    dout = _dout(w)
    s = np.array([O.gate(I.as_f64(inp["x"])[b], I.as_f64(inp["gate_w"]), inp["gate_b"])
                  for b in range(w.batch)])
    tau = float(s.mean())
    got = run_backward(w, inp, dout, branch_drop_tau=tau, saved=saved)
    ref = oracle_backward(w, inp, dout, drop_tau=tau)
    _compare(w, got, ref, names=("dq", "dk", "dv", "dw_p", "dgate_w"))
    lo = int(np.argmin(s))
    assert got["ds"][lo] == 0.0 and np.all(got["dx"][lo] == 0.0)
    s0 = [0.25, 0.6]
    got = run_backward(w, inp, dout, s_override=s0, saved=saved)
    ref = oracle_backward(w, inp, dout, s_override=np.array(s0))
    _compare(w, got, ref, names=("dq", "dk", "dv", "dw_p", "ds"))


def test_backward_one_token():
    """One token: softmax over one key gives P = 1 and dS = P (dP - D) = 0,
    and the linear branch's output v a / (a + eps) hardly depends on q or k,
    so the exact dQ and dK are (nearly) zero.  The device's are the rounding
    residue of that cancellation (M = H W_p is bf16, relative 2^-9 on terms of
    the gradient's size), so they are held to 4e-3 (2^-8, twice that step) of
    the gradient's natural scale, max |dV|; a dropped term or a wrong sign
    would show at that scale itself.  Every other gradient takes the usual
    relative bar."""
    w = C.small("bwd-one-token", (1, 1, 1), 2, 128, "bf16", [1, 2], 3, 64, 1)
    inp = I.make_inputs(w)
    dout = _dout(w)
    for saved in (False, True):
        got = run_backward(w, inp, dout, saved=saved)
        ref = oracle_backward(w, inp, dout)
        _compare(w, got, ref, names=("dv", "dw_p", "dx", "dgate_w", "ds"))
        scale = float(np.abs(ref["dv"]).max())
        for n in ("dq", "dk"):
            assert float(np.abs(ref[n]).max()) <= 1e-6 * scale, n
            assert float(np.abs(got[n]).max()) <= 4e-3 * scale, f"{n}: {np.abs(got[n]).max():.3g} vs {scale:.3g}"


def test_backward_is_deterministic():
    w = CASES[0]
    inp = I.make_inputs(w)
    dout = _dout(w)
    a = run_backward(w, inp, dout)
    b = run_backward(w, inp, dout)
    for n in ("dq", "dk", "dv", "dx", "dw_p", "dgate_w", "ds"):
        assert np.array_equal(a[n], b[n]), n


# ---- full workload sizes: sampled rows --------------------------------------

def _sample(w, n_q, n_kv, seed):
    """(b, n, h) rows at sequence edges and window-tile boundaries of each
    head kind, plus random rows."""
    rng = np.random.default_rng(seed)
    kinds = {}
    for h, kd in enumerate(w.head_kinds):
        kinds.setdefault(kd, []).append(h)
    edge = []
    for kd, hs in sorted(kinds.items()):
        order = O.head_order(kd, *w.grid)
        for p in (0, 127, w.N - 1):
            edge.append((int(rng.integers(w.batch)), int(order[p]), int(rng.choice(hs))))
    rand = [(int(rng.integers(w.batch)), int(rng.integers(w.N)), int(rng.integers(w.n_heads)))
            for _ in range(max(n_q, n_kv))]
    return sorted(set(edge + rand[:n_q])), sorted(set(edge[:len(kinds)] + rand[:n_kv]))


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["480p-stswa-h12", "480p-topk-h40", "480p-cfg-rope-mixed-h40"])
def test_backward_full_size_sampled_rows(name):
    """The bench workloads at full size, through salad_attn_backward as
    bench.py --backward runs it: sampled dQ rows and dK / dV rows, and the
    whole-layer dW_p, dw, db and ds, against the oracle's rows form."""
    w = C.all_workloads()[name]
    inp = I.make_inputs(w)
    dout = _dout(w)
    got = run_backward(w, inp, dout, saved=True, repeat=True)
    print(f"{name}: two backward calls bitwise equal", flush=True)
    rows_q, rows_kv = _sample(w, 10, 4, seed=11)
    args = [inp[n].float().numpy() for n in ("q", "k", "v", "x")] + \
        [I.as_f64(inp[n]) for n in ("w_p", "gate_w")]
    ref = O.attn_backward_rows(*args, inp["gate_b"], dout.float().numpy(), rows_q=rows_q, rows_kv=rows_kv,
                               **oracle_kwargs(w))
    res = []
    for n, rows in (("dq", rows_q), ("dk", rows_kv), ("dv", rows_kv)):
        g_ = np.stack([got[n][b, t, h] for (b, t, h) in rows])
        r_ = np.stack([ref[n][key] for key in rows])
        res.append((n,) + assert_rel(g_, r_, f"{name}: {n} rows"))
    for n in ("dw_p", "dgate_w", "ds"):
        res.append((n,) + assert_rel(got[n], ref[n], f"{name}: {n}"))
    assert abs(got["dgate_b"] - ref["dgate_b"]) <= MAX_REL * abs(ref["dgate_b"]) + 1e-7
    # dX is dt_b w / N on every token: check two rows
    for b in range(w.batch):
        dt = ref["ds"][b] * ref["s"][b] * (1.0 - ref["s"][b])
        exp_row = dt * I.as_f64(inp["gate_w"]) / w.N
        for t in (0, w.N - 1):
            assert_rel(got["dx"][b, t], exp_row, f"{name}: dx row")
    print(name, " ".join(f"{n} {m:.2g}/{f:.2g}" for n, m, f in res))
