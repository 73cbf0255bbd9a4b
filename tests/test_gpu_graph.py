"""The fused layer captured in a HIP graph (torch.cuda.CUDAGraph on ROCm).

salad_attn_forward only launches kernels on the caller's stream (no
allocation, memset or host synchronisation), so a serving loop can capture
it once and replay it.  Each replay is compared bit for bit with the eager
call on the same inputs (the layer is deterministic), with the program's
own eager work and synchronisations between the replays; the eager output
is checked against the oracle first.
"""

import numpy as np
import pytest
import torch

import oracle as O
import sparse_linear_hybrid_st_amd as S
from sparse_linear_hybrid_st_amd import configs as C
from sparse_linear_hybrid_st_amd import inputs as I
from tests.gpu_util import assert_close, dev, host64, oracle_kwargs

pytestmark = pytest.mark.gpu

CASES = [
    (C.small("graph-rope-cfg", (3, 4, 10), 4, 128, "bf16", [0, 1, 2, 2], 20, 64, 1, batch=2,
             rope=True, rope_dims=(44, 42, 42), x_sample_shift=True), "head"),
    (C.small("graph-window-multi-tile", (6, 16, 24), 2, 128, "bf16", [1, 0], 300, 64, 1, seed=9), "head"),
    (C.small("graph-full-width", (5, 6, 7), 4, 128, "bf16", [0, 1, 2, 2], 37, 64, 2), "full"),
]


@pytest.mark.parametrize("w,proj", CASES, ids=[c[0].name for c in CASES])
def test_forward_replays_in_graph(w, proj):
    print(f"[graph] {w.name}: N={w.N} H={w.n_heads} B={w.batch} proj={proj}", flush=True)
    inp = I.make_inputs(w, proj=proj)
    p = S.problem_from_workload(w, proj=proj)
    d = {n: dev(inp[n]) for n in ("q", "k", "v", "x", "w_p", "gate_w")}
    ws = S.workspace(p)

    def layer(out):
        S.salad_attn_forward(p, d["q"], d["k"], d["v"], d["x"], d["w_p"], d["gate_w"], inp["gate_b"], out, ws)

    eager = torch.empty_like(d["q"])
    layer(eager)
    torch.cuda.synchronize()
    ref = O.attn_forward(*(I.as_f64(inp[n]) for n in ("q", "k", "v", "x", "w_p", "gate_w")), inp["gate_b"],
                         proj=proj, **oracle_kwargs(w))["out"]
    assert_close(host64(eager), ref, w.io_dtype, f"{w.name}: eager")

    out = torch.empty_like(d["q"])
    side = torch.cuda.Stream()  # warm-up off the default stream before capture
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer(out)
    torch.cuda.synchronize()
    for i in range(3):
        out.zero_()
        other = (d["x"].float() * (i + 1)).sum()  # unrelated eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(other)
        assert torch.equal(out, eager), f"{w.name}: replay {i} differs from the eager call"


def test_forward_and_backward_replay_in_one_graph():
    """A training step's layer calls, forward (saving out and the row
    normalisers) then backward, captured together; replays bitwise equal
    to the eager calls."""
    w = CASES[0][0]
    print(f"[graph] forward + backward {w.name}", flush=True)
    inp = I.make_inputs(w)
    p = S.problem_from_workload(w)
    d = {n: dev(inp[n]) for n in ("q", "k", "v", "x", "w_p", "gate_w")}
    g = np.random.default_rng(w.seed + 77).standard_normal((w.batch, w.N, w.n_heads, w.head_dim))
    go = dev(I.to_storage(g.astype(np.float32), w.io_dtype))
    ws, bws = S.workspace(p), S.backward_workspace(p)

    def bufs():
        return {"out": torch.empty_like(d["q"]),
                "lse": torch.empty((w.batch, w.n_heads, w.N), dtype=torch.float32, device="cuda"),
                "dq": torch.empty_like(d["q"]), "dk": torch.empty_like(d["q"]), "dv": torch.empty_like(d["q"]),
                "dx": torch.empty_like(d["x"]),
                "dwp": torch.empty((w.head_dim, w.head_dim), dtype=torch.float32, device="cuda"),
                "dgw": torch.empty(w.n_heads * w.head_dim, dtype=torch.float32, device="cuda"),
                "dgb": torch.empty(1, dtype=torch.float32, device="cuda"),
                "ds": torch.empty(w.batch, dtype=torch.float32, device="cuda")}

    def step(b):
        S.salad_attn_forward(p, d["q"], d["k"], d["v"], d["x"], d["w_p"], d["gate_w"], inp["gate_b"], b["out"], ws,
                             lse_out=b["lse"])
        S.salad_attn_backward(p, d["q"], d["k"], d["v"], d["x"], d["w_p"], d["gate_w"], inp["gate_b"], go,
                              b["dq"], b["dk"], b["dv"], b["dwp"], bws, dx=b["dx"], dgate_w=b["dgw"],
                              dgate_b=b["dgb"], ds=b["ds"], out_saved=b["out"], lse_saved=b["lse"])

    eager = bufs()
    step(eager)
    torch.cuda.synchronize()
    got = bufs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(got)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(got)
    torch.cuda.synchronize()
    for i in range(3):
        for t in got.values():
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in eager:
            assert torch.equal(got[n], eager[n]), f"replay {i}: {n} differs from the eager call"
