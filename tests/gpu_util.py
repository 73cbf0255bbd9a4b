"""Helpers shared by the GPU parity tests (not a test module).

Inputs come from the seeded generator; expected values only from the
oracle.  Tolerances: f32 workloads max |err| <= 1e-4; bf16 workloads max
|err| <= 2e-2 and mean |err| <= 2e-3 on layer outputs; block indices and
permutations bit-exact, except query blocks whose k-th and (k+1)-th oracle
scores are within 1e-6 relative (near-ties), which are reported.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle as O
import sparse_linear_hybrid_st_amd as S
from sparse_linear_hybrid_st_amd import inputs as I

TOL = {"f32": dict(max_abs=1e-4, mean_abs=None), "bf16": dict(max_abs=2e-2, mean_abs=2e-3)}
NEAR_TIE = 1e-6


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().cuda()


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def assert_close(got, ref, io_dtype, what="", max_abs=None, mean_abs=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    tol = TOL[io_dtype]
    mx = tol["max_abs"] if max_abs is None else max_abs
    mn = tol["mean_abs"] if mean_abs is None else mean_abs
    assert err.max() <= mx, f"{what}: max abs err {err.max():.3g} > {mx}"
    if mn is not None:
        assert err.mean() <= mn, f"{what}: mean abs err {err.mean():.3g} > {mn}"
    return float(err.max()), float(err.mean())


def rel_fro(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def oracle_kwargs(w):
    return dict(grid=w.grid, head_kinds=w.head_kinds, window_radius=w.window_radius,
                block=w.block, topk=w.topk, io_dtype=w.io_dtype, rope=w.rope,
                rope_dims=w.rope_dims, rope_base=w.rope_base)


def check_selection(gpu_idx, qbar, kbar, k, what=""):
    """Compare one head's selection with the oracle's; near-tie rows may
    differ but must still be a valid top-k.  Returns the differing rows."""
    ref = O.topk_blocks(qbar, kbar, k)
    gap = O.topk_gap(qbar, kbar, k)
    S_ = O.block_scores(qbar, kbar)
    differ = np.where(np.any(np.asarray(gpu_idx) != ref, axis=1))[0]
    for r in differ:
        assert gap[r] <= NEAR_TIE, f"{what}: block row {r} differs with gap {gap[r]:.3g}"
        sel = np.asarray(gpu_idx[r])
        assert len(set(sel.tolist())) == k and np.all(np.diff(sel) > 0)
        rest = np.setdiff1d(np.arange(S_.shape[1]), sel)
        if len(rest):
            lo, hi = S_[r, sel].min(), S_[r, rest].max()
            assert lo >= hi - NEAR_TIE * max(abs(lo), abs(hi)), f"{what}: row {r} not a top-k"
    if len(differ):
        print(f"[near-tie] {what}: {len(differ)} block rows resolved differently (gap <= {NEAR_TIE})")
    return differ


def run_forward(w, inp, s_override=None, stream=None, branch_drop_tau=0.0, proj="head"):
    """salad_attn_forward on the device; returns (out, s, idx) on the host."""
    p = S.problem_from_workload(w, branch_drop_tau=branch_drop_tau, proj=proj)
    q, k, v, x = (dev(inp[n]) for n in ("q", "k", "v", "x"))
    wp, gw = dev(inp["w_p"]), dev(inp["gate_w"])
    out = torch.empty_like(q)
    s = torch.empty(w.batch, dtype=torch.float32, device="cuda")
    idx = torch.full((w.batch, w.n_heads, p.n_blocks, w.topk), -1, dtype=torch.int32, device="cuda")
    ws = S.workspace(p)
    so = None if s_override is None else torch.tensor(s_override, dtype=torch.float32, device="cuda")
    S.salad_attn_forward(p, q, k, v, x, wp, gw, inp["gate_b"], out, ws, s_override=so, s_out=s,
                         idx_out=idx, stream=stream)
    torch.cuda.synchronize()
    return out.cpu(), s.cpu().numpy(), idx.cpu().numpy()
