"""salad_linear_state_noalloc: the linear-attention state ([S]
Prerequisites > Linear Attention) with the library's fixed device scratch
instead of a caller workspace, for callers that cannot allocate.  Its output
must equal salad_linear_state's (same kernels, same split order: bit for
bit) on consecutive calls, the second with a smaller problem, so that the
scratch left by the first call cannot leak into the second."""

import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import sparse_linear_hybrid_st_amd as S
from sparse_linear_hybrid_st_amd import configs as C
from sparse_linear_hybrid_st_amd import inputs as I
from tests.gpu_util import host64, rel_fro


def _state(w, use_noalloc):
    p = S.problem_from_workload(w)
    inp = I.make_inputs(w)
    kw, vw = torch.empty_like(inp["k"].cuda()), torch.empty_like(inp["v"].cuda())
    S.salad_permute(p, 0, 0, inp["k"].cuda(), kw)
    S.salad_permute(p, 0, 0, inp["v"].cuda(), vw)
    bh = w.batch * w.n_heads
    h = torch.full((w.batch, w.n_heads, w.head_dim, w.head_dim), float("nan"), device="cuda")
    z = torch.full((w.batch, w.n_heads, w.head_dim), float("nan"), device="cuda")
    if use_noalloc:
        S.salad_linear_state_noalloc(p, kw, vw, h, z)
    else:
        S.salad_linear_state(p, kw, vw, h, z, S.workspace(p))
    torch.cuda.synchronize()
    assert h.numel() == bh * w.head_dim ** 2
    return inp, h.cpu(), z.cpu()


CASES = [
    # large first, then smaller: a stale partial from the first call would show
    [C.small("na-bf16-big", (8, 20, 30), 12, 128, "bf16", [0, 1] * 6, 64, 64, 1, batch=2),
     C.small("na-bf16-small", (3, 5, 7), 3, 128, "bf16", [1, 0, 2], 9, 64, 1)],
    [C.small("na-f32-big", (4, 9, 16), 5, 64, "f32", [0, 1, 0, 1, 2], 20, 16, 2, batch=2),
     C.small("na-f32-small", (2, 3, 5), 2, 64, "f32", [1, 0], 5, 16, 1)],
]


@pytest.mark.gpu
@pytest.mark.parametrize("pair", CASES, ids=["bf16", "f32"])
def test_noalloc_matches_workspace_entry_point(pair):
    for w in pair:                      # two calls in a row, the second smaller
        inp, h0, z0 = _state(w, False)
        _, h1, z1 = _state(w, True)
        assert torch.equal(h0, h1) and torch.equal(z0, z1), f"{w.name}: noalloc differs from workspace call"
        # and both against the oracle ([S] Prerequisites > Linear Attention)
        k, v = I.as_f64(inp["k"]), I.as_f64(inp["v"])
        for b in range(w.batch):
            for hh in range(w.n_heads):
                Hr, Zr = O.linear_state(k[b, :, hh], v[b, :, hh])
                assert rel_fro(host64(h1)[b, hh], Hr) <= 1e-5 and rel_fro(host64(z1)[b, hh], Zr) <= 1e-5


@pytest.mark.gpu
def test_noalloc_repeat_after_larger_call_is_bitwise_stable():
    big, small = CASES[0]
    _, h_a, z_a = _state(small, True)
    _state(big, True)
    _, h_b, z_b = _state(small, True)
    assert torch.equal(h_a, h_b) and torch.equal(z_a, z_b)


def test_noalloc_rejects_problems_beyond_its_scratch():
    """Validation runs before the scratch is touched: B*H = 1024 heads of
    d = 128 need 1024 * 66,048 bytes of partial states, past the 36 MiB."""
    L = S.lib()
    w = C.small("na-too-big", (1, 4, 32), 256, 128, "bf16", [0] * 256, 4, 64, 1, batch=4)
    p = S.problem_from_workload(w)
    a = ctypes.c_void_p(0x10000)
    assert L.salad_linear_state_noalloc(ctypes.byref(p), a, a, a, a, None) == 5
    assert b"36" in L.salad_last_error() or b"scratch" in L.salad_last_error()
    assert L.salad_linear_state_noalloc(None, a, a, a, a, None) == 1
