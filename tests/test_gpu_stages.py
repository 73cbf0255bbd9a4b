"""Per-stage parity of the HIP path against the oracle on small shapes that
span several tiles and a ragged tail.  Each stage gets the oracle's own
inputs for that stage, so a failure points at one kernel."""

import numpy as np
import pytest
import torch

import oracle as O
import sparse_linear_hybrid_st_amd as S
from sparse_linear_hybrid_st_amd import configs as C
from sparse_linear_hybrid_st_amd import inputs as I
from tests.gpu_util import assert_close, check_selection, dev, host64, rel_fro

pytestmark = pytest.mark.gpu

CASES = {
    # f32: d = 64 and 128, all head kinds, ragged blocks
    "f32-d64": C.small("f32-d64", (3, 5, 7), 3, 64, "f32", [0, 1, 2], 9, 16, 3, qk_channel_scale=False),
    "f32-d128": C.small("f32-d128", (2, 4, 9), 2, 128, "f32", [1, 2], 5, 8, 4, batch=2),
    # bf16: 210 tokens = one full 128-query tile + 82; 4 blocks of 64 with an 18-row tail
    "bf16-small": C.small("bf16-small", (5, 6, 7), 4, 128, "bf16", [0, 1, 2, 2], 37, 64, 2),
    # bf16 window spanning many key tiles (r = 300 > 4 tiles)
    "bf16-mid": C.small("bf16-mid", (6, 16, 24), 2, 128, "bf16", [0, 1], 300, 64, 1),
    # bf16 Top-K over 15 blocks, batch 2
    "bf16-topk": C.small("bf16-topk", (4, 12, 20), 2, 128, "bf16", [2, 2], 0, 64, 4, batch=2),
    # bf16 with 3D RoPE, mixed heads, batch 2
    "bf16-rope": C.small("bf16-rope", (3, 4, 10), 4, 128, "bf16", [0, 1, 2, 2], 20, 64, 1,
                         batch=2, rope=True, rope_dims=(44, 42, 42)),
}


def _inputs(name):
    w = CASES[name]
    return w, I.make_inputs(w), S.problem_from_workload(w)


def _orders(w):
    return [O.head_order(k, *w.grid) for k in w.head_kinds]


def _working_ref(w, inp):
    """Oracle working-order Q, K, V (after RoPE if enabled), float64."""
    q, k, v = (I.as_f64(inp[n]) for n in ("q", "k", "v"))
    if w.rope:
        q = O.round_to_io(O.rope_3d(q, *w.grid, w.rope_dims, w.rope_base), w.io_dtype)
        k = O.round_to_io(O.rope_3d(k, *w.grid, w.rope_dims, w.rope_base), w.io_dtype)
    o = _orders(w)
    return O.to_working(q, o), O.to_working(k, o), O.to_working(v, o)


def _to_dev_storage(a, w):
    return dev(I.to_storage(a.astype(np.float32), w.io_dtype))


@pytest.mark.parametrize("name", list(CASES))
def test_permute_forward_inverse_and_rope(name):
    w, inp, p = _inputs(name)
    qw_ref, kw_ref, vw_ref = _working_ref(w, inp)
    for t, ref, rope in (("q", qw_ref, w.rope), ("k", kw_ref, w.rope), ("v", vw_ref, False)):
        src = dev(inp[t])
        dst = torch.empty_like(src)
        S.salad_permute(p, int(rope), 0, src, dst)
        torch.cuda.synchronize()
        got = host64(dst).reshape(ref.shape)
        np.testing.assert_array_equal(got, ref, err_msg=f"{name}: permute {t}")
        if not rope:
            back = torch.empty_like(src)
            S.salad_permute(p, 0, 1, dst, back)
            torch.cuda.synchronize()
            assert torch.equal(back.cpu(), inp[t]), f"{name}: inverse permute {t}"


@pytest.mark.parametrize("name", [n for n, w in CASES.items() if 2 in w.head_kinds])
def test_block_select(name):
    w, inp, p = _inputs(name)
    qw, kw, _ = _working_ref(w, inp)
    nb = p.n_blocks
    idx = torch.full((w.batch, w.n_heads, nb, w.topk), -1, dtype=torch.int32, device="cuda")
    qbar = torch.zeros((w.batch, w.n_heads, nb, w.head_dim), dtype=torch.float64, device="cuda")
    kbar = torch.zeros_like(qbar)
    S.salad_block_select(p, _to_dev_storage(qw, w), _to_dev_storage(kw, w), idx, S.workspace(p),
                         qbar, kbar)
    torch.cuda.synchronize()
    idx, qbar, kbar = idx.cpu().numpy(), qbar.cpu().numpy(), kbar.cpu().numpy()
    for b in range(w.batch):
        for h, kind in enumerate(w.head_kinds):
            if kind != 2:
                assert np.all(idx[b, h] == -1), "non-Top-K rows must stay untouched"
                continue
            qm, km = O.block_means(qw[b, h], w.block), O.block_means(kw[b, h], w.block)
            np.testing.assert_allclose(qbar[b, h], qm, rtol=1e-15, atol=0)
            np.testing.assert_allclose(kbar[b, h], km, rtol=1e-15, atol=0)
            check_selection(idx[b, h], qm, km, w.topk, f"{name} b{b} h{h}")


@pytest.mark.parametrize("name", list(CASES))
def test_sparse_attention(name):
    w, inp, p = _inputs(name)
    qw, kw, vw = _working_ref(w, inp)
    nb = p.n_blocks
    idx_all = np.zeros((w.batch, w.n_heads, nb, w.topk), np.int32)
    ref = np.zeros_like(qw)
    scale = 1.0 / np.sqrt(w.head_dim)
    for b in range(w.batch):
        for h, kind in enumerate(w.head_kinds):
            o, idx = O.sparse_attention_head(kind, qw[b, h], kw[b, h], vw[b, h], r=w.window_radius,
                                             bs=w.block, k=w.topk, scale=scale)
            ref[b, h] = o
            if idx is not None:
                idx_all[b, h] = idx
    o_s = torch.empty(qw.shape, dtype=torch.float32, device="cuda")
    S.salad_sparse_attn(p, _to_dev_storage(qw, w), _to_dev_storage(kw, w), _to_dev_storage(vw, w),
                        dev(torch.from_numpy(idx_all)) if 2 in w.head_kinds else None, o_s)
    torch.cuda.synchronize()
    mx, mn = assert_close(host64(o_s), ref, w.io_dtype, f"{name}: O_s")
    print(f"{name}: O_s max {mx:.3g} mean {mn:.3g}")


@pytest.mark.parametrize("name", list(CASES))
def test_linear_state_and_apply(name):
    w, inp, p = _inputs(name)
    qw, kw, vw = _working_ref(w, inp)
    BH, D = w.batch * w.n_heads, w.head_dim
    Href = np.zeros((w.batch, w.n_heads, D, D))
    Zref = np.zeros((w.batch, w.n_heads, D))
    Oref = np.zeros_like(qw)
    for b in range(w.batch):
        for h in range(w.n_heads):
            Href[b, h], Zref[b, h] = O.linear_state(kw[b, h], vw[b, h])
            Oref[b, h] = O.linear_apply(qw[b, h], Href[b, h], Zref[b, h], 1e-6)
    hs = torch.empty((w.batch, w.n_heads, D, D), dtype=torch.float32, device="cuda")
    zs = torch.empty((w.batch, w.n_heads, D), dtype=torch.float32, device="cuda")
    ws = S.workspace(p)
    S.salad_linear_state(p, _to_dev_storage(kw, w), _to_dev_storage(vw, w), hs, zs, ws)
    torch.cuda.synchronize()
    assert rel_fro(host64(hs), Href) <= 1e-5, f"{name}: H rel err {rel_fro(host64(hs), Href):.3g}"
    assert rel_fro(host64(zs), Zref) <= 1e-5, f"{name}: Z"
    # apply from the oracle's state (rounded to float32)
    o_l = torch.empty(qw.shape, dtype=torch.float32, device="cuda")
    S.salad_linear_apply(p, _to_dev_storage(qw, w), dev(torch.from_numpy(Href.astype(np.float32))),
                         dev(torch.from_numpy(Zref.astype(np.float32))), o_l)
    torch.cuda.synchronize()
    e = rel_fro(host64(o_l), Oref)
    assert e <= 1e-4, f"{name}: O_l rel err {e:.3g}"
    assert_close(host64(o_l), Oref, "f32", f"{name}: O_l")


@pytest.mark.parametrize("name", list(CASES))
def test_gate_and_combine(name):
    w, inp, p = _inputs(name)
    x = I.as_f64(inp["x"])
    gw = I.as_f64(inp["gate_w"])
    s = torch.empty(w.batch, dtype=torch.float32, device="cuda")
    ws = S.workspace(p)
    S.salad_gate(p, dev(inp["x"]), dev(inp["gate_w"]), 0.25, s, ws)
    torch.cuda.synchronize()
    for b in range(w.batch):
        assert abs(float(s[b]) - O.gate(x[b], gw, 0.25)) <= 1e-6
    # combine from oracle-made stage values
    rng = np.random.default_rng(3)
    shape = (w.batch, w.n_heads, w.N, w.head_dim)
    o_s = rng.standard_normal(shape).astype(np.float32) * 0.1
    o_l = rng.standard_normal(shape).astype(np.float32) * 0.01
    wp = I.as_f64(inp["w_p"]) * 10
    sv = np.array([0.3, 0.7][:w.batch], np.float32)
    out = torch.empty((w.batch, w.N, w.n_heads, w.head_dim), dtype=inp["q"].dtype, device="cuda")
    S.salad_combine(p, dev(torch.from_numpy(o_s)), dev(torch.from_numpy(o_l)),
                    _to_dev_storage(wp, w), dev(torch.from_numpy(sv)), out)
    torch.cuda.synchronize()
    got = host64(out)
    orders = _orders(w)
    for b in range(w.batch):
        for h in range(w.n_heads):
            ref = O.combine(o_s[b, h], o_l[b, h], O.round_to_io(wp, w.io_dtype), float(sv[b]))
            assert_close(got[b, orders[h], h], ref, w.io_dtype, f"{name}: combine b{b} h{h}",
                         max_abs=1e-5 if w.io_dtype == "f32" else 4e-3)
