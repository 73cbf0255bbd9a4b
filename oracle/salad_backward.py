"""fp64 reference for the backward pass of SALAD's hybrid attention layer.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

SALAD is obtained by fine-tuning the hybrid layer (LoRA on the attention
projections, with the zero-initialised projection and the gate trained:
[S] Method step details, steps 4-5, and the training configuration under
复现评估; [G] 2 A-B), so a training step needs the gradients of the layer
output with respect to Q, K, V, X and the layer's own parameters W_p, w, b.
The pages print no backward pass: here it is the derivative of
``salad_oracle.attn_forward`` (head-wise projection) written out by the
chain rule, one forward step at a time in reverse order.  Readings:

* the storage rounding of the rotated Q and K is treated as the identity
  (straight-through), so the gradient of the unrotated Q is the rotated
  gradient turned back by the transposed rotation;
* relu'(0) = 0 (a zero feature passes no gradient);
* the Top-K selection is piecewise constant in Q and K: its indices are
  held fixed and no gradient flows through the block means;
* a sample whose linear branch is dropped (s_b < tau) gets no gradient
  through the linear branch, W_p or the gate;
* with ``s_override`` the gate is replaced by a given s: the gradient with
  respect to s is still reported, and none reaches X, w or b.

Everything is float64.
"""

from __future__ import annotations

import numpy as np

from . import salad_oracle as F

__all__ = [
    "rope_3d_transpose", "sparse_attention_backward", "sparse_attention_head_backward",
    "linear_backward", "gate_backward", "attn_backward", "attn_backward_rows",
]


def rope_3d_transpose(g: np.ndarray, Fr: int, Hg: int, Wg: int,
                      dims=(44, 42, 42), base: float = 10000.0) -> np.ndarray:
    """Gradient through ``rope_3d``: each pair's 2x2 rotation by angle a is
    orthogonal, so the input gradient is the output gradient turned by -a.
    For a pair (x0, x1) -> (x0 c - x1 s, x0 s + x1 c) the transpose maps
    (g0, g1) -> (g0 c + g1 s, -g0 s + g1 c)."""
    g = np.asarray(g, dtype=np.float64)
    B, N, H, d = g.shape
    if sum(dims) != d:
        raise ValueError("rope dims must sum to head_dim")
    n = np.arange(N)
    pos = (n // (Hg * Wg), (n // Wg) % Hg, n % Wg)
    out = g.copy()
    off = 0
    for axis, D in enumerate(dims):
        for i in range(D // 2):
            ang = pos[axis] * base ** (-2.0 * i / D)
            c = np.cos(ang)[None, :, None]
            s = np.sin(ang)[None, :, None]
            g0 = g[..., off + 2 * i]
            g1 = g[..., off + 2 * i + 1]
            out[..., off + 2 * i] = g0 * c + g1 * s
            out[..., off + 2 * i + 1] = -g0 * s + g1 * c
        off += D
    return out


def sparse_attention_backward(qw, kw, vw, keys_of, scale: float, gw):
    """Gradients of the sparse branch of one working-order head.

    Forward per query p over its kept keys J (``salad_oracle.sparse_attention``):
    l = scale * K_J q_p, P = softmax(l), o_p = P V_J.  Given g_p = dL/do_p:
      dV_J += P g_p^T                         (o_p is linear in V_J)
      dP_j  = v_j . g_p
      dl_j  = P_j (dP_j - sum_i P_i dP_i)     (softmax Jacobian; the sum is g_p . o_p)
      dq_p  = scale * sum_j dl_j k_j,   dk_j += scale * dl_j q_p.
    Returns (dq, dk, dv), each [N, d]."""
    qw = np.asarray(qw, np.float64)
    kw = np.asarray(kw, np.float64)
    vw = np.asarray(vw, np.float64)
    gw = np.asarray(gw, np.float64)
    N = qw.shape[0]
    dq = np.zeros_like(qw)
    dk = np.zeros_like(kw)
    dv = np.zeros_like(vw)
    for p in range(N):
        J = keys_of(p)
        logits = scale * (kw[J] @ qw[p])
        e = np.exp(logits - logits.max())
        P = e / e.sum()
        dv[J] += np.outer(P, gw[p])
        dP = vw[J] @ gw[p]
        dl = P * (dP - P @ dP)
        dq[p] = scale * (dl @ kw[J])
        dk[J] += scale * np.outer(dl, qw[p])
    return dq, dk, dv


def sparse_attention_head_backward(kind: int, qw, kw, vw, gw, *, r: int, bs: int, scale: float,
                                   idx=None):
    """``sparse_attention_backward`` with the key sets of a window head
    ({j : |p - j| <= r}) or of a Top-K head (the rows of the selected key
    blocks ``idx`` [nb, k], held fixed)."""
    N = qw.shape[0]
    if kind == F.HEAD_TOPK:
        return sparse_attention_backward(qw, kw, vw, lambda p: F.topk_keys(p, idx, bs, N), scale, gw)
    return sparse_attention_backward(qw, kw, vw, lambda p: F.swa_keys(p, N, r), scale, gw)


def linear_backward(q, k, v, g, eps: float = 1e-6):
    """Gradients of O_l = relu(Q) H / (relu(Q) Z + eps) with H = relu(K)^T V,
    Z = relu(K)^T 1 ([S] Prerequisites > Linear Attention), given
    g = dL/dO_l [N, d_v].  With a = relu(q_n), num_n = a H, den_n = a . Z + eps:
      dnum_n = g_n / den_n,    dden_n = -(g_n . num_n) / den_n^2
      da_n   = dnum_n H^T + dden_n Z,        dq_n = da_n * [q_n > 0]
      dH     = sum_n a_n^T dnum_n,           dZ = sum_n dden_n a_n
      dk_n   = (dH v_n + dZ) * [k_n > 0]     (H and Z are sums over the keys)
      dv_n   = relu(k_n) dH.
    Returns (dq, dk, dv)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    H, Z = F.linear_state(k, v)
    a = np.maximum(q, 0.0)
    num = a @ H
    den = a @ Z + eps
    dnum = g / den[:, None]
    dden = -np.sum(g * num, axis=1) / den ** 2
    da = dnum @ H.T + dden[:, None] * Z[None, :]
    dq = da * (q > 0)
    dH = a.T @ dnum
    dZ = a.T @ dden
    dk = (v @ dH.T + dZ[None, :]) * (k > 0)
    dv = np.maximum(k, 0.0) @ dH
    return dq, dk, dv


def gate_backward(x: np.ndarray, w: np.ndarray, b: float, ds: float):
    """Gradients of s = sigmoid(w . mean_n X[n] + b) (``salad_oracle.gate``)
    for one sample, given ds = dL/ds: with t the logit, dt = ds s (1 - s);
    dw = dt mean_n X[n]; db = dt; dX[n] = dt w / N for every token.
    Returns (dx [N, C], dw [C], db)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    N = x.shape[0]
    s = F.gate(x, w, b)
    dt = ds * s * (1.0 - s)
    return np.broadcast_to(dt * w / N, x.shape).copy(), dt * x.mean(axis=0), dt


def attn_backward(q, k, v, x, w_p, gate_w, gate_b, dout, *, grid, head_kinds, window_radius,
                  block, topk, io_dtype="bf16", rope=False, rope_dims=(44, 42, 42),
                  rope_base=10000.0, softmax_scale=None, linear_eps=1e-6, s_override=None,
                  drop_tau=0.0):
    """Gradients of ``salad_oracle.attn_forward`` (head-wise W_p [d, d]) for
    the output gradient ``dout`` [B, N, H, d].

    Forward, per sample b and head h: (Q, K rotated and rounded when RoPE is
    on) -> working order -> O_s (sparse) and O_l (linear) -> token order ->
    out = O_s + s_b (O_l W_p), s_b = gate(X_b).  Reverse:
      dO_s = G;  dO_l = s_b G W_p^T;  dW_p += s_b O_l^T G;  ds_b += sum G . (O_l W_p)
    (the last three only for kept samples), then each branch's backward on
    its inputs, the working-order gradients scattered back to token order,
    the two branches' dQ, dK, dV added, the RoPE transpose applied to dQ and
    dK, and the gate's backward per sample.

    Returns a dict: dq, dk, dv [B, N, H, d]; dx [B, N, C] (zero with
    s_override); dw_p [d, d]; dgate_w [C]; dgate_b; ds [B] (dL/ds_b, zero for
    dropped samples); s [B].
    """
    Fr, Hg, Wg = grid
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    x = np.asarray(x, np.float64)
    w_p = np.asarray(w_p, np.float64)
    gate_w = np.asarray(gate_w, np.float64)
    G = np.asarray(dout, np.float64)
    B, N, H, d = q.shape
    if N != Fr * Hg * Wg:
        raise ValueError("N must equal F*Hg*Wg")
    scale = 1.0 / np.sqrt(d) if not softmax_scale or softmax_scale <= 0 else softmax_scale

    s = np.empty(B)
    for b in range(B):
        s[b] = F.gate(x[b], gate_w, gate_b) if s_override is None else float(s_override[b])

    if rope:
        qu = F.round_to_io(F.rope_3d(q, Fr, Hg, Wg, rope_dims, rope_base), io_dtype)
        ku = F.round_to_io(F.rope_3d(k, Fr, Hg, Wg, rope_dims, rope_base), io_dtype)
    else:
        qu, ku = q, k

    dq_u = np.zeros_like(q)       # gradients w.r.t. the rotated Q, K
    dk_u = np.zeros_like(k)
    dv = np.zeros_like(v)
    dw_p = np.zeros_like(w_p)
    ds = np.zeros(B)
    for b in range(B):
        kept = F.branch_kept(s[b], drop_tau)
        for h in range(H):
            kind = int(head_kinds[h])
            order = F.head_order(kind, Fr, Hg, Wg)
            qh, kh, vh, gh = qu[b, :, h], ku[b, :, h], v[b, :, h], G[b, :, h]
            # sparse branch, in working order
            qw, kw, vw, gw = qh[order], kh[order], vh[order], gh[order]
            idx = None
            if kind == F.HEAD_TOPK:
                idx = F.topk_blocks(F.block_means(qw, block), F.block_means(kw, block), topk)
            dqw, dkw, dvw = sparse_attention_head_backward(kind, qw, kw, vw, gw, r=window_radius,
                                                           bs=block, scale=scale, idx=idx)
            dq_u[b, order, h] += dqw
            dk_u[b, order, h] += dkw
            dv[b, order, h] += dvw
            if not kept:
                continue
            # linear branch and the combine (token order; the branch ignores order)
            Hm, Zv = F.linear_state(kh, vh)
            o_l = F.linear_apply(qh, Hm, Zv, linear_eps)
            dw_p += s[b] * (o_l.T @ gh)
            ds[b] += float(np.sum(gh * (o_l @ w_p)))
            dql, dkl, dvl = linear_backward(qh, kh, vh, s[b] * (gh @ w_p.T), linear_eps)
            dq_u[b, :, h] += dql
            dk_u[b, :, h] += dkl
            dv[b, :, h] += dvl

    if rope:
        dq = rope_3d_transpose(dq_u, Fr, Hg, Wg, rope_dims, rope_base)
        dk = rope_3d_transpose(dk_u, Fr, Hg, Wg, rope_dims, rope_base)
    else:
        dq, dk = dq_u, dk_u

    dx = np.zeros_like(x)
    dgate_w = np.zeros_like(gate_w)
    dgate_b = 0.0
    if s_override is None:
        for b in range(B):
            dxb, dwb, dbb = gate_backward(x[b], gate_w, gate_b, ds[b])
            dx[b] = dxb
            dgate_w += dwb
            dgate_b += dbb
    return {"dq": dq, "dk": dk, "dv": dv, "dx": dx, "dw_p": dw_p, "dgate_w": dgate_w,
            "dgate_b": dgate_b, "ds": ds, "s": s}


def attn_backward_rows(q, k, v, x, w_p, gate_w, gate_b, dout, *, rows_q=(), rows_kv=(), grid,
                       head_kinds, window_radius, block, topk, io_dtype="bf16", rope=False,
                       rope_dims=(44, 42, 42), rope_base=10000.0, softmax_scale=None,
                       linear_eps=1e-6, s_override=None, drop_tau=0.0):
    """Selected rows of ``attn_backward`` for layers too large to
    differentiate whole: dQ at the (b, n, h) triples of ``rows_q``, dK and
    dV at those of ``rows_kv``, and the whole-layer dW_p, dgate_w, dgate_b
    and ds (their sums over tokens cost one pass over each head).

    The same formulas as ``attn_backward``, evaluated where needed: a dQ row
    needs only its query's kept keys; a dK / dV row of key j needs every
    query i whose kept set holds j (the window is symmetric, so for window
    heads those are the queries within r of j; for Top-K heads the rows of
    the query blocks that selected j's block), each with its full softmax
    row and D_i.  The linear branch's per-row terms use the head's sums
    A = sum_n (a_n / den_n)^T g_n and Bz = sum_n dden_n a_n (see
    ``linear_backward``, written here through M = H W_p).  Inputs may be
    float32 arrays holding the storage values; each head is widened to
    float64 when first used.  Returns a dict with "dq", "dk", "dv" (dicts
    keyed by triple), "dw_p", "dgate_w", "dgate_b", "ds" and "s"."""
    Fr, Hg, Wg = grid
    B, N, H, d = np.shape(q)
    scale = 1.0 / np.sqrt(d) if not softmax_scale or softmax_scale <= 0 else softmax_scale
    w_p = np.asarray(w_p, np.float64)
    gate_w = np.asarray(gate_w, np.float64)
    s = np.empty(B)
    for b in range(B):
        s[b] = F.gate(np.asarray(x[b], np.float64), gate_w, gate_b) if s_override is None \
            else float(s_override[b])
    kept = [F.branch_kept(s[b], drop_tau) for b in range(B)]
    cache = {}

    def head(b, h):
        """Token-order q, k (rotated and rounded as the forward), v, g, the
        working order, the selection and the linear branch's head sums."""
        key = (b, h)
        if key in cache:
            return cache[key]
        qh = np.asarray(q[b:b + 1, :, h:h + 1], np.float64)
        kh = np.asarray(k[b:b + 1, :, h:h + 1], np.float64)
        if rope:
            qh = F.round_to_io(F.rope_3d(qh, Fr, Hg, Wg, rope_dims, rope_base), io_dtype)
            kh = F.round_to_io(F.rope_3d(kh, Fr, Hg, Wg, rope_dims, rope_base), io_dtype)
        qh, kh = qh[0, :, 0], kh[0, :, 0]
        vh = np.asarray(v[b, :, h], np.float64)
        gh = np.asarray(dout[b, :, h], np.float64)
        kind = int(head_kinds[h])
        order = F.head_order(kind, Fr, Hg, Wg)
        c = dict(q=qh, k=kh, v=vh, g=gh, kind=kind, order=order, pos=np.argsort(order),
                 qw=qh[order], kw=kh[order], vw=vh[order], gw=gh[order], idx=None)
        if kind == F.HEAD_TOPK:
            c["idx"] = F.topk_blocks(F.block_means(c["qw"], block), F.block_means(c["kw"], block), topk)
        Hm, Zv = F.linear_state(kh, vh)
        M = Hm @ w_p
        a = np.maximum(qh, 0.0)
        den = a @ Zv + linear_eps
        gm = gh @ M.T
        dden = -s[b] * np.sum(a * gm, axis=1) / den ** 2
        A = (a / den[:, None]).T @ gh
        c.update(H=Hm, Z=Zv, M=M, den=den, gm=gm, dden=dden, A=A, Bz=a.T @ dden,
                 dH=s[b] * (A @ w_p.T))
        cache[key] = c
        return c

    def keys_of(c, p):
        if c["kind"] == F.HEAD_TOPK:
            return F.topk_keys(p, c["idx"], block, N)
        return F.swa_keys(p, N, window_radius)

    def queries_of(c, j):
        if c["kind"] == F.HEAD_TOPK:
            kb = j // block
            qbs = [qb for qb in range(c["idx"].shape[0]) if kb in set(int(t) for t in c["idx"][qb])]
            if not qbs:
                return np.zeros(0, dtype=np.int64)
            return np.concatenate([np.arange(qb * block, min(N, (qb + 1) * block)) for qb in qbs])
        return F.swa_keys(j, N, window_radius)   # |i - j| <= r is symmetric

    def softmax_row(c, p):
        J = keys_of(c, p)
        lg = scale * (c["kw"][J] @ c["qw"][p])
        e = np.exp(lg - lg.max())
        P = e / e.sum()
        dP = c["vw"][J] @ c["gw"][p]
        return J, P, dP, P @ dP

    def rotate_back(row, n):
        if not rope:
            return row
        g = np.zeros((1, N, 1, d))
        g[0, n, 0] = row
        return rope_3d_transpose(g, Fr, Hg, Wg, rope_dims, rope_base)[0, n, 0]

    out = {"dq": {}, "dk": {}, "dv": {}}
    for (b, n, h) in rows_q:
        c = head(b, h)
        p = int(c["pos"][n])
        J, P, dP, D = softmax_row(c, p)
        row = scale * ((P * (dP - D)) @ c["kw"][J])
        if kept[b]:
            row = row + ((s[b] / c["den"][n]) * c["gm"][n] + c["dden"][n] * c["Z"]) * (c["q"][n] > 0)
        out["dq"][(b, n, h)] = rotate_back(row, n)
    for (b, n, h) in rows_kv:
        c = head(b, h)
        j = int(c["pos"][n])
        dk = np.zeros(d)
        dv = np.zeros(v.shape[3])
        for i in queries_of(c, j):
            J, P, dP, D = softmax_row(c, int(i))
            t = np.searchsorted(J, j)
            if t >= len(J) or J[t] != j:
                continue
            dv += P[t] * c["gw"][i]
            dk += scale * P[t] * (dP[t] - D) * c["qw"][i]
        if kept[b]:
            dk = dk + (c["dH"] @ c["v"][n] + c["Bz"]) * (c["k"][n] > 0)
            dv = dv + c["dH"].T @ np.maximum(c["k"][n], 0.0)
        out["dk"][(b, n, h)] = rotate_back(dk, n)
        out["dv"][(b, n, h)] = dv

    dw_p = np.zeros_like(w_p)
    ds = np.zeros(B)
    for b in range(B):
        if not kept[b]:
            continue
        for h in range(H):
            c = head(b, h)
            dw_p += s[b] * (c["H"].T @ c["A"])
            ds[b] += float(np.sum(c["M"] * c["A"]))
            del cache[(b, h)]
    dgate_w = np.zeros_like(gate_w)
    dgate_b = 0.0
    if s_override is None:
        for b in range(B):
            dt = ds[b] * s[b] * (1.0 - s[b])
            dgate_w += dt * np.asarray(x[b], np.float64).mean(axis=0)
            dgate_b += dt
    out.update(dw_p=dw_p, dgate_w=dgate_w, dgate_b=dgate_b, ds=ds, s=s)
    return out
