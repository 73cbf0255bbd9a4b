"""fp64 reference implementation of SALAD's hybrid attention forward.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources (web pages about arXiv 2601.16515; cited by tag and section):

[S]  "SALAD: Achieve High-Sparsity Attention via Efficient Linear Attention
     Tuning for Video Diffusion Transformer", structured summary at
     paper.rainbus.top/paper/2601.16515.  Sections used: Prerequisites
     (前置知识) > "Sparse Attention" (the {-inf, 0} mask) and "Linear
     Attention" (H, Z, O formulas); Method step details (方法步骤详情),
     steps 1-8.
[I]  ijyty.com/news/870645, article on sparse attention in video diffusion
     models.  Sections: 1.1 (spatial-temporal sliding-window attention and
     the head-wise token re-ordering), 1.2 (Top-K block-sparse attention),
     2.3 (the scalar gate), 4.1 (fixed-gate sensitivity, gate 0).
[A]  news.axiwang.com/a/172924.html, popular-science article on SALAD.
     Section 六 (technical details): ReLU linear branch with 3D rotary
     position encoding; sigmoid gate from a token average.
[G]  gist.science/fr/paper/2601.16515, French explainer.  Section 2
     (Méthodologie): A hybrid architecture, B multi-level static/dynamic
     scaling, C post-tuning branch dropping.

Where the pages leave a step open, the reading taken is stated at the
function.  Everything is float64 unless a function says it rounds.

Head kinds: 0 = spatial (frame-major order, sliding window),
1 = temporal (spatial-major order, sliding window), 2 = Top-K block sparse
(frame-major order).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "HEAD_SPATIAL", "HEAD_TEMPORAL", "HEAD_TOPK",
    "st_permutation", "head_order",
    "rope_3d", "round_to_bf16", "round_to_io",
    "to_working", "block_means", "block_scores", "topk_blocks", "topk_gap",
    "swa_keys", "topk_keys", "sparse_attention", "sparse_attention_head",
    "linear_state", "linear_apply", "gate", "combine", "combine_full", "output_projection",
    "swa_pair_count", "topk_pair_count", "branch_kept", "attn_forward",
    "dense_attention", "window_errors", "calibrate_windows",
]

HEAD_SPATIAL = 0
HEAD_TEMPORAL = 1
HEAD_TOPK = 2


# --------------------------------------------------------------------------
# Token order  ([I] 1.1)
# --------------------------------------------------------------------------

def st_permutation(F: int, Hg: int, Wg: int) -> np.ndarray:
    """Working order of a temporal head: position p holds token ``pi[p]``.

    [I] 1.1: the latent [F, Hg, Wg] is flattened with time slowest, so one
    frame's tokens are contiguous and one spatial site recurs every Hg*Wg
    tokens; temporal heads regroup the tokens by spatial site so that the
    frames of one site become contiguous.  Reading: sites in row-major
    (y, x) order, frames ascending inside a site, i.e. p = site*F + f holds
    token f*Hg*Wg + site.
    """
    S = Hg * Wg
    p = np.arange(F * S, dtype=np.int64)
    return (p % F) * S + p // F


def head_order(kind: int, F: int, Hg: int, Wg: int) -> np.ndarray:
    """Working order for one head: identity unless the head is temporal
    ([I] 1.1; Top-K heads keep the frame-major order, [I] 1.2 is silent)."""
    if kind == HEAD_TEMPORAL:
        return st_permutation(F, Hg, Wg)
    return np.arange(F * Hg * Wg, dtype=np.int64)


# --------------------------------------------------------------------------
# Rounding of materialised tensors
# --------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits (7 stored) and float32's exponent
    range.  For |x| in [2^(e-1), 2^e) the spacing of bf16 values is
    2^(e-8); below 2^-126 the spacing is fixed at 2^-133 (subnormals).
    Dividing by the spacing is exact (a power of two), so ``np.rint`` (round
    half to even) performs the single correct rounding.  Results of
    magnitude >= 2^128 overflow to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    spacing = np.ldexp(1.0, np.maximum(e.astype(np.int64) - 8, -133))
    y = np.rint(x / spacing) * spacing
    y = np.where(np.abs(y) >= 2.0 ** 128, np.copysign(np.inf, x), y)
    return np.where(np.isfinite(x), y, x)


def round_to_io(x: np.ndarray, io_dtype: str) -> np.ndarray:
    """Round a materialised tensor to the layer's storage type ("bf16" or
    "f32"); the result stays float64.  "f64" keeps every value (no storage
    rounding anywhere: the layer as a smooth function, for derivative
    checks)."""
    if io_dtype == "bf16":
        return round_to_bf16(x)
    if io_dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if io_dtype == "f64":
        return np.array(x, dtype=np.float64)
    raise ValueError(io_dtype)


# --------------------------------------------------------------------------
# 3D rotary position encoding  ([S] method step 3, [A] 六)
# --------------------------------------------------------------------------

def rope_3d(x: np.ndarray, F: int, Hg: int, Wg: int,
            dims=(44, 42, 42), base: float = 10000.0) -> np.ndarray:
    """Rotate each head vector of ``x`` [B, N, H, d] by its token's 3D position.

    [S] step 3 and [A] 六 add a 3D rotary position encoding to the linear
    branch; the layer configuration applies it to Q and K before both
    branches.  Readings: token n = f*Hg*Wg + y*Wg + xx sits at integer
    position (f, y, xx); the head dimension is cut into consecutive axis
    segments of ``dims`` (frame, height, width); inside a segment of D dims
    the pair (2i, 2i+1) turns by angle pos * base^(-2i/D).
    """
    x = np.asarray(x, dtype=np.float64)
    B, N, H, d = x.shape
    if sum(dims) != d:
        raise ValueError("rope dims must sum to head_dim")
    n = np.arange(N)
    pos = (n // (Hg * Wg), (n // Wg) % Hg, n % Wg)
    out = x.copy()
    off = 0
    for axis, D in enumerate(dims):
        for i in range(D // 2):
            theta = base ** (-2.0 * i / D)
            ang = pos[axis] * theta
            c = np.cos(ang)[None, :, None]
            s = np.sin(ang)[None, :, None]
            a = x[..., off + 2 * i]
            b = x[..., off + 2 * i + 1]
            out[..., off + 2 * i] = a * c - b * s
            out[..., off + 2 * i + 1] = a * s + b * c
        off += D
    return out


def to_working(x: np.ndarray, orders) -> np.ndarray:
    """Gather [B, N, H, d] into per-head working order [B, H, N, d]:
    working row p of head h is token orders[h][p]."""
    B, N, H, d = x.shape
    return np.stack([x[:, orders[h], h, :] for h in range(H)], axis=1)


# --------------------------------------------------------------------------
# Top-K block selection  ([I] 1.2)
# --------------------------------------------------------------------------

def block_means(xw: np.ndarray, bs: int) -> np.ndarray:
    """Mean of each block of ``bs`` consecutive rows of ``xw`` [N, d].

    [I] 1.2, first step: cut the tokens into blocks and take each block's
    mean vector.  Reading: the last block may be short and averages only
    its valid rows.
    """
    N, d = xw.shape
    nb = -(-N // bs)
    out = np.empty((nb, d), dtype=np.float64)
    for b in range(nb):
        rows = xw[b * bs:min(N, (b + 1) * bs)]
        out[b] = rows.sum(axis=0) / rows.shape[0]
    return out


def block_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """Score of key block kb for query block qb: qbar[qb] . kbar[kb].

    [I] 1.2, second step compares queries with key-block means.  Reading:
    one selection per query block, scored by the block's mean query; the
    mean over the block of q_i . kbar equals qbar . kbar by linearity, so
    both descriptions agree.  Unscaled: the ranking ignores any positive
    scale.
    """
    return np.asarray(qbar, np.float64) @ np.asarray(kbar, np.float64).T


def topk_blocks(qbar: np.ndarray, kbar: np.ndarray, k: int) -> np.ndarray:
    """Indices [nb_q, k] of the k best key blocks per query block, ascending.

    Highest score first, equal scores resolved toward the lower block index
    (a stable sort of the negated scores); no block is forced in.
    """
    S = block_scores(qbar, kbar)
    order = np.argsort(-S, axis=1, kind="stable")[:, :k]
    return np.sort(order, axis=1).astype(np.int64)


def topk_gap(qbar: np.ndarray, kbar: np.ndarray, k: int) -> np.ndarray:
    """Relative gap between the k-th and (k+1)-th best score per query
    block (inf when every block is kept).  Rows with a gap of at most 1e-6
    are near-ties whose selection legitimately depends on rounding order."""
    S = block_scores(qbar, kbar)
    nb = S.shape[1]
    if k >= nb:
        return np.full(S.shape[0], np.inf)
    srt = -np.sort(-S, axis=1)
    a, b = srt[:, k - 1], srt[:, k]
    den = np.maximum(np.maximum(np.abs(a), np.abs(b)), np.finfo(np.float64).tiny)
    return (a - b) / den


# --------------------------------------------------------------------------
# Sparse attention  ([S] Prerequisites > Sparse Attention; [I] 1.1, 1.2)
# --------------------------------------------------------------------------

def swa_keys(p: int, N: int, r: int) -> np.ndarray:
    """Keys kept for working query p under a sliding window of radius r.

    Reading of [S] Prerequisites > Sparse Attention and [I] 1.1: a
    symmetric, non-causal window {j : |p - j| <= r} on the (permuted)
    sequence, clipped at both ends.
    """
    return np.arange(max(0, p - r), min(N, p + r + 1), dtype=np.int64)


def topk_keys(p: int, idx: np.ndarray, bs: int, N: int) -> np.ndarray:
    """Keys kept for query p under Top-K selection: every row of every key
    block selected for p's query block ([I] 1.2, third step)."""
    qb = p // bs
    return np.concatenate([np.arange(kb * bs, min(N, (kb + 1) * bs), dtype=np.int64)
                           for kb in sorted(int(v) for v in idx[qb])])


def sparse_attention(qw, kw, vw, keys_of, scale: float, rows=None) -> np.ndarray:
    """Softmax attention of each working query over its kept keys.

    [S] Prerequisites > Sparse Attention: scores outside the mask are -inf,
    so each query's softmax runs over its kept keys only.  Reading: logits
    are scale * q.k with scale = 1/sqrt(d) (the pages give no scale).
    ``keys_of(p)`` returns the kept key indices; ``rows`` restricts the
    queries computed (all by default).  Returns [len(rows), d].
    """
    qw = np.asarray(qw, np.float64)
    kw = np.asarray(kw, np.float64)
    vw = np.asarray(vw, np.float64)
    N, d = qw.shape
    if rows is None:
        rows = range(N)
    rows = list(rows)
    out = np.empty((len(rows), vw.shape[1]), dtype=np.float64)
    for i, p in enumerate(rows):
        J = keys_of(int(p))
        logits = scale * (kw[J] @ qw[p])
        w = np.exp(logits - logits.max())
        out[i] = (w @ vw[J]) / w.sum()
    return out


def sparse_attention_head(kind: int, qw, kw, vw, *, r: int, bs: int, k: int,
                          scale: float, rows=None, idx=None):
    """Sparse branch for one working-order head.  Returns (O_s rows, idx)
    where idx is the Top-K selection [nb, k] (None for window heads)."""
    N = qw.shape[0]
    if kind == HEAD_TOPK:
        if idx is None:
            idx = topk_blocks(block_means(qw, bs), block_means(kw, bs), k)
        return sparse_attention(qw, kw, vw, lambda p: topk_keys(p, idx, bs, N),
                                scale, rows), idx
    return sparse_attention(qw, kw, vw, lambda p: swa_keys(p, N, r), scale, rows), None


def swa_pair_count(N: int, r: int) -> int:
    """Number of (query, key) pairs with |i - j| <= r in a length-N sequence."""
    r = min(r, N - 1)
    return N * (2 * r + 1) - r * (r + 1)


def topk_pair_count(idx: np.ndarray, bs: int, N: int) -> int:
    """Number of (query, key) pairs computed under a Top-K selection."""
    nb = idx.shape[0]
    rows_in = np.array([min(N, (b + 1) * bs) - b * bs for b in range(nb)])
    return int(sum(rows_in[qb] * rows_in[idx[qb]].sum() for qb in range(nb)))


# --------------------------------------------------------------------------
# Linear attention  ([S] Prerequisites > Linear Attention, step 3)
# --------------------------------------------------------------------------

def linear_state(k: np.ndarray, v: np.ndarray):
    """H = relu(K)^T V  [d, d_v] and Z = relu(K)^T 1  [d] over all tokens
    ([S] Prerequisites > Linear Attention, kernel phi = ReLU)."""
    pk = np.maximum(np.asarray(k, np.float64), 0.0)
    return pk.T @ np.asarray(v, np.float64), pk.sum(axis=0)


def linear_apply(q: np.ndarray, H: np.ndarray, Z: np.ndarray, eps: float = 1e-6):
    """O_l = relu(Q) H / (relu(Q) Z + eps), row by row.

    The pages' form has no eps; reading: eps = 1e-6 keeps a query whose
    features are all non-positive at O_l = 0 instead of 0/0.
    """
    pq = np.maximum(np.asarray(q, np.float64), 0.0)
    return (pq @ H) / (pq @ Z + eps)[:, None]


# --------------------------------------------------------------------------
# Gate and combine  ([S] steps 4-6, [I] 2.3, [A] 六, [G] 2.B)
# --------------------------------------------------------------------------

def gate(x: np.ndarray, w: np.ndarray, b: float) -> float:
    """s = sigmoid(w . mean_n X[n, :] + b) for one sample's X [N, C].

    [I] 2.3 and [A] 六: average the hidden state over tokens, then a linear
    layer and a sigmoid give one scalar in (0, 1).  ([S] step 5 prints the
    mean outside the sigmoid; the token-average-first order is taken.)
    """
    m = np.asarray(x, np.float64).mean(axis=0)
    t = float(np.dot(np.asarray(w, np.float64), m) + b)
    return 1.0 / (1.0 + np.exp(-t))


def combine(o_s: np.ndarray, o_l: np.ndarray, w_p: np.ndarray, s: float) -> np.ndarray:
    """O = O_s + s * (O_l W_p)  ([S] steps 4 and 6).

    [S] step 4 passes the linear output through a zero-initialised
    projection; reading: W_p is [d_in, d_out], shared by the heads of a
    layer, applied as row-vector times matrix, with no bias.
    """
    return np.asarray(o_s, np.float64) + s * (np.asarray(o_l, np.float64) @ np.asarray(w_p, np.float64))


def combine_full(o_s: np.ndarray, o_l: np.ndarray, w_p: np.ndarray, s: float) -> np.ndarray:
    """Full-width reading of the static projection ([S] step 4; the extra
    parameter count of about 5 % that [S] reports fits one [C, C] matrix per
    layer): the linear outputs of all heads of a token, concatenated in head
    order (C = H*d), pass through one projection.  o_s, o_l: [N, C] token
    rows; w_p [C, C]; O = O_s + s * (O_l W_p)."""
    return np.asarray(o_s, np.float64) + s * (np.asarray(o_l, np.float64) @ np.asarray(w_p, np.float64))


def output_projection(o: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """[S] step 7: the combined output's token rows (length C) times W^O
    [C, C] (row vector times matrix, no bias)."""
    return np.asarray(o, np.float64) @ np.asarray(w_o, np.float64)


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------

def branch_kept(s: float, tau: float) -> bool:
    """Post-tuning branch dropping ([G] 2 C; [S] step 8): at inference the
    linear branch of a sample is switched off when its dynamic scale s is
    below a threshold tau (the pages calibrate one per timestep; it is an
    input here).  Reading: s < tau drops, so tau <= 0 never drops (s > 0)."""
    return not (s < tau)


def attn_forward(q, k, v, x, w_p, gate_w, gate_b, *, grid, head_kinds,
                 window_radius, block, topk, io_dtype="bf16", rope=False,
                 rope_dims=(44, 42, 42), rope_base=10000.0, softmax_scale=None,
                 linear_eps=1e-6, s_override=None, rows=None, drop_tau=0.0,
                 proj="head", w_o=None):
    """Hybrid attention layer output for Q, K, V [B, N, H, d] and X [B, N, C].

    Steps ([S] steps 2-6): optional 3D RoPE on Q and K (materialised in the
    storage type ``io_dtype``); per-head working order ([I] 1.1); sparse
    branch per head (window or Top-K); linear branch on the same Q, K, V;
    gate per sample; O = O_s + s * (O_l W_p) written back in token order.
    With ``drop_tau`` a sample whose gate value is below it keeps only the
    sparse branch, O = O_s ([G] 2 C; see ``branch_kept``).  ``proj="full"``
    takes W_p as one [C, C] projection of each token's concatenated linear
    outputs (``combine_full``); ``w_o`` (optional, [C, C]) applies the output
    projection of [S] step 7 to each token's combined row.

    Everything but the gate is per (sample, head), so each head's inputs
    are prepared only when that head is needed.  ``rows`` (optional, a list
    of (b, n, h) triples) limits the output to those rows and returns a
    dict mapping each triple to its output vector.  Otherwise returns a dict
    with "out" [B, N, H, d] and the stage results ("o_s", "o_l", "H", "Z",
    "s", "idx", "orders", "q_used", "k_used").
    """
    F, Hg, Wg = grid
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, N, H, d = q.shape
    if N != F * Hg * Wg:
        raise ValueError("N must equal F*Hg*Wg")
    scale = 1.0 / np.sqrt(d) if not softmax_scale or softmax_scale <= 0 else softmax_scale
    orders = [head_order(int(head_kinds[h]), F, Hg, Wg) for h in range(H)]
    inv = [np.argsort(o) for o in orders]

    s = np.empty(B)
    for b in range(B):
        s[b] = gate(x[b], gate_w, gate_b) if s_override is None else float(s_override[b])

    cache = {}

    def head(b, h):
        """Token-order q, k (RoPE'd if enabled), v, working-order copies and
        the linear state of one (sample, head)."""
        key = (b, h)
        if key not in cache:
            qh = np.asarray(q[b:b + 1, :, h:h + 1], np.float64)
            kh = np.asarray(k[b:b + 1, :, h:h + 1], np.float64)
            if rope:
                qh = round_to_io(rope_3d(qh, F, Hg, Wg, rope_dims, rope_base), io_dtype)
                kh = round_to_io(rope_3d(kh, F, Hg, Wg, rope_dims, rope_base), io_dtype)
            qh, kh = qh[0, :, 0], kh[0, :, 0]
            vh = np.asarray(v[b, :, h], np.float64)
            Hm, Zv = linear_state(kh, vh)
            o = orders[h]
            cache[key] = dict(q=qh, k=kh, v=vh, qw=qh[o], kw=kh[o], vw=vh[o], H=Hm, Z=Zv, idx=None)
            if int(head_kinds[h]) == HEAD_TOPK:
                c = cache[key]
                c["idx"] = topk_blocks(block_means(c["qw"], block), block_means(c["kw"], block), topk)
        return cache[key]

    def row_parts(b, n, h):
        """O_s and O_l of one (sample, token, head), token order."""
        c = head(b, h)
        o_s, _ = sparse_attention_head(int(head_kinds[h]), c["qw"], c["kw"], c["vw"],
                                       r=window_radius, bs=block, k=topk, scale=scale,
                                       rows=[int(inv[h][n])], idx=c["idx"])
        return o_s[0], linear_apply(c["q"][n:n + 1], c["H"], c["Z"], linear_eps)[0]

    if rows is not None:
        result = {}
        token_rows = {}
        for (b, n, h) in rows:
            if proj == "head" and w_o is None:
                o_s, o_l = row_parts(b, n, h)
                result[(b, n, h)] = combine(o_s[None], o_l[None], w_p, s[b])[0] \
                    if branch_kept(s[b], drop_tau) else o_s
                continue
            # cross-head projections need the token's whole row
            if (b, n) not in token_rows:
                parts = [row_parts(b, n, hh) for hh in range(H)]
                os_row = np.concatenate([p_[0] for p_ in parts])
                ol_row = np.concatenate([p_[1] for p_ in parts])
                if not branch_kept(s[b], drop_tau):
                    row = os_row
                elif proj == "full":
                    row = combine_full(os_row[None], ol_row[None], w_p, s[b])[0]
                else:
                    row = np.concatenate([combine(parts[hh][0][None], parts[hh][1][None], w_p,
                                                  s[b])[0] for hh in range(H)])
                token_rows[(b, n)] = output_projection(row[None], w_o)[0] if w_o is not None else row
            dv = v.shape[3]
            result[(b, n, h)] = token_rows[(b, n)][h * dv:(h + 1) * dv]
        return result

    out = np.empty((B, N, H, v.shape[3]))
    o_s_all = np.empty_like(out)
    o_l_all = np.empty_like(out)
    Hs = np.empty((B, H, d, v.shape[3]))
    Zs = np.empty((B, H, d))
    q_used = np.empty((B, N, H, d))
    k_used = np.empty((B, N, H, d))
    idx_all = {}
    for b in range(B):
        for h in range(H):
            c = head(b, h)
            kind = int(head_kinds[h])
            o_s_w, _ = sparse_attention_head(kind, c["qw"], c["kw"], c["vw"], r=window_radius,
                                             bs=block, k=topk, scale=scale, idx=c["idx"])
            if c["idx"] is not None:
                idx_all[(b, h)] = c["idx"]
            o_s = o_s_w[inv[h]]  # back to token order
            o_l = linear_apply(c["q"], c["H"], c["Z"], linear_eps)
            o_s_all[b, :, h] = o_s
            o_l_all[b, :, h] = o_l
            if proj == "head":
                out[b, :, h] = combine(o_s, o_l, w_p, s[b]) if branch_kept(s[b], drop_tau) else o_s
            Hs[b, h], Zs[b, h] = c["H"], c["Z"]
            q_used[b, :, h], k_used[b, :, h] = c["q"], c["k"]
            del cache[(b, h)]
        dv = v.shape[3]
        if proj == "full":
            os_tok = o_s_all[b].reshape(N, H * dv)
            out[b] = (combine_full(os_tok, o_l_all[b].reshape(N, H * dv), w_p, s[b])
                      if branch_kept(s[b], drop_tau) else os_tok).reshape(N, H, dv)
        if w_o is not None:
            out[b] = output_projection(out[b].reshape(N, H * dv), w_o).reshape(N, H, dv)
    return {"out": out, "o_s": o_s_all, "o_l": o_l_all, "H": Hs, "Z": Zs, "s": s,
            "idx": idx_all, "orders": orders, "q_used": q_used, "k_used": k_used}


# --------------------------------------------------------------------------
# Per-head window calibration  ([I] 1.1)
# --------------------------------------------------------------------------

def dense_attention(qw, kw, vw, scale: float) -> np.ndarray:
    """Full softmax attention of every query over every key (the reference
    the window is calibrated against): one row at a time, as
    ``sparse_attention`` with every key kept."""
    N = np.shape(qw)[0]
    return sparse_attention(qw, kw, vw, lambda p: np.arange(N, dtype=np.int64), scale)


def window_errors(qw, kw, vw, radii, scale: float) -> np.ndarray:
    """Relative squared error of window attention against dense attention
    for one working-order head, per radius:
    e(r) = ||O_window(r) - O_dense||_F^2 / ||O_dense||_F^2 over all the head's
    rows ([I] 1.1 scores a window by a relative squared error against full
    attention; reading: Frobenius norms over the head's tokens)."""
    od = dense_attention(qw, kw, vw, scale)
    N = od.shape[0]
    den = float(np.sum(od * od))
    out = np.empty(len(radii))
    for i, r in enumerate(radii):
        ow = sparse_attention(qw, kw, vw, lambda p, r=int(r): swa_keys(p, N, r), scale)
        out[i] = float(np.sum((ow - od) ** 2)) / den
    return out


def calibrate_windows(q, k, v, *, grid, head_kinds, radii, tau=2.0, softmax_scale=None):
    """Per-head window radius by the greedy rule of [I] 1.1: the smallest
    radius, among ``radii`` (ascending), whose relative squared error
    against dense attention is at most ``tau`` on every calibration sample
    (the batch entries stand in for the pages' eight analysis prompts);
    N - 1 (the dense window, error 0) when none is.  Each head is evaluated
    in its working order (Top-K heads as window heads in token order).
    Readings: the bound is on the maximum over samples of the per-sample
    error; tau is an input (the pages print 2.0).  Returns (errors
    [len(radii), B, H], radius per head [H])."""
    F, Hg, Wg = grid
    q = np.asarray(q)
    B, N, H, d = q.shape
    scale = 1.0 / np.sqrt(d) if not softmax_scale or softmax_scale <= 0 else softmax_scale
    radii = [int(r) for r in radii]
    if any(b <= a for a, b in zip(radii, radii[1:])):
        raise ValueError("radii must be ascending")
    err = np.empty((len(radii), B, H))
    for h in range(H):
        order = head_order(int(head_kinds[h]), F, Hg, Wg)
        for b in range(B):
            w = [np.asarray(t[b, :, h], np.float64)[order] for t in (q, k, v)]
            err[:, b, h] = window_errors(*w, radii, scale)
    choice = np.full(H, N - 1, dtype=np.int64)
    for h in range(H):
        for i, r in enumerate(radii):
            if err[i, :, h].max() <= tau:
                choice[h] = r
                break
    return err, choice
