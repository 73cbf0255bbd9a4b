"""Planted mistakes: each plausible error in the oracle must fail a pin.

Every case swaps one oracle function for a subtly wrong variant (a dropped
term, a wrong sign, an off-by-one, a transposed operand) and checks that
the named pin test then fails.  Runs on the CPU only.
"""

import numpy as np
import pytest

import oracle
import oracle.salad_backward as sb
import oracle.salad_oracle as so
from tests import test_oracle_attention as TA
from tests import test_oracle_backward as TB
from tests import test_oracle_calibrate as TC
from tests import test_oracle_linear as TL
from tests import test_oracle_order as TO
from tests import test_oracle_rope as TR


def _patch(monkeypatch, name, fn):
    for mod in (so, sb, oracle):
        if hasattr(mod, name):
            monkeypatch.setattr(mod, name, fn)


def _perm_inverse(F, Hg, Wg):          # frame-major read as site-major (the inverse map)
    S = Hg * Wg
    n = np.arange(F * S)
    return (n % S) * F + n // S


def _swa_keys_short(p, N, r):          # window one key short on the right
    return np.arange(max(0, p - r), min(N, p + r), dtype=np.int64)


def _attn_no_shift(qw, kw, vw, keys_of, scale, rows=None):   # scale dropped
    return so.__dict__["_orig_sparse_attention"](qw, kw, vw, keys_of, 1.0, rows)


def _topk_smallest(qbar, kbar, k):     # keeps the lowest scores
    S = so.block_scores(qbar, kbar)
    return np.sort(np.argsort(S, axis=1, kind="stable")[:, :k], axis=1)


def _topk_high_ties(qbar, kbar, k):    # equal scores resolved toward the higher index
    S = so.block_scores(qbar, kbar)[:, ::-1]
    nb = S.shape[1]
    return np.sort(nb - 1 - np.argsort(-S, axis=1, kind="stable")[:, :k], axis=1)


def _topk_gap_next_ranks(qbar, kbar, k):   # compares ranks k+1 and k+2 (off by one)
    S = so.block_scores(qbar, kbar)
    if k + 1 >= S.shape[1]:
        return np.full(S.shape[0], np.inf)
    srt = -np.sort(-S, axis=1)
    a, b = srt[:, k], srt[:, k + 1]
    return (a - b) / np.maximum(np.maximum(np.abs(a), np.abs(b)), np.finfo(np.float64).tiny)


def _topk_gap_min_scale(qbar, kbar, k):     # divides by the smaller magnitude
    S = so.block_scores(qbar, kbar)
    if k >= S.shape[1]:
        return np.full(S.shape[0], np.inf)
    srt = -np.sort(-S, axis=1)
    a, b = srt[:, k - 1], srt[:, k]
    return (a - b) / np.maximum(np.minimum(np.abs(a), np.abs(b)), np.finfo(np.float64).tiny)


def _means_tail_by_bs(xw, bs):         # short last block divided by the full size
    N, d = xw.shape
    nb = -(-N // bs)
    return np.stack([xw[b * bs:(b + 1) * bs].sum(0) / bs for b in range(nb)])


def _linear_apply_no_relu(q, H, Z, eps=1e-6):
    q = np.asarray(q, np.float64)
    return (q @ H) / (q @ Z + eps)[:, None]


def _linear_state_relu_v(k, v):
    pk = np.maximum(k, 0)
    return pk.T @ np.maximum(v, 0), pk.sum(0)


def _rot(x, F, Hg, Wg, dims, base, sign):
    x = np.asarray(x, np.float64)
    N = x.shape[1]
    n = np.arange(N)
    pos = (n // (Hg * Wg), (n // Wg) % Hg, n % Wg)
    out = x.copy()
    off = 0
    for axis, D in enumerate(dims):
        for i in range(D // 2):
            ang = sign * pos[axis] * base ** (-2.0 * i / D)
            c, s = np.cos(ang)[None, :, None], np.sin(ang)[None, :, None]
            a, b = x[..., off + 2 * i], x[..., off + 2 * i + 1]
            out[..., off + 2 * i] = a * c - b * s
            out[..., off + 2 * i + 1] = a * s + b * c
        off += D
    return out


def _gate_sum(x, w, b):                # token sum instead of mean
    t = float(np.dot(w, np.asarray(x, np.float64).sum(0)) + b)
    return 1.0 / (1.0 + np.exp(-t))


def _combine_transposed(o_s, o_l, w_p, s):
    return np.asarray(o_s, np.float64) + s * (np.asarray(o_l) @ np.asarray(w_p).T)


def _bf16_truncate(x):                 # rounds toward zero instead of to nearest
    x = np.asarray(x, np.float64)
    _, e = np.frexp(x)
    sp = np.ldexp(1.0, np.maximum(e.astype(np.int64) - 8, -133))
    return np.trunc(x / sp) * sp


def _drop_inverted(s, tau):            # drops the samples above the threshold
    return s < tau


def _drop_at_equality(s, tau):         # drops a gate value equal to the threshold
    return s > tau


def _combine_full_transposed(o_s, o_l, w_p, s):   # W_p applied as its transpose
    return np.asarray(o_s, np.float64) + s * (np.asarray(o_l, np.float64) @ np.asarray(w_p, np.float64).T)


def _output_projection_transposed(o, w_o):          # W^O applied as its transpose
    return np.asarray(o, np.float64) @ np.asarray(w_o, np.float64).T


def _sparse_bwd_uncentred(qw, kw, vw, keys_of, scale, gw):   # softmax Jacobian without - P.dP
    qw, kw, vw, gw = (np.asarray(t, np.float64) for t in (qw, kw, vw, gw))
    dq, dk, dv = np.zeros_like(qw), np.zeros_like(kw), np.zeros_like(vw)
    for p in range(qw.shape[0]):
        J = keys_of(p)
        lg = scale * (kw[J] @ qw[p])
        P = np.exp(lg - lg.max())
        P /= P.sum()
        dv[J] += np.outer(P, gw[p])
        dl = P * (vw[J] @ gw[p])
        dq[p] = scale * (dl @ kw[J])
        dk[J] += scale * np.outer(dl, qw[p])
    return dq, dk, dv


def _rope_t_as_forward(g, F, Hg, Wg, dims=(44, 42, 42), base=10000.0):   # rotation, not its transpose
    return so.rope_3d(g, F, Hg, Wg, dims, base)


def _linear_bwd_no_den(q, k, v, g, eps=1e-6):      # the normaliser's gradient dropped
    H, Z = so.linear_state(k, v)
    a = np.maximum(q, 0.0)
    den = a @ Z + eps
    dnum = g / den[:, None]
    dH = a.T @ dnum
    return (dnum @ H.T) * (q > 0), (v @ dH.T) * (k > 0), np.maximum(k, 0.0) @ dH


def _gate_bwd_no_one_minus_s(x, w, b, ds):         # sigmoid derivative taken as s
    x, w = np.asarray(x, np.float64), np.asarray(w, np.float64)
    dt = ds * so.gate(x, w, b)
    return np.broadcast_to(dt * w / x.shape[0], x.shape).copy(), dt * x.mean(axis=0), dt


def _window_errors_by_window_norm(qw, kw, vw, radii, scale):   # divides by ||O_window|| instead
    od = so.dense_attention(qw, kw, vw, scale)
    N = od.shape[0]
    out = np.empty(len(radii))
    for i, r in enumerate(radii):
        ow = so.sparse_attention(qw, kw, vw, lambda p, r=int(r): so.swa_keys(p, N, r), scale)
        out[i] = float(np.sum((ow - od) ** 2)) / float(np.sum(ow * ow))
    return out


def _calibrate_mean_over_samples(q, k, v, *, grid, head_kinds, radii, tau=2.0, softmax_scale=None):
    err, _ = _orig_calibrate(q, k, v, grid=grid, head_kinds=head_kinds, radii=radii, tau=tau,
                             softmax_scale=softmax_scale)
    N = np.shape(q)[1]
    choice = np.full(err.shape[2], N - 1, dtype=np.int64)
    for h in range(err.shape[2]):
        for i, r in enumerate(radii):
            if err[i, :, h].mean() <= tau:         # the bound on the average sample
                choice[h] = r
                break
    return err, choice


_orig_calibrate = so.calibrate_windows

CASES = [
    ("st_permutation", _perm_inverse, lambda: TO.test_st_permutation_matches_sort_construction((4, 8, 8))),
    ("swa_keys", _swa_keys_short, lambda: TA.test_window_matches_masked_dense(64, 5)),
    ("sparse_attention", _attn_no_shift, lambda: TA.test_full_window_is_dense_attention(50, 49)),
    ("topk_blocks", _topk_smallest, lambda: TA.test_topk_matches_brute_force(13, 5)),
    ("topk_blocks", _topk_high_ties, TA.test_topk_ties_prefer_lower_index_and_planted_block),
    ("block_means", _means_tail_by_bs, TA.test_block_means_even_and_tail),
    ("topk_gap", _topk_gap_next_ranks, TA.test_topk_gap_finite_values),
    ("topk_gap", _topk_gap_next_ranks, TA.test_topk_gap_matches_exact_rational_brute_force),
    ("topk_gap", _topk_gap_min_scale, TA.test_topk_gap_finite_values),
    ("linear_apply", _linear_apply_no_relu, TL.test_linear_closed_form_equals_quadratic_expansion),
    ("linear_state", _linear_state_relu_v, TL.test_linear_closed_form_equals_quadratic_expansion),
    ("rope_3d", lambda x, F, Hg, Wg, dims=(44, 42, 42), base=10000.0: _rot(x, F, Hg, Wg, dims, base, -1.0),
     lambda: TR.test_rope_matches_complex_form((3, 4, 5), (4, 6, 6))),
    ("gate", _gate_sum, TL.test_gate_values),
    ("combine", _combine_transposed, TL.test_combine_special_cases),
    ("round_to_bf16", _bf16_truncate, TO.test_round_to_bf16_exact_on_float64_values),
    ("branch_kept", _drop_inverted, TL.test_layer_branch_dropping),
    ("branch_kept", _drop_at_equality, TL.test_layer_branch_dropping),
    ("combine_full", _combine_full_transposed, TL.test_layer_full_width_projection_and_output_projection),
    ("output_projection", _output_projection_transposed,
     TL.test_layer_full_width_projection_and_output_projection),
    ("sparse_attention_backward", _sparse_bwd_uncentred, lambda: TB.test_backward_matches_finite_differences(False)),
    ("rope_3d_transpose", _rope_t_as_forward, lambda: TB.test_backward_matches_finite_differences(True)),
    ("linear_backward", _linear_bwd_no_den, lambda: TB.test_backward_matches_finite_differences(False)),
    ("gate_backward", _gate_bwd_no_one_minus_s, lambda: TB.test_backward_matches_finite_differences(False)),
    ("window_errors", _window_errors_by_window_norm, TC.test_errors_match_masked_sdpa_and_dense_is_exact),
    ("calibrate_windows", _calibrate_mean_over_samples, TC.test_greedy_choice_is_smallest_radius_meeting_the_bound),
]


@pytest.mark.parametrize("name,mutant,pin", CASES, ids=[c[0] + str(i) for i, c in enumerate(CASES)])
def test_pin_catches_planted_mistake(monkeypatch, name, mutant, pin):
    so.__dict__.setdefault("_orig_sparse_attention", so.sparse_attention)
    pin()                       # the pin passes on the real oracle
    _patch(monkeypatch, name, mutant)
    with pytest.raises(AssertionError):
        pin()
