"""Seeded synthetic inputs for a workload (shared by tests, bench and smoke).

This module draws random numbers and rounds them to the storage type; it
holds none of the attention arithmetic.  Tensors come back as float32
numpy arrays whose values are exactly representable in the storage type
(bf16 workloads are rounded to nearest-even once, here), so the HIP path
and the oracle see bit-identical inputs.

Recipe (N(mu, sigma) is mean and standard deviation):
  stream(t) = numpy default_rng(SeedSequence([seed, t]))
  Q = N(0,1) [B,N,H,d] (t=0) times c_Q, c_Q = exp(N(0,0.5)) per channel (t=6)
  K = N(0,1) [B,N,H,d] (t=1) times c_K = exp(N(0,0.5)) per channel (t=7)
  (the channel scales are 1 for workloads without them)
  V = N(0,1) [B,N,H,d] (t=2)
  X = N(0,1) [B,N,C] (t=3) plus, if enabled, a per-sample N(0,0.5) shift (t=8)
  W_p = N(0,0.02) [d,d] (t=4), gate w = N(0,0.02) [C] (t=5), gate b = 0
  full-width W_p = N(0,0.02) [C,C] (t=9); output projection
  W^O = N(0, 1/sqrt(C)) [C,C] (t=10)
"""

from __future__ import annotations

import numpy as np
import torch

T_Q, T_K, T_V, T_X, T_WP, T_W, T_CQ, T_CK, T_SHIFT, T_WPF, T_WO = range(11)


def _rng(seed: int, t: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, t]))


def _normal(seed: int, t: int, shape, std: float = 1.0) -> np.ndarray:
    a = _rng(seed, t).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def to_storage(a: np.ndarray, io_dtype: str) -> torch.Tensor:
    """CPU tensor in the storage type (bf16 rounding is nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16) if io_dtype == "bf16" else t


def make_inputs(w, wp_std: float = 0.02, wp_zero: bool = False, proj: str = "head") -> dict:
    """CPU storage-type tensors q, k, v [B,N,H,d], x [B,N,C], w_p ([d,d], or
    [C,C] with proj="full"), gate_w [C] and the float gate_b, for workload
    ``w``."""
    B, N, H, d = w.batch, w.N, w.n_heads, w.head_dim
    C = H * d
    s = w.seed
    out = {}
    for name, t, tc in (("q", T_Q, T_CQ), ("k", T_K, T_CK)):
        a = _normal(s, t, (B, N, H, d))
        if w.qk_channel_scale:
            c = np.exp(_normal(s, tc, (H, d), 0.5)).astype(np.float32)
            a *= c[None, None]
        out[name] = to_storage(a, w.io_dtype)
        del a
    out["v"] = to_storage(_normal(s, T_V, (B, N, H, d)), w.io_dtype)
    x = _normal(s, T_X, (B, N, C))
    if w.x_sample_shift:
        x += _normal(s, T_SHIFT, (B,), 0.5)[:, None, None]
    out["x"] = to_storage(x, w.io_dtype)
    del x
    shape, t_wp = ((C, C), T_WPF) if proj == "full" else ((d, d), T_WP)
    wp = np.zeros(shape, np.float32) if wp_zero else _normal(s, t_wp, shape, wp_std)
    out["w_p"] = to_storage(wp, w.io_dtype)
    out["gate_w"] = to_storage(_normal(s, T_W, (C,), 0.02), w.io_dtype)
    out["gate_b"] = 0.0
    return out


def make_w_o(w) -> torch.Tensor:
    """Output projection W^O [C, C] in the storage type of workload ``w``."""
    C = w.n_heads * w.head_dim
    return to_storage(_normal(w.seed, T_WO, (C, C), 1.0 / np.sqrt(C)), w.io_dtype)


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a storage-type CPU tensor (for the oracle)."""
    return t.to(torch.float64).numpy()
