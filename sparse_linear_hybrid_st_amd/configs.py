"""Synthetic workloads for the hybrid attention layer (video-DiT shapes).

Each workload fixes the latent grid, heads, head dim, storage type, the
per-head kind and the sparsity parameters.  The window radius at 90 %
sparsity is the smallest r whose symmetric window keeps at least 10 % of
all query-key pairs; the Top-K count is ceil(0.1 * number of key blocks).

Head kinds: 0 spatial (frame-major, window), 1 temporal (spatial-major,
window), 2 Top-K block sparse (frame-major).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

HEAD_SPATIAL, HEAD_TEMPORAL, HEAD_TOPK = 0, 1, 2


def window_pairs(N: int, r: int) -> int:
    """Query-key pairs with |i - j| <= r in a length-N sequence."""
    r = min(r, N - 1)
    return N * (2 * r + 1) - r * (r + 1)


def radius_for_density(N: int, density: float) -> int:
    """Smallest window radius keeping at least ``density`` of the N^2 pairs."""
    target = density * N * N
    lo, hi = 0, N - 1
    while lo < hi:
        mid = (lo + hi) // 2
        if window_pairs(N, mid) >= target:
            hi = mid
        else:
            lo = mid + 1
    return lo


@dataclass
class Workload:
    name: str
    seed: int
    batch: int
    grid: tuple            # (F, Hg, Wg), frame-major flattening
    n_heads: int
    head_dim: int
    io_dtype: str          # "f32" or "bf16"
    head_kinds: list
    window_radius: int
    block: int
    topk: int
    rope: bool = False
    rope_dims: tuple = (44, 42, 42)
    rope_base: float = 10000.0
    qk_channel_scale: bool = True   # Q, K = N(0,1) * exp(N(0, 0.5)) per channel
    x_sample_shift: bool = False    # X[b] += N(0, 0.5) per sample
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        F, H, W = self.grid
        return F * H * W

    @property
    def hidden(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def n_blocks(self) -> int:
        return -(-self.N // self.block)


def _alternate(h: int) -> list:
    return [HEAD_SPATIAL if i % 2 == 0 else HEAD_TEMPORAL for i in range(h)]


def _mixed(h: int) -> list:
    return [(HEAD_SPATIAL, HEAD_TEMPORAL, HEAD_TOPK, HEAD_TOPK)[i % 4] for i in range(h)]


def tiny_f32(topk: bool = False) -> Workload:
    """4 x 8 x 8 = 256 tokens, 2 heads of 64, fp32; 64-token window
    (radius 32); Top-K variant with block 32 keeping 2 of 8 key blocks."""
    return Workload(
        name="tiny-f32-topk" if topk else "tiny-f32", seed=1001, batch=1, grid=(4, 8, 8),
        n_heads=2, head_dim=64, io_dtype="f32",
        head_kinds=[HEAD_TOPK, HEAD_TOPK] if topk else [HEAD_SPATIAL, HEAD_TEMPORAL],
        window_radius=32, block=32, topk=2, qk_channel_scale=False,
        description="tiny fp32 parity case, N=256, 2 heads, d=64")


def swa_480p() -> Workload:
    """480p-like: 20 x 30 x 52 = 31,200 tokens, 12 heads of 128, bf16,
    half spatial / half temporal, window at 90 % sparsity."""
    N = 20 * 30 * 52
    return Workload(
        name="480p-stswa-h12", seed=1002, batch=1, grid=(20, 30, 52), n_heads=12,
        head_dim=128, io_dtype="bf16", head_kinds=_alternate(12),
        window_radius=radius_for_density(N, 0.1), block=64, topk=math.ceil(0.1 * (-(-N // 64))),
        description="N=31,200, 12 heads, d=128, ST sliding window, 90% sparsity")


def topk_480p() -> Workload:
    """480p-like Top-K: 31,200 tokens, 40 heads, block 64, top 49 of 488."""
    N = 20 * 30 * 52
    return Workload(
        name="480p-topk-h40", seed=1003, batch=1, grid=(20, 30, 52), n_heads=40,
        head_dim=128, io_dtype="bf16", head_kinds=[HEAD_TOPK] * 40,
        window_radius=radius_for_density(N, 0.1), block=64,
        topk=math.ceil(0.1 * (-(-N // 64))),
        description="N=31,200, 40 heads, d=128, Top-K block 64, k=49 of 488")


def swa_720p() -> Workload:
    """720p-like: 21 x 45 x 80 = 75,600 tokens, 40 heads, window at 90 %."""
    N = 21 * 45 * 80
    return Workload(
        name="720p-stswa-h40", seed=1004, batch=1, grid=(21, 45, 80), n_heads=40,
        head_dim=128, io_dtype="bf16", head_kinds=_alternate(40),
        window_radius=radius_for_density(N, 0.1), block=64, topk=math.ceil(0.1 * (-(-N // 64))),
        description="N=75,600, 40 heads, d=128, ST sliding window, 90% sparsity")


def cfg_rope_480p() -> Workload:
    """CFG pair: batch 2 at 31,200 tokens, 40 heads, 3D RoPE 44/42/42,
    heads mixed (h mod 4: spatial, temporal, Top-K, Top-K)."""
    N = 20 * 30 * 52
    return Workload(
        name="480p-cfg-rope-mixed-h40", seed=1005, batch=2, grid=(20, 30, 52), n_heads=40,
        head_dim=128, io_dtype="bf16", head_kinds=_mixed(40),
        window_radius=radius_for_density(N, 0.1), block=64,
        topk=math.ceil(0.1 * (-(-N // 64))), rope=True, x_sample_shift=True,
        description="B=2, N=31,200, 40 heads, RoPE, 50% Top-K / 50% ST window")


def all_workloads() -> dict:
    return {w.name: w for w in (tiny_f32(), tiny_f32(True), swa_480p(), topk_480p(),
                                swa_720p(), cfg_rope_480p())}


def small(name: str, grid, n_heads: int, head_dim: int, io_dtype: str, head_kinds,
          window_radius: int, block: int, topk: int, batch: int = 1, rope: bool = False,
          rope_dims=None, seed: int = 7, **kw) -> Workload:
    """A custom small workload for parity and edge-case tests."""
    if rope_dims is None:
        a = (head_dim // 3) // 2 * 2
        rope_dims = (head_dim - 2 * a, a, a)
    return Workload(name=name, seed=seed, batch=batch, grid=tuple(grid), n_heads=n_heads,
                    head_dim=head_dim, io_dtype=io_dtype, head_kinds=list(head_kinds),
                    window_radius=window_radius, block=block, topk=topk, rope=rope,
                    rope_dims=tuple(rope_dims), **kw)
