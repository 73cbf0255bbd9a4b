"""Whole heads of the oracle's layer output at full size, on several CPU
processes.

TEST INFRASTRUCTURE ONLY, like the rest of this package: used by the
full-size parity tests and by bench.py's CPU baseline.  It adds no
arithmetic: it only splits the rows of one head into chunks and runs the
oracle's own ``attn_forward`` on each chunk.

The oracle computes output rows one at a time; one head of a 31,200-token
layer is about forty seconds of that on one core.  Here the rows of one
(sample, head) are split into contiguous chunks and each chunk runs in its
own spawned process, which calls ``oracle.attn_forward`` unchanged on that
head's slice of the inputs (everything in the layer except the gate is per
sample and head, and the gate value is passed in).  The workers import only
numpy and the oracle and never touch the GPU.
"""

from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import tempfile

import numpy as np

from . import salad_oracle as O


def _chunk(args):
    paths, s_b, kw, rows = args
    q, k, v, wp = (np.load(p, mmap_mode="r") for p in paths)
    res = O.attn_forward(q, k, v, None, wp, None, 0.0, s_override=[s_b],
                         rows=[(0, int(n), 0) for n in rows], **kw)
    return np.stack([res[(0, int(n), 0)] for n in rows])


def _ready(_):
    return np.float64(O.gate(np.ones((2, 2)), np.ones(2), 0.0))


def warm(n_proc: int | None = None) -> None:
    """Start and stop one pool of workers that import numpy and the oracle,
    so that a timed run does not pay the first, cold start of the
    interpreters and their imports."""
    n_proc = n_proc or workers()
    with cf.ProcessPoolExecutor(n_proc, mp_context=mp.get_context("spawn")) as pool:
        list(pool.map(_ready, range(n_proc)))


def workers() -> int:
    """CPU processes to use: the host's cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def whole_head(w, args, s_b: float, b: int, h: int, n_proc: int | None = None) -> np.ndarray:
    """Oracle output out[b, :, h, :] (token order, float64) for workload
    ``w``; ``args`` are the oracle inputs (q, k, v, x, w_p, gate_w) as float
    arrays holding the storage values, ``s_b`` the sample's gate value."""
    n_proc = n_proc or workers()
    q, k, v = (np.ascontiguousarray(a[b:b + 1, :, h:h + 1], np.float64) for a in args[:3])
    kw = dict(grid=w.grid, head_kinds=[int(w.head_kinds[h])], window_radius=w.window_radius,
              block=w.block, topk=w.topk, io_dtype=w.io_dtype, rope=w.rope,
              rope_dims=w.rope_dims, rope_base=w.rope_base)
    with tempfile.TemporaryDirectory() as tmp:
        paths = []
        for name, a in (("q", q), ("k", k), ("v", v), ("wp", np.asarray(args[4], np.float64))):
            p = os.path.join(tmp, name + ".npy")
            np.save(p, a)
            paths.append(p)
        bounds = np.linspace(0, w.N, 2 * n_proc + 1).astype(int)
        jobs = [(paths, float(s_b), kw, range(bounds[i], bounds[i + 1]))
                for i in range(len(bounds) - 1) if bounds[i + 1] > bounds[i]]
        # one BLAS thread per worker; the environment is read when the
        # spawned worker imports numpy
        saved = {n: os.environ.get(n) for n in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")}
        for n in saved:
            os.environ[n] = "1"
        try:
            # a worker that dies raises BrokenProcessPool here (no respawn loop)
            with cf.ProcessPoolExecutor(n_proc, mp_context=mp.get_context("spawn")) as pool:
                parts = list(pool.map(_chunk, jobs))
        finally:
            for n, val in saved.items():
                if val is None:
                    os.environ.pop(n, None)
                else:
                    os.environ[n] = val
    return np.concatenate(parts)
