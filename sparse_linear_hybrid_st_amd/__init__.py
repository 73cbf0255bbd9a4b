"""Python binding of the gfx950 hybrid attention library (libsalad.so).

The functions here carry the C ABI's names and only marshal arguments:
torch tensors become device pointers, the current torch stream becomes the
hipStream_t, and shapes are checked against the problem before the call so
that no kernel is launched on a buffer of the wrong size.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  If
libsalad.so is missing the first call raises.

Problem: :class:`Problem` mirrors ``salad_problem``; build one from a
workload with :func:`problem_from_workload`.
"""

from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# SALAD_LIB: another build of the same library (the sanitizer test's
# host-instrumented build); by default the in-tree libsalad.so.
LIB_PATH = os.environ.get("SALAD_LIB") or os.path.join(HERE, "libsalad.so")

SALAD_F32, SALAD_BF16 = 0, 1
HEAD_SPATIAL, HEAD_TEMPORAL, HEAD_TOPK = 0, 1, 2
PROJ_HEAD, PROJ_FULL = 0, 1
MAX_HEADS = 256

STATUS = {0: "SALAD_OK", 1: "SALAD_ERR_NULL", 2: "SALAD_ERR_SHAPE", 3: "SALAD_ERR_UNSUPPORTED",
          4: "SALAD_ERR_ALIGN", 5: "SALAD_ERR_WORKSPACE", 6: "SALAD_ERR_HIP"}

EXPORTS = ("salad_workspace_size", "salad_permute", "salad_block_select", "salad_sparse_attn",
           "salad_linear_state", "salad_linear_apply", "salad_gate", "salad_combine",
           "salad_attn_forward", "salad_output_projection", "salad_backward_workspace_size",
           "salad_attn_backward", "salad_calibrate_workspace_size", "salad_window_calibrate",
           "salad_attn_forward_timed", "salad_attn_backward_timed", "salad_linear_state_noalloc",
           "salad_last_error")


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("grid_f", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
        ("head_kind", ctypes.c_uint8 * MAX_HEADS),
        ("window_radius", ctypes.c_int32), ("block", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("linear_eps", ctypes.c_float),
        ("rope", ctypes.c_int32), ("rope_dims", ctypes.c_int32 * 3), ("rope_base", ctypes.c_float),
        ("io_dtype", ctypes.c_int32), ("branch_drop_tau", ctypes.c_float),
        ("proj_mode", ctypes.c_int32),
    ]

    @property
    def N(self) -> int:
        return self.grid_f * self.grid_h * self.grid_w

    @property
    def n_blocks(self) -> int:
        return -(-self.N // self.block) if self.block > 0 else 0

    @property
    def C(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def w_p_numel(self) -> int:
        """Elements of W_p: [d, d] per head, or [C, C] full width."""
        return self.C ** 2 if self.proj_mode == PROJ_FULL else self.head_dim ** 2

    @property
    def kinds(self):
        return [self.head_kind[h] for h in range(self.n_heads)]


class SaladError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libsalad.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: build it with "
                               "`python -m sparse_linear_hybrid_st_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, vp, sz = ctypes.POINTER(Problem), ctypes.c_void_p, ctypes.c_size_t
        i32, f32 = ctypes.c_int, ctypes.c_float
        sigs = {
            "salad_workspace_size": [P, ctypes.POINTER(sz)],
            "salad_permute": [P, i32, i32, vp, vp, vp],
            "salad_block_select": [P, vp, vp, vp, vp, vp, vp, sz, vp],
            "salad_sparse_attn": [P, vp, vp, vp, vp, vp, vp],
            "salad_linear_state": [P, vp, vp, vp, vp, vp, sz, vp],
            "salad_linear_state_noalloc": [P, vp, vp, vp, vp, vp],
            "salad_linear_apply": [P, vp, vp, vp, vp, vp],
            "salad_gate": [P, vp, vp, f32, vp, vp, sz, vp],
            "salad_combine": [P, vp, vp, vp, vp, vp, vp],
            "salad_attn_forward": [P, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, vp, sz, vp],
            "salad_output_projection": [P, vp, vp, vp, vp],
            "salad_backward_workspace_size": [P, ctypes.POINTER(sz)],
            "salad_calibrate_workspace_size": [P, ctypes.POINTER(sz)],
            "salad_window_calibrate": [P, vp, vp, vp, vp, i32, f32, vp, vp, vp, sz, vp],
            "salad_attn_backward": [P, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                    vp, vp, vp, sz, vp],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        for name in ("salad_attn_forward", "salad_attn_backward"):
            fn = getattr(L, name + "_timed")
            fn.argtypes = sigs[name] + [vp, vp]
            fn.restype = ctypes.c_int
        L.salad_last_error.argtypes = []
        L.salad_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise SaladError(status, lib().salad_last_error().decode())


def make_problem(*, batch, n_heads, head_dim, grid, head_kinds, window_radius=0, block=64,
                 topk=1, softmax_scale=0.0, linear_eps=1e-6, rope=False, rope_dims=(0, 0, 0),
                 rope_base=10000.0, io_dtype="bf16", branch_drop_tau=0.0, proj="head") -> Problem:
    p = Problem()
    p.batch, p.n_heads, p.head_dim = batch, n_heads, head_dim
    p.grid_f, p.grid_h, p.grid_w = grid
    for h, k in enumerate(head_kinds):
        p.head_kind[h] = int(k)
    p.window_radius, p.block, p.topk = window_radius, block, topk
    p.softmax_scale, p.linear_eps = softmax_scale, linear_eps
    p.rope = int(bool(rope))
    for i in range(3):
        p.rope_dims[i] = int(rope_dims[i])
    p.rope_base = rope_base
    p.io_dtype = SALAD_BF16 if io_dtype == "bf16" else SALAD_F32
    p.branch_drop_tau = branch_drop_tau
    if proj not in ("head", "full"):
        raise ValueError(f"proj must be 'head' or 'full' (got {proj!r})")
    p.proj_mode = PROJ_FULL if proj == "full" else PROJ_HEAD
    return p


def problem_from_workload(w, branch_drop_tau=0.0, proj="head") -> Problem:
    return make_problem(batch=w.batch, n_heads=w.n_heads, head_dim=w.head_dim, grid=w.grid,
                        head_kinds=w.head_kinds, window_radius=w.window_radius, block=w.block,
                        topk=w.topk, rope=w.rope, rope_dims=w.rope_dims, rope_base=w.rope_base,
                        io_dtype=w.io_dtype, branch_drop_tau=branch_drop_tau, proj=proj)


# ---- marshalling helpers --------------------------------------------------

def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t, name, numel=None, dtype=None):
    """Device pointer of a contiguous tensor after checking its size/type."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _io_dtype(p: Problem):
    import torch
    return torch.bfloat16 if p.io_dtype == SALAD_BF16 else torch.float32


def _sizes(p: Problem):
    rows = p.batch * p.n_heads * p.N * p.head_dim
    return rows, p.batch * p.N * p.n_heads * p.head_dim


# ---- entry points (same names as the C ABI) -------------------------------

def salad_workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().salad_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def salad_permute(p: Problem, apply_rope: int, inverse: int, src, dst, stream=None):
    import torch
    n, _ = _sizes(p)
    dt = _io_dtype(p)
    _check(lib().salad_permute(ctypes.byref(p), int(apply_rope), int(inverse),
                               _ptr(src, "src", n, dt), _ptr(dst, "dst", n, dt), _stream(stream)))


def salad_block_select(p: Problem, qw, kw, idx, ws, qbar=None, kbar=None, stream=None):
    import torch
    n, _ = _sizes(p)
    dt = _io_dtype(p)
    nb = p.n_blocks
    means = p.batch * p.n_heads * nb * p.head_dim
    _check(lib().salad_block_select(
        ctypes.byref(p), _ptr(qw, "qw", n, dt), _ptr(kw, "kw", n, dt),
        _ptr(idx, "idx", p.batch * p.n_heads * nb * p.topk, torch.int32),
        _ptr(qbar, "qbar", means, torch.float64), _ptr(kbar, "kbar", means, torch.float64),
        _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)))


def salad_sparse_attn(p: Problem, qw, kw, vw, idx, o_s, stream=None):
    import torch
    n, _ = _sizes(p)
    dt = _io_dtype(p)
    nidx = p.batch * p.n_heads * p.n_blocks * p.topk
    _check(lib().salad_sparse_attn(
        ctypes.byref(p), _ptr(qw, "qw", n, dt), _ptr(kw, "kw", n, dt), _ptr(vw, "vw", n, dt),
        _ptr(idx, "idx", nidx, torch.int32), _ptr(o_s, "o_s", n, torch.float32), _stream(stream)))


def salad_linear_state(p: Problem, kw, vw, h, z, ws, stream=None):
    import torch
    n, _ = _sizes(p)
    dt = _io_dtype(p)
    bh = p.batch * p.n_heads
    _check(lib().salad_linear_state(
        ctypes.byref(p), _ptr(kw, "kw", n, dt), _ptr(vw, "vw", n, dt),
        _ptr(h, "h", bh * p.head_dim ** 2, torch.float32), _ptr(z, "z", bh * p.head_dim, torch.float32),
        _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)))


def salad_linear_state_noalloc(p: Problem, kw, vw, h, z, stream=None):
    """salad_linear_state with the library's own fixed device scratch (no
    workspace; allocates nothing)."""
    import torch
    n, _ = _sizes(p)
    dt = _io_dtype(p)
    bh = p.batch * p.n_heads
    _check(lib().salad_linear_state_noalloc(
        ctypes.byref(p), _ptr(kw, "kw", n, dt), _ptr(vw, "vw", n, dt),
        _ptr(h, "h", bh * p.head_dim ** 2, torch.float32), _ptr(z, "z", bh * p.head_dim, torch.float32),
        _stream(stream)))


def salad_linear_apply(p: Problem, qw, h, z, o_l, stream=None):
    import torch
    n, _ = _sizes(p)
    bh = p.batch * p.n_heads
    _check(lib().salad_linear_apply(
        ctypes.byref(p), _ptr(qw, "qw", n, _io_dtype(p)),
        _ptr(h, "h", bh * p.head_dim ** 2, torch.float32), _ptr(z, "z", bh * p.head_dim, torch.float32),
        _ptr(o_l, "o_l", n, torch.float32), _stream(stream)))


def salad_gate(p: Problem, x, w, bias: float, s, ws, stream=None):
    import torch
    C = p.n_heads * p.head_dim
    dt = _io_dtype(p)
    _check(lib().salad_gate(
        ctypes.byref(p), _ptr(x, "x", p.batch * p.N * C, dt), _ptr(w, "w", C, dt), float(bias),
        _ptr(s, "s", p.batch, torch.float32), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
        _stream(stream)))


def salad_combine(p: Problem, o_s, o_l, w_p, s, out, stream=None):
    import torch
    n, _ = _sizes(p)
    dt = _io_dtype(p)
    _check(lib().salad_combine(
        ctypes.byref(p), _ptr(o_s, "o_s", n, torch.float32), _ptr(o_l, "o_l", n, torch.float32),
        _ptr(w_p, "w_p", p.head_dim ** 2, dt), _ptr(s, "s", p.batch, torch.float32),
        _ptr(out, "out", n, dt), _stream(stream)))


def salad_attn_forward(p: Problem, q, k, v, x, w_p, gate_w, gate_b: float, out, ws,
                       s_override=None, s_out=None, idx_out=None, lse_out=None, stream=None,
                       events=None):
    """The whole layer.  events: optional (begin, end) raw hipEvent_t handles
    (see :class:`HipEvents`), recorded around the sparse-attention kernel
    through salad_attn_forward_timed."""
    import torch
    n, _ = _sizes(p)
    dt = _io_dtype(p)
    C = p.n_heads * p.head_dim
    nidx = p.batch * p.n_heads * p.n_blocks * p.topk
    fn, extra = (lib().salad_attn_forward, ()) if events is None else \
        (lib().salad_attn_forward_timed, tuple(ctypes.c_void_p(e) for e in events))
    _check(fn(
        ctypes.byref(p), _ptr(q, "q", n, dt), _ptr(k, "k", n, dt), _ptr(v, "v", n, dt),
        _ptr(x, "x", p.batch * p.N * C, dt), _ptr(w_p, "w_p", p.w_p_numel, dt),
        _ptr(gate_w, "gate_w", C, dt), float(gate_b),
        _ptr(s_override, "s_override", p.batch, torch.float32), _ptr(out, "out", n, dt),
        _ptr(s_out, "s_out", p.batch, torch.float32), _ptr(idx_out, "idx_out", nidx, torch.int32),
        _ptr(lse_out, "lse_out", p.batch * p.n_heads * p.N, torch.float32),
        _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream), *extra))


def salad_output_projection(p: Problem, x, w_o, out, stream=None):
    """out [B, N, C] = x [B, N, C] @ w_o [C, C] (storage type of p)."""
    n, _ = _sizes(p)
    dt = _io_dtype(p)
    _check(lib().salad_output_projection(
        ctypes.byref(p), _ptr(x, "in", n, dt), _ptr(w_o, "w_o", p.C ** 2, dt), _ptr(out, "out", n, dt),
        _stream(stream)))


def salad_backward_workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().salad_backward_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def salad_attn_backward(p: Problem, q, k, v, x, w_p, gate_w, gate_b: float, dout, dq, dk, dv, dw_p, ws,
                        dx=None, dgate_w=None, dgate_b=None, ds=None, s_override=None, out_saved=None,
                        lse_saved=None, stream=None, events=None):
    """Gradients of sum(dout * salad_attn_forward(...)): dq, dk, dv [B,N,H,d]
    and dx [B,N,C] in bf16; dw_p [d,d], dgate_w [C], dgate_b [1], ds [B] in
    float32 (dx, dgate_w, dgate_b, ds optional).  out_saved / lse_saved: the
    forward's out and lse_out for the same inputs (skips the recompute).
    events: optional (begin, end) hipEvent_t handles recorded around the
    sparse-branch gradient kernels (salad_attn_backward_timed)."""
    import torch
    n, _ = _sizes(p)
    dt = _io_dtype(p)
    C = p.n_heads * p.head_dim
    fn, extra = (lib().salad_attn_backward, ()) if events is None else \
        (lib().salad_attn_backward_timed, tuple(ctypes.c_void_p(e) for e in events))
    _check(fn(
        ctypes.byref(p), _ptr(q, "q", n, dt), _ptr(k, "k", n, dt), _ptr(v, "v", n, dt),
        _ptr(x, "x", p.batch * p.N * C, dt), _ptr(w_p, "w_p", p.w_p_numel, dt),
        _ptr(gate_w, "gate_w", C, dt), float(gate_b),
        _ptr(s_override, "s_override", p.batch, torch.float32), _ptr(dout, "dout", n, dt),
        _ptr(out_saved, "out_saved", n, dt),
        _ptr(lse_saved, "lse_saved", p.batch * p.n_heads * p.N, torch.float32),
        _ptr(dq, "dq", n, dt), _ptr(dk, "dk", n, dt), _ptr(dv, "dv", n, dt),
        _ptr(dw_p, "dw_p", p.head_dim ** 2, torch.float32), _ptr(dx, "dx", p.batch * p.N * C, dt),
        _ptr(dgate_w, "dgate_w", C, torch.float32), _ptr(dgate_b, "dgate_b", 1, torch.float32),
        _ptr(ds, "ds", p.batch, torch.float32), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
        _stream(stream), *extra))


def salad_calibrate_workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().salad_calibrate_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def salad_window_calibrate(p: Problem, qw, kw, vw, radii, tau: float, err, choice, ws, stream=None):
    """Per-head window calibration: err (float64 [len(radii), B, H]) and
    choice (int32 [H]) on the device; radii is a host sequence of ints."""
    import torch
    n, _ = _sizes(p)
    dt = _io_dtype(p)
    r = (ctypes.c_int32 * len(radii))(*[int(x) for x in radii])
    _check(lib().salad_window_calibrate(
        ctypes.byref(p), _ptr(qw, "qw", n, dt), _ptr(kw, "kw", n, dt), _ptr(vw, "vw", n, dt),
        ctypes.cast(r, ctypes.c_void_p), len(radii), float(tau),
        _ptr(err, "err", len(radii) * p.batch * p.n_heads, torch.float64),
        _ptr(choice, "choice", p.n_heads, torch.int32), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
        _stream(stream)))


def calibrate_workspace(p: Problem, device="cuda"):
    import torch
    return torch.empty(max(salad_calibrate_workspace_size(p), 16), dtype=torch.uint8, device=device)


def backward_workspace(p: Problem, device="cuda"):
    """A device workspace of salad_backward_workspace_size(p) bytes."""
    import torch
    return torch.empty(max(salad_backward_workspace_size(p), 16), dtype=torch.uint8, device=device)


def workspace(p: Problem, device="cuda"):
    """A device workspace of salad_workspace_size(p) bytes (16-byte aligned)."""
    import torch
    return torch.empty(max(salad_workspace_size(p), 16), dtype=torch.uint8, device=device)


class HipEvents:
    """Timing events from the HIP runtime (plumbing for measurement, not part
    of the computation): ``count`` event pairs created up front, handed to
    the ``*_timed`` entry points as raw handles, read back after a sync."""

    def __init__(self, count: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        for _ in range(count):
            pair = []
            for _ in range(2):
                e = ctypes.c_void_p()
                if self._hip.hipEventCreate(ctypes.byref(e)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                pair.append(e.value)
            self.pairs.append(tuple(pair))

    def elapsed_ms(self, n: int):
        """Milliseconds between begin and end of the first n pairs (each end
        event waited for)."""
        out = []
        for b, e in self.pairs[:n]:
            if self._hip.hipEventSynchronize(ctypes.c_void_p(e)) != 0:
                raise RuntimeError("hipEventSynchronize failed")
            ms = ctypes.c_float(0.0)
            if self._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(b), ctypes.c_void_p(e)) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value)
        return out

    def close(self):
        for pair in self.pairs:
            for e in pair:
                self._hip.hipEventDestroy(ctypes.c_void_p(e))
        self.pairs = []
