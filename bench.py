"""Throughput of the hybrid attention layer on one MI355X.

One step = one salad_attn_forward call (every stage of the layer: gate,
head-wise permutation, sparse attention, linear state and apply, combine)
over one batch of synthetic input already resident in HBM.

Default workload: 480p-like ST sliding window, N = 31,200 tokens (20 x 30 x
52 latent), 12 heads of 128, bf16, half the heads temporal, window radius
1601 (90 % sparsity).  value = effective TFLOP/s = 4 * d * (computed
query-key pairs) / layer time; ms_per_step is the layer time (ms/layer).

Also reported:
  roofline      the sparse-attention kernel's own launch time, read from
                HIP events the library records on its stream during the
                timed steps, against the bf16 dense MFMA peak;
  cpu_baseline  the fp64 oracle on whole heads of the same layer on this
                host's cores (one head per head kind, scaled to the layer);
  workloads     the other full-size workloads (480p Top-K, 720p window, CFG
                pair with RoPE) timed the same way in the same run.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms/layer and effective TFLOP/s of hybrid attention at N=31,200, 90% sparsity"
METRIC_BWD = "ms/layer and effective TFLOP/s of the hybrid attention backward at N=31,200, 90% sparsity"
MFMA_BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "attn_counters.json")


def pair_count(w) -> int:
    """Computed query-key pairs per layer (window heads: closed form; Top-K
    heads: every selected block's rows, which needs the selection)."""
    from sparse_linear_hybrid_st_amd.configs import window_pairs
    n_win = sum(1 for k in w.head_kinds if k != 2)
    return w.batch * n_win * window_pairs(w.N, w.window_radius)


def topk_pairs_from_idx(w, idx) -> int:
    import numpy as np
    nb = -(-w.N // w.block)
    rows = np.array([min(w.N, (b + 1) * w.block) - b * w.block for b in range(nb)], np.int64)
    tot = 0
    for h, k in enumerate(w.head_kinds):
        if k != 2:
            continue
        for b in range(w.batch):
            sel = idx[b, h]                                   # [nb, k]
            tot += int((rows[:, None] * rows[sel]).sum())
    return tot


def source_sha() -> str:
    src = os.path.join(ROOT, "sparse_linear_hybrid_st_amd", "csrc", "attn.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, flops_total: float, full: bool = False):
    """Time the fp64 oracle on whole heads of the layer on this host's cores.

    One whole (sample, head) per head kind present (every one of its N
    output rows, its linear state and, for Top-K heads, its selection),
    each run by oracle.parallel over one single-threaded process per core;
    the layer time is the sum over all heads of the time of a head of the
    same kind (the heads of one kind cost the same).  With full=True every
    head of every sample is run and nothing is extrapolated."""
    import numpy as np

    import oracle as O
    from oracle.parallel import warm, whole_head, workers
    from sparse_linear_hybrid_st_amd import inputs as I

    args = [inp[n].float().numpy() for n in ("q", "k", "v", "x")] + \
        [I.as_f64(inp[n]) for n in ("w_p", "gate_w")]
    procs = workers()
    warm(procs)  # the first start of the worker interpreters is not part of the oracle's time
    t0 = time.perf_counter()
    s_ref = [O.gate(args[3][b], args[5], inp["gate_b"]) for b in range(w.batch)]
    t_gate = time.perf_counter() - t0
    units = [(b, h) for b in range(w.batch) for h in range(w.n_heads)]
    if not full:
        first = {}
        for (b, h) in units:
            first.setdefault(int(w.head_kinds[h]), (b, h))
        run = sorted(first.values())
    else:
        run = units
    t_kind = {}
    spent = t_gate
    for (b, h) in run:
        t0 = time.perf_counter()
        whole_head(w, args, s_ref[b], b, h, procs)
        dt = time.perf_counter() - t0
        spent += dt
        t_kind.setdefault(int(w.head_kinds[h]), []).append(dt)
    if full:
        t_layer = spent
    else:
        t_layer = t_gate + sum(np.mean(t_kind[int(w.head_kinds[h])]) for (b, h) in units)
    kinds = ", ".join(f"{'spatial temporal Top-K'.split()[k]} head {np.mean(v):.1f} s"
                      for k, v in sorted(t_kind.items()))
    return {
        "value": flops_total / t_layer / 1e12, "unit": "TFLOP/s", "cores": int(procs),
        "kind": "oracle", "ms_per_layer": t_layer * 1e3,
        # wall time of the sample, and the core time it held (every process busy)
        "wall_seconds_spent": spent, "core_seconds_spent": t_gate + (spent - t_gate) * procs,
        "extrapolated": not full, "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(),
        "sample": ("the whole layer: every head of every sample, all rows" if full else
                   f"one whole head per head kind ({kinds}; every output row, the head's linear state "
                   f"and selection), scaled to the layer's {len(units)} (sample, head) pairs")
                  + f", fp64 numpy oracle on {procs} single-threaded processes",
    }


def calibrate_bench(args, w, inp, p):
    """One JSON line for salad_window_calibrate on this workload's inputs:
    time per call, and the dense pass's rate (4 d N^2 per head) as its
    roofline figure."""
    import numpy as np
    import torch

    import sparse_linear_hybrid_st_amd as S
    radii = [int(r) for r in args.calibrate.split(",")]
    qkv = [torch.empty_like(inp[n].cuda()) for n in ("q", "k", "v")]
    for n, dst in zip(("q", "k", "v"), qkv):
        S.salad_permute(p, 0, 0, inp[n].cuda(), dst)
    err = torch.empty((len(radii), w.batch, w.n_heads), dtype=torch.float64, device="cuda")
    choice = torch.empty(w.n_heads, dtype=torch.int32, device="cuda")
    ws = S.calibrate_workspace(p)

    def call():
        S.salad_window_calibrate(p, *qkv, radii, 2.0, err, choice, ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    pairs_dense = w.batch * w.n_heads * w.N * w.N
    pairs_win = sum(w.batch * w.n_heads * (w.N * (2 * min(r, w.N - 1) + 1) - min(r, w.N - 1) * (min(r, w.N - 1) + 1))
                    for r in radii)
    flops = 4.0 * w.head_dim * (pairs_dense + pairs_win)
    print(json.dumps({
        "metric": "window calibration: ms per call (dense attention + one window pass per radius)",
        "value": ms, "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.io_dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "radii": radii, "tau": 2.0,
                   "chosen": choice.cpu().tolist(),
                   "worst_error": err.max(dim=1).values.cpu().numpy().round(4).tolist()},
        "effective_tflops": flops / (ms * 1e-3) / 1e12}), flush=True)
    return 0


def stages_bench(args, w, inp, p):
    """--stages: each C-ABI stage entry point alone on the workload (inputs
    resident, warm), its average time over the timed calls from HIP events,
    and its algorithmic bytes (or flops) per call: the staged layer, stage by
    stage.  Prints one JSON line."""
    import torch

    import sparse_linear_hybrid_st_amd as S

    B, N, H, d = w.batch, w.N, w.n_heads, w.head_dim
    esz = 2 if w.io_dtype == "bf16" else 4
    dev = {n: inp[n].cuda() for n in ("q", "k", "v", "x", "w_p", "gate_w")}
    tensor = B * N * H * d                              # elements of Q, K, V or out
    qw, kw, vw = (torch.empty_like(dev["q"]) for _ in range(3))
    o_s = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    o_l = torch.empty_like(o_s)
    hs = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda")
    zs = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
    s = torch.empty(B, dtype=torch.float32, device="cuda")
    out = torch.empty_like(dev["q"])
    ws = S.workspace(p)
    topk = 2 in w.head_kinds
    idx = torch.zeros((B, H, p.n_blocks, w.topk), dtype=torch.int32, device="cuda") if topk else None
    n_topk = sum(1 for k in w.head_kinds if k == 2)
    rope = int(w.rope)
    stages = [
        ("a2 permute Q into working order" + (" with RoPE" if rope else ""),
         lambda: S.salad_permute(p, rope, 0, dev["q"], qw), "GB/s", 2.0 * tensor * esz),
        ("a2 permute K", lambda: S.salad_permute(p, rope, 0, dev["k"], kw), "GB/s", 2.0 * tensor * esz),
        ("a2 permute V", lambda: S.salad_permute(p, 0, 0, dev["v"], vw), "GB/s", 2.0 * tensor * esz),
    ]
    if topk:
        stages.append(("a3-a4 block means, scores, Top-K selection",
                       lambda: S.salad_block_select(p, qw, kw, idx, ws), "GB/s",
                       2.0 * B * n_topk * N * d * esz))
    pairs = pair_count(w)
    stages += [
        ("a6 linear state", lambda: S.salad_linear_state(p, kw, vw, hs, zs, ws), "GB/s", 2.0 * tensor * esz),
        ("a8 gate", lambda: S.salad_gate(p, dev["x"], dev["gate_w"], inp["gate_b"], s, ws), "GB/s",
         1.0 * tensor * esz),
    ]
    results = []

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for name, fn, unit, amount in stages:
        ms = timed(fn, args.steps)
        results.append({"stage": name, "ms": ms, "unit": unit, "achieved": amount / (ms * 1e-3) / 1e9,
                        "frac_of_peak": amount / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS})
    # a5 needs the selection (made above) for Top-K heads; the window pairs
    # are counted in closed form, the Top-K pairs from the selection
    if topk:
        pairs += topk_pairs_from_idx(w, idx.cpu().numpy())
    ms = timed(lambda: S.salad_sparse_attn(p, qw, kw, vw, idx, o_s), args.steps)
    results.append({"stage": "a5 sparse attention (staged: fp32 O_s in working order)", "ms": ms,
                    "unit": "TFLOP/s", "achieved": 4.0 * d * pairs / (ms * 1e-3) / 1e12,
                    "frac_of_peak": 4.0 * d * pairs / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS})
    for name, fn, amount in (
            ("a7 linear apply (fp32 O_l)", lambda: S.salad_linear_apply(p, qw, hs, zs, o_l),
             1.0 * tensor * esz + 4.0 * tensor),
            ("a9 combine + inverse permutation", lambda: S.salad_combine(p, o_s, o_l, dev["w_p"], s, out),
             8.0 * tensor + 1.0 * tensor * esz)):
        ms = timed(fn, args.steps)
        results.append({"stage": name, "ms": ms, "unit": "GB/s", "achieved": amount / (ms * 1e-3) / 1e9,
                        "frac_of_peak": amount / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS})
    total = sum(r["ms"] for r in results)
    print(json.dumps({
        "metric": "per-stage ms of the staged layer (each C-ABI stage entry point alone)",
        "value": total, "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": 2,
        "ms_per_step": total, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.io_dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "bytes": "algorithmic: each stage's compulsory reads and writes"},
        "stages": results}), flush=True)
    return 0


def measure_forward(w, steps: int, warmup: int) -> dict:
    """One full-size forward workload in this process: inputs resident, one
    forward, warm-up, then ``steps`` timed layer calls (wall clock around
    them, and the library's HIP events around the attention kernel)."""
    import torch

    import sparse_linear_hybrid_st_amd as S
    from sparse_linear_hybrid_st_amd import inputs as I

    t0 = time.perf_counter()
    inp = I.make_inputs(w)
    p = S.problem_from_workload(w)
    dev = {n: inp[n].cuda() for n in ("q", "k", "v", "x", "w_p", "gate_w")}
    del inp
    out = torch.empty_like(dev["q"])
    s_out = torch.empty(w.batch, dtype=torch.float32, device="cuda")
    idx = torch.zeros((w.batch, w.n_heads, p.n_blocks, w.topk), dtype=torch.int32, device="cuda")
    ws = S.workspace(p)
    print(f"[bench] {w.name}: inputs ready in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    def fwd(events=None):
        S.salad_attn_forward(p, dev["q"], dev["k"], dev["v"], dev["x"], dev["w_p"], dev["gate_w"], 0.0,
                             out, ws, s_out=s_out, idx_out=idx, events=events)

    fwd()
    for _ in range(warmup):
        fwd()
    torch.cuda.synchronize()
    pairs = pair_count(w)
    if 2 in w.head_kinds:
        pairs += topk_pairs_from_idx(w, idx.cpu().numpy())
    flops = 4.0 * w.head_dim * pairs
    events = S.HipEvents(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fwd(events=events.pairs[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    attn = events.elapsed_ms(steps)
    events.close()
    attn_ms = sum(attn) / len(attn)
    del dev, out, ws
    torch.cuda.empty_cache()
    return {"workload": w.name, "description": w.description, "ms_per_layer": ms,
            "effective_tflops": flops / (ms * 1e-3) / 1e12, "computed_pairs": pairs,
            "attention_kernel_ms": attn_ms,
            "attention_frac_of_mfma_peak": flops / (attn_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "steps": steps, "warmup": warmup}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="480p-stswa-h12")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="CPU baseline over every head of the layer (minutes) instead of one whole "
                         "head per head kind")
    ap.add_argument("--branch-drop-tau", type=float, default=0.0,
                    help="post-tuning branch dropping threshold (samples whose gate value is "
                         "below it keep only the sparse branch); 0 never drops")
    ap.add_argument("--proj", choices=("head", "full"), default="head",
                    help="static projection W_p: one [d, d] matrix per head (default) or one "
                         "[C, C] matrix over each token's concatenated heads (a GEMM after the "
                         "attention kernel)")
    ap.add_argument("--backward", action="store_true",
                    help="time salad_attn_backward (gradients of Q, K, V, X, W_p and the gate "
                         "for a random output gradient) instead of the forward")
    ap.add_argument("--recompute", action="store_true",
                    help="with --backward: do not hand the forward's output and row normalisers to "
                         "the backward (it then recomputes the forward's sparse branch)")
    ap.add_argument("--calibrate", default=None, metavar="R1,R2,...",
                    help="time salad_window_calibrate (dense attention plus one window pass per "
                         "radius in this comma-separated list) instead of the forward")
    ap.add_argument("--stages", action="store_true",
                    help="time each C-ABI stage entry point alone (the staged layer) instead of the "
                         "fused forward")
    ap.add_argument("--cold-runs", type=int, default=20,
                    help="forward only: after the timed steps, this many more layer calls, each after "
                         "writing a 512 MiB buffer (L2 and MALL flushed), timed one by one; median and "
                         "min reported as cold_cache (0: skip)")
    ap.add_argument("--workloads", default="480p-topk-h40,720p-stswa-h40,480p-cfg-rope-mixed-h40",
                    help="plain forward runs only: the other full-size workloads timed after the "
                         "headline one in the same run (comma-separated names; 'none' to skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a "
                         "known-size reference for the HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the layer shards by (sample, head) with no communication, so a multi-GPU figure "
              "is N independent single-GPU layers; it is not measured here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_linear_hybrid_st_amd as S
    from sparse_linear_hybrid_st_amd import configs as C
    from sparse_linear_hybrid_st_amd import inputs as I

    w = C.all_workloads()[args.workload]
    print(f"[bench] workload {w.name}: {w.description}", file=sys.stderr, flush=True)
    inp = I.make_inputs(w, proj=args.proj)
    p = S.problem_from_workload(w, branch_drop_tau=args.branch_drop_tau, proj=args.proj)
    dev = {n: inp[n].cuda() for n in ("q", "k", "v", "x", "w_p", "gate_w")}
    out = torch.empty_like(dev["q"])
    s_out = torch.empty(w.batch, dtype=torch.float32, device="cuda")
    idx = torch.zeros((w.batch, w.n_heads, p.n_blocks, w.topk), dtype=torch.int32, device="cuda")
    ws = S.workspace(p)

    if args.calibrate:
        sys.exit(calibrate_bench(args, w, inp, p))
    if args.stages:
        sys.exit(stages_bench(args, w, inp, p))

    def fwd(events=None):
        S.salad_attn_forward(p, dev["q"], dev["k"], dev["v"], dev["x"], dev["w_p"], dev["gate_w"],
                             inp["gate_b"], out, ws, s_out=s_out, idx_out=idx, events=events)

    step = fwd
    if args.backward:
        if args.proj != "head":
            sys.exit("--backward supports the per-head projection only")
        g_out = I.to_storage(np.random.default_rng(w.seed + 77).standard_normal(
            (w.batch, w.N, w.n_heads, w.head_dim), dtype=np.float32), w.io_dtype).cuda()
        grads = {n: torch.empty_like(dev["q"]) for n in ("dq", "dk", "dv")}
        dx = torch.empty_like(dev["x"])
        dwp = torch.empty((w.head_dim, w.head_dim), dtype=torch.float32, device="cuda")
        dgw = torch.empty(w.n_heads * w.head_dim, dtype=torch.float32, device="cuda")
        dgb = torch.empty(1, dtype=torch.float32, device="cuda")
        bws = S.backward_workspace(p)
        lse = None if args.recompute else torch.empty((w.batch, w.n_heads, w.N), dtype=torch.float32,
                                                      device="cuda")

        def step(events=None):
            S.salad_attn_backward(p, dev["q"], dev["k"], dev["v"], dev["x"], dev["w_p"], dev["gate_w"],
                                  inp["gate_b"], g_out, grads["dq"], grads["dk"], grads["dv"], dwp, bws,
                                  dx=dx, dgate_w=dgw, dgate_b=dgb,
                                  out_saved=None if args.recompute else out, lse_saved=lse, events=events)

    # the forward once (its output and, for the backward, row normalisers)
    S.salad_attn_forward(p, dev["q"], dev["k"], dev["v"], dev["x"], dev["w_p"], dev["gate_w"],
                         inp["gate_b"], out, ws, s_out=s_out, idx_out=idx,
                         lse_out=lse if args.backward else None)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    pairs = pair_count(w)
    if 2 in w.head_kinds:
        pairs += topk_pairs_from_idx(w, idx.cpu().numpy())
    # forward: QK^T and PV, 2 flops per multiply-add; backward: QK^T, dP,
    # dV, dK and dQ (the algorithmic count, not counting recomputation)
    flops = (10.0 if args.backward else 4.0) * w.head_dim * pairs

    # HIP events the library records on its stream around the sparse-branch
    # kernel(s) of every timed step (the *_timed entry points)
    events = S.HipEvents(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events=events.pairs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_times = events.elapsed_ms(args.steps)
    events.close()
    calls = len(attn_times)
    ms = wall * 1e3 / args.steps
    attn_avg = sum(attn_times) / max(calls, 1)
    achieved = flops / (attn_avg * 1e-3) / 1e12

    # measured ceilings on this GPU, the second denominator of the fractions:
    # a large square bf16 GEMM through torch (hipBLASLt) and a 1 GiB device copy
    ceilings = None
    if not args.backward:
        a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
        bm = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.matmul(a, bm)
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record()
        for _ in range(10):
            torch.matmul(a, bm)
        e1.record()
        for _ in range(10):
            dst.copy_(src)
        e2.record()
        torch.cuda.synchronize()
        gemm_tf = 2.0 * 8192 ** 3 / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e12
        copy_gbs = 2.0 * (1 << 30) / (e1.elapsed_time(e2) / 10 * 1e-3) / 1e9
        ceilings = {"gemm_bf16_8192_tflops": gemm_tf, "copy_1gib_gbs": copy_gbs}
        del a, bm, src, dst

    cold = None
    if not args.backward and args.cold_runs > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        times = []
        for _ in range(args.cold_runs):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        del flush
        times.sort()
        cold = {"median_ms": times[len(times) // 2], "min_ms": times[0], "runs": len(times),
                "flush_mib": 512,
                "median_effective_tflops": flops / (times[len(times) // 2] * 1e-3) / 1e12}

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    traffic = None
    if os.path.exists(PROFILE_COUNTERS):
        c = json.load(open(PROFILE_COUNTERS))
        if c.get("source_sha") == source_sha() and c.get("workload") == w.name:
            traffic = c.get("traffic_bytes_per_launch")

    rec = {
        "metric": METRIC_BWD if args.backward else METRIC, "value": flops / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "ms_per_layer": ms,
        "config": {"workload": w.name, "batch": w.batch, "tokens": w.N, "grid": list(w.grid),
                   "heads": w.n_heads, "head_dim": w.head_dim,
                   "head_kinds": "".join("STK"[k] for k in w.head_kinds),
                   "window_radius": w.window_radius, "block": w.block, "topk": w.topk,
                   "rope": w.rope, "proj": args.proj,
                   "pass": ("backward (recomputing the forward's sparse branch)" if args.recompute else
                            "backward (given the forward's output and row normalisers)")
                   if args.backward else "forward",
                   "projection_gemm_flop": (2.0 * w.batch * w.N * (w.n_heads * w.head_dim) ** 2
                                            if args.proj == "full" else None),
                   "branch_drop_tau": args.branch_drop_tau,
                   "samples_dropped": int((s_out.cpu() < args.branch_drop_tau).sum()),
                   "computed_pairs": pairs,
                   "density": pairs / (w.batch * w.n_heads * w.N * w.N)},
        "roofline": {"bound": "mfma",
                     "kernel": ("sparse-branch gradients (attn_bwd_dq_kernel + attn_bwd_dkv_kernel)"
                                if args.backward else "sparse attention (attn_bf16_kernel)"),
                     "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic,
                     "avg_launch_ms": attn_avg, "launches": calls},
    }
    if cold is not None:
        rec["cold_cache"] = cold
    if ceilings is not None:
        rec["ceilings"] = ceilings
        rec["roofline"]["frac_of_measured_gemm"] = achieved / ceilings["gemm_bf16_8192_tflops"]
    if w.io_dtype != "bf16":
        rec["dtype"] = "f32"
    if traffic is not None and args.backward:
        traffic = None          # the stored counters are the forward kernel's
    rec["roofline"]["traffic"] = traffic
    if args.backward:
        rec["cpu_baseline"] = None  # the oracle's backward is timed in the test suite, not here
    elif not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w, inp, flops, args.cpu_full) if args.proj == "head" else None
    if (not args.backward and args.proj == "head" and args.branch_drop_tau == 0.0
            and args.workloads != "none"):
        names = [n for n in args.workloads.split(",") if n and n != w.name]
        del dev, out, ws
        torch.cuda.empty_cache()
        rec["workloads"] = [measure_forward(C.all_workloads()[n], args.steps, args.warmup) for n in names]
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
