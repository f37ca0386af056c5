"""Benchmark of the hybrid MuonAdamW optimizer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--serial]

One step is the whole hot path over the full parameter table of the
workload: clip norm over every trainable gradient, AdamW over the AdamW
group, momentum/normalise and 5 bf16 Newton-Schulz steps with the fused
update over the Muon group.  Inputs (parameters, gradients, states) are
synthetic, seeded, and resident in HBM before timing starts.

The headline steps run the AdamW group beside the Muon group (the library's
overlap_groups plan option; --serial turns it off).  After them, a roofline
pass times serial steps with HIP events that the library records on its own
stream at the phase boundaries, so the AdamW phase is exactly one k_adamw
launch and the Newton-Schulz phase its GEMM launches (two batches on two
streams, joined before the closing event); a plain device copy is timed as
the HBM rate reachable on this GPU.

Prints one JSON line: whole-step params/s (the metric's headline value),
step time, the serial pass's per-phase times, Newton-Schulz TFLOP/s and
AdamW GB/s against the MI355X peaks, the roofline of the dominant kernel,
and the CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import ctypes as C
import json
import math
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0       # dense MFMA
PEAK_FP32_TFLOPS = 157.3        # dense MFMA fp32
METRIC = "hybrid MuonAdamW step: params/s; NS TFLOP/s (MFMA %); AdamW HBM GB/s"


class HipEvents:
    """Timing events from the HIP runtime, recorded by the library itself on
    the stream its kernels run on."""

    def __init__(self, n: int):
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.ev = []
        for _ in range(n):
            e = C.c_void_p()
            rc = self.hip.hipEventCreate(C.byref(e))
            if rc != 0:
                raise RuntimeError("hipEventCreate failed (%d)" % rc)
            self.ev.append(e.value)

    def elapsed(self, a: int, b: int) -> float:
        ms = C.c_float()
        self.hip.hipEventSynchronize(C.c_void_p(self.ev[b]))
        rc = self.hip.hipEventElapsedTime(C.byref(ms), C.c_void_p(self.ev[a]), C.c_void_p(self.ev[b]))
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(C.c_void_p(e))


KERNEL_SOURCES = {
    "k_adamw": os.path.join(HERE, "muon_newton_schulz_02_amd", "csrc", "elementwise.hip"),
    "k_ns_*": os.path.join(HERE, "muon_newton_schulz_02_amd", "csrc", "ns_gemm.hip"),
}


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` (for "k_ns_*": per serial step of all
    Newton-Schulz launches) from the committed rocprofv3 summary (FETCH_SIZE
    + WRITE_SIZE, calibrated against a plain copy), or None when there is
    none or the kernel's source changed since it was taken."""
    import hashlib
    path = os.path.join(HERE, "profiles", "kernels_%s.md" % workload)
    if not os.path.exists(path):
        return None
    sha = hashlib.sha256(open(KERNEL_SOURCES[kernel], "rb").read()).hexdigest()[:16]
    for line in open(path):
        if not line.startswith("traffic:"):
            continue
        f = dict(kv.split("=", 1) for kv in line.split()[1:])
        if f.get("kernel") == kernel and f.get("workload") == workload:
            return float(f["bytes_per_launch"]) if f.get("source_sha256") == sha else None
    return None


def ns_flops(shapes, ns_steps: int) -> float:
    """Dense algorithmic flops of NS: per step and matrix (r <= c) the Gram
    X X^T (2 r^2 c), the square A A (2 r^3) and B X (2 r^2 c)."""
    tot = 0.0
    for m, n in shapes:
        r, c = min(m, n), max(m, n)
        tot += 4.0 * r * r * c + 2.0 * r ** 3
    return tot * ns_steps


def ns_executed_flops(shapes, ns_steps: int, ns_precision: str) -> float:
    """Flops the matrix cores execute for NS: both sides padded to 256, and
    the symmetric Gram and square results computed over their upper tiles
    only (mirrored on write), so this is below the dense count for r > 256
    and above it where padding dominates.  Tiles are 256 x 256, except for
    fp32 operands (fp32 NS, or fewer than 16 rows) when no fp32 matrix has
    more than 256 rows: the library then runs the Gram and square of those
    as 32 x 32 tiles (and the X update as 64 x 64 ones, full either way).
    bf16 matrices of at most 64 x 512 run in one workgroup each, on their
    sides rounded up to 32, every product in full."""
    f32 = [(min(m, n), max(m, n)) for m, n in shapes if ns_precision == "fp32" or min(m, n) < 16]
    small = all(-(-r // 256) * 256 <= 256 for r, _ in f32)
    tot = 0.0
    for m, n in shapes:
        r, c = min(m, n), max(m, n)
        if ns_precision == "bf16" and 16 <= r <= 64 and -(-c // 32) * 32 <= 512:
            R, C = -(-r // 32) * 32, -(-c // 32) * 32
            tot += 4.0 * R * R * C + 2.0 * R ** 3
            continue
        R, C = -(-r // 256) * 256, -(-c // 256) * 256
        t = 32 if (small and (ns_precision == "fp32" or r < 16)) else 256
        up = (R // t) * (R // t + 1) // 2 * float(t * t)
        tot += 2.0 * up * C + 2.0 * up * R + 2.0 * R * R * C
    return tot * ns_steps


def copy_bandwidth(torch, mib: int = 2048, reps: int = 5) -> float:
    """Bytes moved per second (read + write) by a plain device-to-device copy
    of `mib` MiB, timed with events: the HBM rate this GPU reaches for a
    read/write mix, next to the datasheet peak."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return 2.0 * n * 4 / (ms * 1e-3) / 1e9


def gemm_tflops(torch, dtype, n: int = 8192, reps: int = 10) -> float:
    """Dense n x n x n matrix product through torch (hipBLASLt), timed with
    events: the matrix-core rate a library GEMM reaches on this GPU, next to
    the datasheet peak."""
    a = torch.randn((n, n), device="cuda").to(dtype)
    b = torch.randn((n, n), device="cuda").to(dtype)
    c = torch.mm(a, b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.mm(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    return 2.0 * n ** 3 / (ms * 1e-3) / 1e12


def library_ns_ms(torch, shapes, ns_steps: int, coeffs, dtype, reps: int = 3) -> float:
    """The same Newton-Schulz iterations written as plain torch batched
    matrix products (hipBLASLt) over the same canonical shapes, one bmm
    batch per shape bucket, timed with events: a library implementation of
    the phase on identical work, for comparison only.  X X^T takes a
    contiguous copy of X^T (torch's batched bf16 product with a transposed
    right operand is avoided on this platform); operands are random and
    normalised, the arithmetic is not checked here."""
    a, b, c = (float(x) for x in coeffs)
    buckets = {}
    for m, n in shapes:
        r, cc = min(m, n), max(m, n)
        buckets[(r, cc)] = buckets.get((r, cc), 0) + 1
    xs = [torch.randn((cnt, r, cc), device="cuda").div_(math.sqrt(r * cc)).to(dtype)
          for (r, cc), cnt in buckets.items()]

    def one():
        for k, x in enumerate(xs):
            for _ in range(ns_steps):
                at = torch.bmm(x, x.transpose(1, 2).contiguous())
                bm = torch.bmm(at, at).mul_(c).add_(at, alpha=b)
                x = torch.bmm(bm, x).add_(x, alpha=a)
            xs[k] = x

    one()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        one()
    e1.record()
    torch.cuda.synchronize()
    del xs
    return e0.elapsed_time(e1) / reps


def percentile(xs, q: float) -> float:
    xs = sorted(xs)
    k = (len(xs) - 1) * q
    lo, hi = int(math.floor(k)), int(math.ceil(k))
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


def cpu_baseline(w, hp_overrides, budget_s: float = 12.0) -> dict:
    """The oracle, as it stands, on a bounded sample of the workload, scaled
    to the whole table's params/s:

      * Muon: per distinct canonical shape (rows <= cols), matrices are
        timed one by one (momentum, Newton-Schulz, update) until the shape's
        share of the budget is spent, then scaled by the shape's count; a
        shape whose dense Newton-Schulz cost exceeds 6 TFLOP is not run and
        takes the flop rate of the costliest shape that was;
      * AdamW: tensors in table order until a quarter of the budget is
        spent, scaled by element count;
      * clip norm: over the sampled gradients, scaled by element count.
    A table small enough to fit the budget is thereby timed whole."""
    import numpy as np
    import oracle as O
    import workloads as W

    hp = O.HParams()
    hp.param_storage = w.param_storage
    for k, v in hp_overrides.items():
        setattr(hp, k, v)
    names = w.names
    as_stored = O.bf16_round if w.param_storage == "bf16" else (lambda x: x)
    mode = W.mode_id(w)
    train = [i for i, p in enumerate(w.params) if p.trainable]
    groups = {i: O.route_one(names[i], w.params[i].shape, True, mode) for i in train}
    muon_by_shape = {}
    for i in train:
        if groups[i] == O.MUON:
            sh = tuple(sorted(w.params[i].shape))
            muon_by_shape.setdefault(sh, []).append(i)
    adam = [i for i in train if groups[i] == O.ADAMW]
    cap = 6e12

    def muon_time(i):
        p, g = as_stored(W.np_param(w, i)), as_stored(W.np_grad(w, 1, i))
        buf = W.np_momentum(w, i)
        m, n = w.params[i].shape
        s = O.lr_shape_scale(m, n, hp.moonlight_coefficient)
        t0 = time.perf_counter()
        O.muon_matrix_update(p, g, buf, 0.5, hp, s)
        return time.perf_counter() - t0

    est, notes, sample_params, sample_s = 0.0, [], 0, 0.0
    sampled_grads = []
    shapes = sorted(muon_by_shape, key=lambda sh: W.ns_cost(sh))
    per_shape = 0.5 * budget_s / max(1, len(shapes))
    rate = None    # flops per second of the costliest shape timed
    skipped = []
    for sh in shapes:
        idx = muon_by_shape[sh]
        if W.ns_cost(sh) > cap:
            skipped.append(sh)
            continue
        ts = []
        for i in idx:
            ts.append(muon_time(i))
            sample_params += w.params[i].numel
            if sum(ts) >= per_shape:
                break
        t_one = sum(ts) / len(ts)
        est += t_one * len(idx)
        sample_s += sum(ts)
        rate = W.ns_cost(sh) / t_one
        notes.append("%d of %d %dx%d (%.2f s each)" % (len(ts), len(idx), sh[0], sh[1], t_one))
    for sh in skipped:
        if rate is None:
            raise RuntimeError("no Muon shape cheap enough to time")
        t_one = W.ns_cost(sh) / rate
        est += t_one * len(muon_by_shape[sh])
        notes.append("%d %dx%d at the flop rate of the largest timed shape (%.1f s each)"
                     % (len(muon_by_shape[sh]), sh[0], sh[1], t_one))
    if adam:
        t_adam, n_done, k = 0.0, 0, 0
        for i in adam:
            p, g = as_stored(W.np_param(w, i)), as_stored(W.np_grad(w, 1, i))
            z = np.zeros(w.params[i].shape, np.float32)
            t0 = time.perf_counter()
            O.adamw_update(p, g, z, z, 1, 0.5, hp)
            t_adam += time.perf_counter() - t0
            n_done += w.params[i].numel
            sampled_grads.append(g)
            k += 1
            if t_adam >= 0.25 * budget_s:
                break
        n_adam = sum(w.params[i].numel for i in adam)
        est += t_adam * n_adam / n_done
        sample_s += t_adam
        sample_params += n_done
        notes.append("%d of %d AdamW tensors (%d of %d elements, %.2f s)"
                     % (k, len(adam), n_done, n_adam, t_adam))
    if not sampled_grads:
        sampled_grads = [as_stored(W.np_grad(w, 1, i)) for i in muon_by_shape[shapes[0]][:4]]
    t0 = time.perf_counter()
    O.global_grad_norm(sampled_grads)
    t_norm = time.perf_counter() - t0
    n_sampled = sum(g.size for g in sampled_grads)
    total_params = sum(w.params[i].numel for i in train)
    est += t_norm * total_params / n_sampled
    sample_s += t_norm
    notes.append("clip norm over %d sampled gradient elements (%.2f s)" % (n_sampled, t_norm))
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    blas = "unknown BLAS"
    try:
        from threadpoolctl import threadpool_info
        pools = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if pools:
            threads = int(pools[0].get("num_threads") or threads)
            blas = "%s %s, %d threads" % (pools[0].get("internal_api"), pools[0].get("version"),
                                          threads)
    except ImportError:
        pass
    return {
        "value": total_params / est,
        "unit": "params/s",
        "cores": min(cores, threads),
        "kind": "oracle",
        "sample": ("%s: %s; scaled to the whole table (%d params, est. %.1f s per step); NumPy "
                   "fp64, BLAS threads for matmuls, elementwise single-threaded"
                   % (w.name, "; ".join(notes), total_params, est)),
        "sample_seconds": sample_s,
        "step_seconds_estimated": est,
        "numpy": np.__version__,
        "blas": blas,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="vla_hybrid_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--serial", action="store_true",
                    help="time the groups one after the other (default: the AdamW group runs "
                         "beside the Muon group on its own stream)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the extra pass that times replays of one step captured in a "
                         "HIP graph (device step counter)")
    ap.add_argument("--roofline-steps", type=int, default=10,
                    help="serial steps timed after the headline ones, for per-kernel rooflines")
    ap.add_argument("--no-b2", action="store_true",
                    help="skip the ceiling probes (MFMA issue rate, LDS reads, HBM streams)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 times), to calibrate "
                         "the FETCH_SIZE / WRITE_SIZE counters against known bytes")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 3}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(every matrix is held whole on one device); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import muon_newton_schulz_02_amd as M

    M.load_library()  # fails loudly if the HIP library is not built
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    w = W.WORKLOADS[args.workload]()
    hp_over = W.hparams_for(w)
    hp = M.muon_adamw_default_hparams(ns_precision=w.ns_precision, **hp_over)
    table = list(zip(w.names, w.shapes, w.trainable))
    plan = M.muon_adamw_plan(table, mode=W.mode_id(w), overlap_groups=not args.serial,
                             param_dtype=w.param_storage)
    serial_plan = M.muon_adamw_plan(table, mode=W.mode_id(w), overlap_groups=False,
                                    param_dtype=w.param_storage)
    bf16_store = w.param_storage == "bf16"
    pdt = torch.bfloat16 if bf16_store else torch.float32
    n = len(table)
    groups = [M.muon_adamw_plan_entry(plan, i)["group"] for i in range(n)]
    params, grads = [None] * n, [None] * n
    state = M.State(n)
    print("[bench] allocating %s" % w.name, file=sys.stderr, flush=True)
    for i, spec in enumerate(w.params):
        if groups[i] == M.MA_GROUP_NONE:
            continue
        params[i] = W.torch_param(w, i, dev).to(pdt)
        grads[i] = W.torch_grad(w, 1, i, dev).to(pdt)
        if groups[i] == M.MA_GROUP_MUON:
            state.muon_momentum[i] = W.torch_momentum(w, i, dev)
        else:
            state.adam_m[i] = torch.zeros(spec.shape, dtype=torch.float32, device=dev)
            state.adam_v[i] = torch.zeros(spec.shape, dtype=torch.float32, device=dev)
    # one workspace serves both plans (their tile lists differ in length)
    ws = torch.empty(max(M.muon_adamw_workspace_size(plan, hp.ns_precision),
                         M.muon_adamw_workspace_size(serial_plan, hp.ns_precision)),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    muon_shapes = [w.params[i].shape for i in range(n) if groups[i] == M.MA_GROUP_MUON]
    n_muon = sum(w.params[i].numel for i in range(n) if groups[i] == M.MA_GROUP_MUON)
    n_adam = sum(w.params[i].numel for i in range(n) if groups[i] == M.MA_GROUP_ADAMW)
    n_train = n_muon + n_adam

    stream = torch.cuda.current_stream()
    K = 5  # MA_PROFILE_EVENTS
    R = max(args.roofline_steps, 1)
    evs = HipEvents(K * R)
    print("[bench] warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        M.muon_adamw_step(plan, params, grads, state, hp, ws, stream=stream)
    torch.cuda.synchronize()

    def one_step():
        M.muon_adamw_step(plan, params, grads, state, hp, ws, stream=stream)
    print("[bench] timing %d steps" % args.steps, file=sys.stderr, flush=True)
    # an event between steps on the caller's stream (the side stream joins
    # it before a step's work ends) gives the per-step distribution
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    marks[0].record(stream)
    for s in range(args.steps):
        one_step()
        marks[s + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    step_ms = [marks[s].elapsed_time(marks[s + 1]) for s in range(args.steps)]

    # The same step captured once in a HIP graph and replayed: every launch
    # of a step takes the same arguments with the step number on the device,
    # and an eager step has just uploaded the descriptor tables it reuses.
    graph_out = None
    if not args.no_graph:
        print("[bench] graph replay: %d steps" % args.steps, file=sys.stderr, flush=True)
        state.device_step = torch.full((1,), state.step, dtype=torch.int64, device=dev)
        M.muon_adamw_step(plan, params, grads, state, hp, ws, stream=stream)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            M.muon_adamw_step(plan, params, grads, state, hp, ws)
        graph.replay()
        torch.cuda.synchronize()
        gm = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        tg = time.perf_counter()
        gm[0].record(stream)
        for s in range(args.steps):
            graph.replay()
            gm[s + 1].record(stream)
        torch.cuda.synchronize()
        g_wall = (time.perf_counter() - tg) * 1e3 / args.steps
        g_ms = [gm[s].elapsed_time(gm[s + 1]) for s in range(args.steps)]
        graph_out = {"ms_per_step": g_wall, "value": n_train / (g_wall * 1e-3),
                     "step_ms_p10_p50_p90": [percentile(g_ms, q) for q in (0.1, 0.5, 0.9)]}
        del graph
        state.step = int(state.device_step.item())
        state.device_step = None

    # Per-kernel rooflines come from serial steps, where the library's phase
    # events bracket single kernels: [1] -> [2] is the one AdamW launch.
    print("[bench] roofline pass: %d serial steps" % R, file=sys.stderr, flush=True)
    M.muon_adamw_step(serial_plan, params, grads, state, hp, ws, stream=stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(R):
        M.muon_adamw_step_profiled(serial_plan, params, grads, state, hp, ws,
                                   evs.ev[K * s:K * s + K], stream=stream)
    torch.cuda.synchronize()
    serial_ms = (time.perf_counter() - t1) * 1e3 / R
    phases = {"clip_norm": [], "adamw": [], "muon_prep": [], "newton_schulz": [], "step": []}
    for s in range(R):
        b = K * s
        phases["clip_norm"].append(evs.elapsed(b, b + 1))
        phases["adamw"].append(evs.elapsed(b + 1, b + 2))
        phases["muon_prep"].append(evs.elapsed(b + 2, b + 3))
        phases["newton_schulz"].append(evs.elapsed(b + 3, b + 4))
        phases["step"].append(evs.elapsed(b, b + 4))
    evs.close()
    mean = {k: sum(v) / len(v) for k, v in phases.items()}
    b2 = None
    if not args.no_b2:
        print("[bench] ceiling probes (b2)", file=sys.stderr, flush=True)
        from muon_newton_schulz_02_amd import peaks
        b2 = peaks.measure_all(torch)
    copy_gbps = copy_bandwidth(torch)
    gemm = gemm_tflops(torch, torch.bfloat16 if w.ns_precision == "bf16" else torch.float32) \
        if n_muon > 0 else None
    flops = ns_flops(muon_shapes, hp.muon_ns_steps)
    lib_ms = (library_ns_ms(torch, muon_shapes, hp.muon_ns_steps, hp.ns_coeffs,
                            torch.bfloat16 if w.ns_precision == "bf16" else torch.float32)
              if n_muon > 0 else None)
    ns_peak = PEAK_BF16_TFLOPS if w.ns_precision == "bf16" else PEAK_FP32_TFLOPS
    ns_tflops = flops / (mean["newton_schulz"] * 1e-3) / 1e12 if mean["newton_schulz"] > 0 else 0.0
    ns_exec_tflops = (ns_executed_flops(muon_shapes, hp.muon_ns_steps, w.ns_precision) /
                      (mean["newton_schulz"] * 1e-3) / 1e12 if mean["newton_schulz"] > 0 else 0.0)
    # AdamW reads p, g, m, v and writes p, m, v: 28 B per element with fp32
    # parameters, 22 B with bf16 ones (m, v fp32 either way); the clip norm
    # reads every gradient once
    esz = 2.0 if bf16_store else 4.0
    adam_bytes = (3.0 * esz + 16.0) * n_adam
    norm_bytes = esz * n_train
    adam_gbps = adam_bytes / (mean["adamw"] * 1e-3) / 1e9 if mean["adamw"] > 0 else 0.0
    norm_gbps = norm_bytes / (mean["clip_norm"] * 1e-3) / 1e9 if mean["clip_norm"] > 0 else 0.0
    # the bf16 GEMMs copy 32 KB of operands into LDS per 256 x 256 x 32
    # product (4.19 M executed flops): 128 executed flops per staged byte
    ns_dma_gbps = (ns_exec_tflops * 1e3 / 128.0
                   if (n_muon > 0 and w.ns_precision == "bf16") else None)
    b2_mfma = (b2 or {}).get("mfma_bf16_tflops" if w.ns_precision == "bf16" else "mfma_fp32_tflops")
    b2_mix = (b2 or {}).get("hbm_adamw_mix_gbps")
    if n_adam > 0 and mean["adamw"] >= mean["newton_schulz"]:
        roofline = {"kernel": "k_adamw", "bound": "hbm", "achieved": adam_gbps,
                    "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": adam_gbps / PEAK_HBM_GBPS,
                    "traffic": measured_traffic("k_adamw", w.name),
                    "algorithmic_bytes": adam_bytes, "frac_of_copy": adam_gbps / copy_gbps,
                    "b2_peak": b2_mix, "frac_of_b2": adam_gbps / b2_mix if b2_mix else None}
    else:
        # achieved: the flops the matrix cores execute (the symmetric
        # products' upper tiles, padded; the MFMA counters agree), so frac
        # is the matrix-core utilisation and cannot pass 1; the dense
        # algorithmic rate is reported beside it
        roofline = {"kernel": "k_ns_* GEMMs (5 steps x 3 launches)", "bound": "mfma",
                    "achieved": ns_exec_tflops, "peak": ns_peak, "unit": "TFLOP/s",
                    "frac": ns_exec_tflops / ns_peak,
                    "traffic": measured_traffic("k_ns_*", w.name),  # bytes per serial step
                    "dense_tflops": ns_tflops, "dense_frac": ns_tflops / ns_peak,
                    "b2_peak": b2_mfma, "frac_of_b2": ns_exec_tflops / b2_mfma if b2_mfma else None}
    out = {
        "metric": METRIC,
        "value": n_train / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16+fp32" if (bf16_store or (n_muon > 0 and w.ns_precision == "bf16"))
                  else "fp32"),
        "data": "synthetic",
        "config": {"workload": w.name, "muon_params": n_muon, "adamw_params": n_adam,
                   "muon_matrices": len(muon_shapes), "ns_precision": w.ns_precision,
                   "ns_steps": hp.muon_ns_steps, "parallelism": "single GPU",
                   "param_storage": w.param_storage,
                   "launch": "eager (graph_replay: the same step replayed from a HIP graph)",
                   "optimizer": w.mode, "lr_schedule": hp_over.get("lr_schedule", "constant"),
                   "streams": ("one stream" if n_muon == 0 else
                               "newton-schulz batches over two streams" +
                               ("" if (args.serial or n_adam == 0) else
                                ", adamw beside them on a third"))},
        "step_ms_p10_p50_p90": [percentile(step_ms, q) for q in (0.1, 0.5, 0.9)],
        "step_ms_events": [round(x, 3) for x in step_ms],
        "graph_replay": graph_out,
        "serial_ms_per_step": serial_ms,
        "phase_ms": mean,
        "ns_tflops": ns_tflops,
        "ns_dense_frac": ns_tflops / ns_peak,
        "ns_executed_tflops": ns_exec_tflops,
        "ns_mfma_frac": ns_exec_tflops / ns_peak,
        "ns_mfma_frac_of_b2": ns_exec_tflops / b2_mfma if b2_mfma else None,
        "ns_lds_dma_gbps": ns_dma_gbps,
        "ns_lds_dma_frac_of_b2_l2": (ns_dma_gbps / b2["lds_dma_l2_gbps"]) if (b2 and ns_dma_gbps) else None,
        "ns_lds_dma_frac_of_b2_far": (ns_dma_gbps / b2["lds_dma_far_gbps"]) if (b2 and ns_dma_gbps) else None,
        "ns_library_ms": lib_ms,
        "ns_library_tflops": flops / (lib_ms * 1e-3) / 1e12 if lib_ms else None,
        "gemm_tflops_measured": gemm,
        "ns_frac_of_gemm": (ns_tflops / gemm) if gemm else None,
        "adamw_gbps": adam_gbps,
        "adamw_hbm_frac": adam_gbps / PEAK_HBM_GBPS,
        "adamw_frac_of_b2": adam_gbps / b2_mix if b2_mix else None,
        "clip_norm_gbps": norm_gbps,
        "clip_norm_frac_of_b2": (norm_gbps / b2["hbm_read_gbps"]) if b2 else None,
        "hbm_copy_gbps": copy_gbps,
        "b2": b2,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle on a sample)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, hp_over)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
