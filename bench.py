#!/usr/bin/env python3
"""Benchmark of the chunked fused linear-cross-entropy path on one MI355X.

Default workload (the large-vocabulary head): N=8192 rows, D=4096, V=128256,
bf16 inputs with fp32 accumulation, no bias, Zipf(1.1) targets with 410 rows
set to ignore_index, reduction='mean', 2048-row chunks, grad_W accumulated
in fp32 ("accurate").  One step = one lce_forward_backward: loss, grad_X,
grad_W, with the inputs already resident in HBM.

Prints one JSON line: tokens/s (value), TFLOP/s counting 6*N*V*D, the
roofline of the dominant kernel (its average launch duration measured with
HIP events recorded on the library's stream during the timed steps), and the
fp64 CPU oracle timed on a bounded row sample of the same workload.  The
default run adds three records to the same line:
  per_chunk  the same workload on the per-chunk path (group_rows = 2048: each
             chunk's dL consumed by both gradient GEMMs right after it is
             formed, grad_W carried across chunks in an fp32 accumulator);
  ce         the standalone in-place softmax cross-entropy on fp32 logits
             [16384, 131072] (GB/s against 8 TB/s);
  copy       a plain 1 GiB device-to-device copy in the same process, the
             achievable read + write bandwidth.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused LCE fwd+bwd tokens/sec and TFLOP/s (6NVD) at N=8192,D=4096,V=128256 bf16"
PEAK_16BIT_TFLOPS = 2500.0     # MI355X dense bf16 / fp16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "linear_cross_entropy_chunk_amd", "csrc", f)
                  for f in ("lce_gemm.hip", "lce_rowops.hip", "lce_kernels.h", "lce_device.h")]


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(workload, {}).get(kernel)
    if not entry or entry.get("source_sha") != kernel_source_sha():
        return None
    return entry.get("bytes_per_launch")


def counted_plan(args, label: str, cfg) -> bool:
    """Whether this run launches the kernels the committed counters were taken
    on: the workload's own dtype and the default plan (accurate, the default
    chunk and group sizes, forward and backward).  Other plans change the
    launches' shapes, so their traffic is not the counted one."""
    return (label == cfg.name and args.acc_policy == "accurate" and args.group_rows == 0
            and args.chunk_rows is None and not args.forward_only)


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return os.cpu_count() or 1


def host_cpu() -> dict:
    """The host's logical CPU count (all of them, and those this process may
    run on) and the CPU model, for the CPU baseline's record."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"nproc": os.cpu_count(), "nproc_usable": usable, "cpu_model": model}


def cpu_baseline_lce(inputs: dict, rows: int, label: str) -> dict:
    """The fp64 oracle as it stands on the first `rows` rows (full W)."""
    import numpy as np

    import oracle
    X = inputs["X"][:rows]
    t = inputs["t"][:rows]
    t0 = time.perf_counter()
    r = oracle.linear_cross_entropy(X, inputs["W"], inputs["b"], t, reduction="mean")
    dt = time.perf_counter() - t0
    assert np.isfinite(r["loss"])
    # `cores` is the number of threads the oracle ran on: numpy's matmul
    # (the oracle's only library primitive, and nearly all of its time) uses
    # the BLAS thread pool; its elementwise passes use one core.
    return {"value": rows / dt, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            **host_cpu(),
            "sample": f"rows 0-{rows - 1} of the {label} workload with the full W: "
                      f"loss, grad_X, grad_W, grad_b in float64 ({dt:.1f} s)"}


GEMM_MASK = (1 << 1) | (1 << 4) | (1 << 7)          # logits, gemm_x, gemm_w


def time_steps(op, io, steps: int, warmup: int, breakdown: bool = False):
    """Run `warmup` untimed steps, then time `steps` steps between
    synchronisations with events on torch's current stream (the library's
    stream), and the selected kernel classes with the library's timing hook.
    Returns (ms per step, per-class timing, wall seconds)."""
    import torch

    from linear_cross_entropy_chunk_amd import _binding as B
    for _ in range(warmup):
        op.run_io(io)
    torch.cuda.synchronize()
    mask = (1 << B.LCE_K_COUNT) - 1 if breakdown else GEMM_MASK
    B.lce_timing_enable(op.handle, mask)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        op.run_io(io)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    timing = B.lce_timing_read(op.handle)
    B.lce_timing_enable(op.handle, 0)
    return start.elapsed_time(end) / steps, timing, wall


def bench_per_chunk(args, cfg, X, W, t, b, group_rows: int) -> dict:
    """The same workload on the per-chunk path: group_rows rows of dL per
    grad_W GEMM (one chunk when it equals the chunk rows), grad_W carried
    across chunks in an fp32 accumulator."""
    import torch

    from linear_cross_entropy_chunk_amd import LinearCrossEntropy
    op = LinearCrossEntropy(cfg.N, cfg.D, cfg.V, X.dtype, bias=b is not None,
                            reduction=cfg.reduction, chunk_rows=cfg.chunk_rows,
                            acc_policy="accurate", grad_x=True, grad_w=True,
                            grad_b=b is not None, device=X.device, group_rows=group_rows)
    out = op.make_outputs(grads=True)
    io = op.make_io(X, W, t, b, out=out)
    ms_step, timing, _ = time_steps(op, io, args.steps, args.warmup)
    loss = float(out["loss"].cpu()[0])
    N, D, V = cfg.N, cfg.D, cfg.V
    rec = {"group_rows": group_rows, "chunk_rows": op.chunk_rows, "ms_per_step": ms_step,
           "tokens_per_s": N / (ms_step / 1e3),
           "tflops": 6.0 * N * V * D / (ms_step / 1e3) / 1e12,
           "workspace_bytes": op.ws_bytes, "loss": loss,
           "kernels": {k: round(ms / args.steps, 4) for k, (ms, n) in timing.items() if n},
           "launches_per_step": {k: n // args.steps for k, (ms, n) in timing.items() if n}}
    rec["frac_of_peak"] = rec["tflops"] / PEAK_16BIT_TFLOPS
    log(f"per-chunk path (group_rows={group_rows}): {ms_step:.3f} ms/step, "
        f"{rec['tflops']:.0f} TFLOP/s, workspace {op.ws_bytes / 2**30:.2f} GiB, "
        f"kernels {rec['kernels']}")
    del op, out, io
    torch.cuda.empty_cache()
    return rec


def bench_lce(args) -> dict:
    import numpy as np
    import torch

    import lce_inputs as li
    from linear_cross_entropy_chunk_amd import LinearCrossEntropy
    from linear_cross_entropy_chunk_amd import _binding as B

    cfg = li.LCE_CONFIGS[args.workload]
    label = cfg.name
    if args.dtype is not None and args.dtype != cfg.dtype:
        # the same workload with its inputs rounded to another input type
        cfg = dataclasses.replace(cfg, dtype=args.dtype)
        label = f"{cfg.name} with {cfg.dtype} inputs"
    chunk = cfg.chunk_rows if args.chunk_rows is None else args.chunk_rows
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[cfg.dtype]
    log(f"generating {cfg.name}: N={cfg.N} D={cfg.D} V={cfg.V}")
    inputs = li.lce_inputs(cfg)
    dev = torch.device("cuda", 0)
    X = torch.from_numpy(inputs["X"]).to(dev).to(dt)
    W = torch.from_numpy(inputs["W"]).to(dev).to(dt)
    b = None if inputs["b"] is None else torch.from_numpy(inputs["b"]).to(dev).to(dt)
    t = torch.from_numpy(inputs["t"]).to(dev)
    if args.forward_only and cfg.reduction != "none":
        raise SystemExit("--forward-only applies to the reduction='none' workload")
    # 'none' with --forward-only: the loss-only forward (logits, row statistics,
    # per-row loss; 2*N*V*D flops); otherwise the call forms the gradients
    u = None if not cfg.upstream or args.forward_only else \
        torch.from_numpy(inputs["u"]).to(dev)
    op = LinearCrossEntropy(cfg.N, cfg.D, cfg.V, dt, bias=b is not None,
                            reduction=cfg.reduction, chunk_rows=chunk,
                            acc_policy=args.acc_policy, grad_x=True, grad_w=True,
                            grad_b=b is not None, device=dev, group_rows=args.group_rows)
    out = op.make_outputs(grads=True)
    io = op.make_io(X, W, t, b, out=out, grad_output=u)
    log(f"chunk_rows={op.chunk_rows} chunks={op.n_chunks} group_rows={args.group_rows} "
        f"workspace={op.ws_bytes / 2**30:.2f} GiB")
    ms_step, timing, wall = time_steps(op, io, args.steps, args.warmup, args.breakdown)
    loss = float(out["loss"].cpu()[0]) if cfg.reduction != "none" else float("nan")
    log(f"{ms_step:.3f} ms/step (wall {1e3 * wall / args.steps:.3f}), loss {loss:.6f}")
    eager_ms = ms_step
    if args.graph:
        # One call captured into a HIP graph and replayed: the same kernels
        # without the host's per-launch cost (the per-kernel figures and the
        # roofline come from the eager steps above).
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            op.run_io(io)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(args.steps):
            graph.replay()
        end.record()
        torch.cuda.synchronize()
        ms_step = start.elapsed_time(end) / args.steps
        log(f"graph replay: {ms_step:.3f} ms/step (eager {eager_ms:.3f})")

    N, D, V = cfg.N, cfg.D, cfg.V
    op_chunk_rows = op.chunk_rows
    per_kernel = {}
    for name, (ms, n) in timing.items():
        if n:
            per_kernel[name] = {"ms_total": ms, "launches": n, "avg_ms": ms / n}
    for name, k in per_kernel.items():
        log(f"  {name:10s} {k['launches']:5d} launches  avg {k['avg_ms']:.3f} ms  "
            f"total/step {k['ms_total'] / args.steps:.3f} ms")
    dom = max((n for n in ("logits", "gemm_x", "gemm_w") if n in per_kernel),
              key=lambda n: per_kernel[n]["ms_total"])
    avg_s = per_kernel[dom]["avg_ms"] / 1e3
    # Each GEMM class does 2*N*V*D flops per step: logits and grad_X one chunk
    # of rows per launch (2*c*V*D), grad_W one group of chunks per launch
    # (2*c*group*V*D).  Per launch that is the step's flops over the launches
    # per step (an average when the last chunk is ragged).
    launches_per_step = per_kernel[dom]["launches"] / args.steps
    flops_per_launch = 2.0 * N * V * D / launches_per_step
    achieved = flops_per_launch / avg_s / 1e12
    peak = PEAK_F32_TFLOPS if cfg.dtype == "f32" else PEAK_16BIT_TFLOPS
    tokens_s = N / (ms_step / 1e3)
    flop_factor = 2.0 if args.forward_only else 6.0     # 2NVD forward only, 6NVD with grads
    tflops = flop_factor * N * V * D / (ms_step / 1e3) / 1e12
    result = {
        "metric": METRIC, "value": tokens_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic (seeded numpy, the workload's distributions)",
        "config": {"workload": f"{label} N={N} D={D} V={V} chunk_rows={op.chunk_rows} "
                               f"reduction={cfg.reduction} acc_fp32 {args.acc_policy}",
                   "N": N, "D": D, "V": V, "chunk_rows": op.chunk_rows,
                   "acc_policy": args.acc_policy, "parallelism": "single GPU"},
        "tflops": tflops,
        "flops_counted": f"{int(flop_factor)}NVD",
        "frac_of_peak": tflops / peak,
        "workspace_bytes": op.ws_bytes,
        "group_rows": args.group_rows,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": load_traffic(dom, cfg.name) if counted_plan(args, label, cfg)
                                else None,
                     "avg_launch_ms": per_kernel[dom]["avg_ms"],
                     "flops_per_launch": flops_per_launch},
        "kernels": {k: round(v["ms_total"] / args.steps, 4) for k, v in per_kernel.items()},
        # every GEMM class does 2*N*V*D flops per step (grad_W's class includes
        # its K-split tail launch), so its rate is those flops over its time
        "kernel_tflops": {k: round(2.0 * N * V * D / (per_kernel[k]["ms_total"] / args.steps / 1e3)
                                   / 1e12, 1)
                          for k in ("logits", "gemm_x", "gemm_w") if k in per_kernel},
    }
    result["kernel_frac"] = {k: round(v / peak, 4) for k, v in result["kernel_tflops"].items()}
    if args.graph:
        result["graph"] = True
        result["eager_ms_per_step"] = eager_ms
    if args.per_chunk and args.workload == "large-vocab-bf16" and cfg.dtype != "f32" \
            and args.group_rows == 0 and args.acc_policy == "accurate":
        del op, out, io
        torch.cuda.empty_cache()
        result["per_chunk"] = bench_per_chunk(args, cfg, X, W, t, b, op_chunk_rows)
    if not args.no_cpu_baseline:
        rows = args.cpu_rows
        log(f"cpu baseline: oracle on {rows} rows")
        result["cpu_baseline"] = cpu_baseline_lce(inputs, rows, label)
        log(f"cpu baseline {result['cpu_baseline']['value']:.1f} tokens/s")
    return result


def time_ce(steps: int, warmup: int):
    """The standalone in-place CE on the [16384, 131072] fp32 workload:
    (config, inputs, ms per call, GB/s, loss).  Each call overwrites the
    logits, so they are restored before each call; only the in-place CE call
    is inside the events."""
    import torch

    import lce_inputs as li
    from linear_cross_entropy_chunk_amd import CrossEntropyInplace

    cfg = li.CE_F32
    log(f"generating {cfg.name}: N={cfg.N} V={cfg.V}")
    inputs = li.ce_inputs(cfg)
    dev = torch.device("cuda", 0)
    pristine = torch.from_numpy(inputs["logits"]).to(dev)
    z = torch.empty_like(pristine)
    t = torch.from_numpy(inputs["t"]).to(dev)
    op = CrossEntropyInplace(cfg.N, cfg.V, reduction=cfg.reduction, device=dev)
    for _ in range(warmup):
        z.copy_(pristine)
        op(z, t)
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        z.copy_(pristine)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        op(z, t)
        e.record()
        times.append((s, e))
    torch.cuda.synchronize()
    ms = [s.elapsed_time(e) for s, e in times]
    ms_step = sum(ms) / len(ms)
    nbytes = 2.0 * cfg.N * cfg.V * 4          # logits read once, gradient written once
    gbs = nbytes / (ms_step / 1e3) / 1e9
    loss = float(op.loss.cpu()[0])
    log(f"standalone CE: {ms_step:.3f} ms/call, {gbs:.0f} GB/s, loss {loss:.6f}")
    del pristine, z, t, op
    torch.cuda.empty_cache()
    return cfg, inputs, ms_step, gbs, loss


def ce_record(args) -> dict:
    """The standalone CE as a record of the default line, with the plain copy
    measured in the same process as the achievable-bandwidth yardstick."""
    cfg, _, ms_step, gbs, loss = time_ce(args.steps, args.warmup)
    copy = copy_calibration()
    log(f"copy: {copy['gbs_read_plus_write']:.0f} GB/s (read + write)")
    return {"workload": f"{cfg.name} N={cfg.N} V={cfg.V} reduction={cfg.reduction}, "
                        "gradient written over the logits",
            "kernel": "ce_rows", "ms_per_call": ms_step, "bytes_per_call": 2 * cfg.N * cfg.V * 4,
            "gbs": gbs, "peak_gbs": PEAK_HBM_GBS, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS,
            "frac_of_copy": gbs / copy["gbs_read_plus_write"], "loss": loss,
            "steps": args.steps, "warmup": args.warmup, "copy": copy}


def bench_ce(args) -> dict:
    cfg, inputs, ms_step, gbs, loss = time_ce(args.steps, args.warmup)
    result = {
        "metric": "standalone in-place softmax CE GB/s (2*N*V*4 bytes) at N=16384,V=131072 fp32",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded numpy N(0,1) logits)",
        "config": {"workload": f"{cfg.name} N={cfg.N} V={cfg.V} reduction={cfg.reduction}"},
        "roofline": {"kernel": "ce_rows", "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                     "traffic": load_traffic("ce_rows", cfg.name)},
    }
    if not args.no_cpu_baseline:
        import oracle
        # leading rows, 512 at a time, until about 10 s of CPU work (the
        # mean's 1/N weight is the full workload's); numpy's elementwise
        # passes use one core
        rows, blk = 0, 512
        t0 = time.perf_counter()
        while rows < cfg.N and time.perf_counter() - t0 < 10.0:
            sl = slice(rows, min(cfg.N, rows + blk))
            oracle.softmax_cross_entropy(inputs["logits"][sl], inputs["t"][sl],
                                         reduction="sum", grad_scale=1.0 / cfg.N)
            rows = sl.stop
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": rows * cfg.V * 8.0 / dt / 1e9, "unit": "GB/s", "cores": 1,
            "kind": "oracle", **host_cpu(),
            "sample": f"rows 0-{rows - 1} of {cfg.name} in float64, 512-row blocks ({dt:.1f} s)"}
    return result


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5) -> dict:
    """A plain device-to-device copy of `nbytes`: the achievable-bandwidth
    yardstick, and the kernel whose FETCH_SIZE / WRITE_SIZE counters scale
    the others' (it moves exactly nbytes each way)."""
    import torch
    dev = torch.device("cuda", 0)
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    return {"bytes_each_way": nbytes, "ms": ms, "gbs_read_plus_write": 2 * nbytes / ms / 1e6}


# rocprofv3 kernel names of each timed kernel class.  grad_W's main launch
# stores bf16 (epilogue mode 3); the launch of its trailing tile columns, K
# split into fp32 partials, is mode 0.
KERNEL_NAMES = {"logits": "k_logits_lse", "gemm_x": "k_gemm_grad_x",
                "gemm_w": "k_gemm_grad_w<unsigned short, 3,",
                "gemm_w_tail": "k_gemm_grad_w<unsigned short, 0,",
                "ce_rows": "k_ce_rows", "copy": "copyBuffer"}


def summarize_counters(fetch_csv: str, write_csv: str, workload: str, command: str) -> dict:
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of each kernel class from two
    rocprofv3 --pmc runs, scaled by the same counters of the calibration copy
    (known bytes each way); written to the traffic file with the kernel
    sources' hash, so a later kernel change invalidates them."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                for cls, sub in KERNEL_NAMES.items():
                    if sub in r["Kernel_Name"]:
                        vals.setdefault(cls, []).append(float(r["Counter_Value"]))
        return {k: statistics.median(v) for k, v in vals.items()}

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    known_kib = (1 << 30) / 1024.0
    f_scale = known_kib / fetch["copy"] if fetch.get("copy") else None
    w_scale = known_kib / write["copy"] if write.get("copy") else None
    out = {}
    for cls in fetch:
        if cls == "copy" or cls not in write or not f_scale or not w_scale:
            continue
        rd = fetch[cls] * f_scale * 1024
        wr = write[cls] * w_scale * 1024
        out[cls] = {"bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr,
                    "fetch_kib_raw": fetch[cls], "write_kib_raw": write[cls],
                    "copy_scale_fetch": f_scale, "copy_scale_write": w_scale,
                    "source_sha": kernel_source_sha(), "command": command}
    data = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    data[workload] = out
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large-vocab-bf16",
                    choices=["tiny-f32", "mid-bf16", "large-vocab-bf16", "none-bf16", "ce-f32"])
    ap.add_argument("--dtype", default=None, choices=["bf16", "f16", "f32"],
                    help="round the workload's inputs to this type instead of its own")
    ap.add_argument("--forward-only", action="store_true",
                    help="reduction='none' workload: time the loss-only forward")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one call captured into a HIP graph")
    ap.add_argument("--acc-policy", default="accurate", choices=["accurate", "compact"])
    ap.add_argument("--chunk-rows", type=int, default=None)
    ap.add_argument("--group-rows", type=int, default=0,
                    help="rows of dL held per grad_W GEMM (0: the library's default; the "
                         "chunk rows: the per-chunk path with an fp32 accumulator)")
    ap.add_argument("--no-per-chunk", dest="per_chunk", action="store_false",
                    help="skip the per-chunk record of the default line")
    ap.add_argument("--no-ce", dest="ce", action="store_false",
                    help="skip the standalone-CE record of the default line")
    ap.add_argument("--cpu-rows", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true",
                    help="time every kernel class, not only the GEMMs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also time a plain 1 GiB device copy (bandwidth yardstick)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs into the traffic file")
    ap.add_argument("--counters-command", default="",
                    help="the command that produced the counter CSVs (recorded)")
    args = ap.parse_args()
    if args.summarize_counters:
        out = summarize_counters(*args.summarize_counters, args.workload, args.counters_command)
        print(json.dumps(out, indent=1))
        return 0
    if args.gpus != 1:
        print(f"the library runs on one GPU only (--gpus {args.gpus} requested); sharding over "
              "several GPUs is designed but not implemented", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs the GPU", file=sys.stderr)
        return 1
    result = bench_ce(args) if args.workload == "ce-f32" else bench_lce(args)
    if args.ce and args.workload == "large-vocab-bf16" and args.dtype in (None, "bf16"):
        result["ce"] = ce_record(args)
    if args.calibrate_copy:
        result["copy_calibration"] = copy_calibration()
        log(f"copy: {result['copy_calibration']['gbs_read_plus_write']:.0f} GB/s (read + write)")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
