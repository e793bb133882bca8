#!/usr/bin/env python3
"""Throughput of the fused chunked KL loss (forward + backward) on one MI355X.

One step = one ckl_fwd_bwd call over the whole batch: every chunk's logits
GEMM, row pass (log-normaliser, gather, KL, in-place gradient), dH and dW
GEMMs, with inputs already resident in HBM.  Default workload: the
gpt-oss-like head, N = 32,768 tokens (1 x 32K), d = 2880, V = 201,088, K = 100,
chunk chosen by the planner under the 6 GiB workspace budget.

Prints one JSON line on stdout; progress goes to stderr.
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

BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
# sources (and the build script, which holds the compiler flags) a traffic record is valid for
BUILD = "chunked_kl_loss_seq_amd/build.py"
GEMM_SOURCES = ["chunked_kl_loss_seq_amd/csrc/gemm_core.hpp", "chunked_kl_loss_seq_amd/csrc/kernels_gemm.hip", BUILD]
LOGITS_SOURCES = ["chunked_kl_loss_seq_amd/csrc/gemm_core.hpp", "chunked_kl_loss_seq_amd/csrc/kernels_logits.hip",
                  BUILD]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(kind):
    return os.path.join(ROOT, "profiles", f"{kind}_gemm_hbm_traffic.json" if kind != "topk"
                        else "topk_hbm_traffic.json")


def traffic_from_profile(kernel_kind):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current sources of that kernel; else None."""
    path = traffic_path(kernel_kind)
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        if rec.get("source_sha") != source_hash(TRAFFIC_KINDS[kernel_kind][1]):
            return None
        return rec.get("bytes_per_launch")
    except (OSError, ValueError):
        return None


TOPK_SOURCES = ["chunked_kl_loss_seq_amd/csrc/kernels_topk.hip", BUILD]
# traffic record kind -> (substrings of the kernel name, sources the record is valid for)
TRAFFIC_KINDS = {
    "logits": (("gemm_kernel", "ELb1ELb1ELi0E"), LOGITS_SOURCES),
    "dh": (("gemm_kernel", "ELb1ELb0ELi1E"), GEMM_SOURCES),
    "dw": (("gemm_kernel", "ELb0ELb0ELi2E"), GEMM_SOURCES),
    "topk": (("topk_kernel", "DF16b"), TOPK_SOURCES),
}


def _counter_per_launch(path, name_filter, counter):
    import csv

    vals = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and name_filter(r["Kernel_Name"]):
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows matched in {path}")
    return sum(vals) / len(vals), len(vals)


def traffic_summary(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, commands):
    """Write profiles/<kind>_gemm_hbm_traffic.json from rocprofv3 --pmc counter
    files: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of each GEMM, each
    scaled by what the same counter reads for a plain device copy of 1 GiB."""
    is_copy = lambda n: "copyBuffer" in n  # noqa: E731
    cal_f, _ = _counter_per_launch(cal_fetch_csv, is_copy, "FETCH_SIZE")
    cal_w, _ = _counter_per_launch(cal_write_csv, is_copy, "WRITE_SIZE")
    copy_kib = float(1 << 20)
    sf, sw = copy_kib / cal_f, copy_kib / cal_w
    for kind, (tags, sources) in TRAFFIC_KINDS.items():
        sel = lambda n, tags=tags: all(t in n for t in tags)  # noqa: E731
        try:
            f, nf = _counter_per_launch(fetch_csv, sel, "FETCH_SIZE")
            w, nw = _counter_per_launch(write_csv, sel, "WRITE_SIZE")
        except SystemExit:
            continue  # that kernel did not run in these profiles
        rec = {"kernel": kind if kind == "topk" else f"{kind} GEMM", "source_sha": source_hash(sources),
               "launches": [nf, nw],
               "fetch_kib_per_launch_raw": f, "write_kib_per_launch_raw": w,
               "copy_calibration": {"bytes": 1 << 30, "fetch_kib": cal_f, "write_kib": cal_w,
                                    "fetch_scale": sf, "write_scale": sw},
               "fetch_bytes_per_launch": f * sf * 1024, "write_bytes_per_launch": w * sw * 1024,
               "bytes_per_launch": (f * sf + w * sw) * 1024, "commands": commands}
        out = traffic_path(kind)
        with open(out, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        log(f"[traffic] {kind}: fetch {rec['fetch_bytes_per_launch'] / 1e9:.2f} GB, "
            f"write {rec['write_bytes_per_launch'] / 1e9:.2f} GB per launch -> {out}")


def resolve_workload(number, dtype=None):
    """Named workload ``number``, with H, W and dH in ``dtype`` instead of its own
    type when given (same shapes, seed and recipe; the name records the change)."""
    import dataclasses

    from chunked_kl_loss_seq_amd import workloads as WL

    wl = WL.WORKLOADS[number]
    if dtype and dtype != wl.dtype:
        wl = dataclasses.replace(wl, dtype=dtype, name=f"{wl.name}-{dtype}")
    return wl


def cpu_baseline(number, rows, wl=None):
    """The oracle as it stands, timed on the host cores over a bounded sample."""
    import numpy as np  # noqa: F401

    from chunked_kl_loss_seq_amd import workloads as WL
    from oracle import kl_oracle as O

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    wl = wl or WL.WORKLOADS[number]
    inp = WL.make_custom(wl, number, rows=rows)
    t0 = time.perf_counter()
    O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"])
    dt = time.perf_counter() - t0
    valid = int(inp["mask"].sum())
    n = len(inp["mask"])
    return {"value": valid / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": (f"first {n} positions of the same workload" if n < wl.N
                       else "the whole workload")
            + f", float64 NumPy/BLAS dense definition, {dt:.2f} s wall"}


def cpu_model():
    """Model name of the host CPU (lscpu, else /proc/cpuinfo), or None."""
    import subprocess

    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def bench_topk(args):
    """Teacher cache writer: per row of bf16 teacher logits [R, V], the top K ids and values."""
    import numpy as np  # noqa: F401
    import torch

    from chunked_kl_loss_seq_amd import binding
    from chunked_kl_loss_seq_amd import workloads as WL

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    binding.lib()
    R, V, K = args.topk_rows, 201088, 100
    log(f"[bench] generating {R} x {V} bf16 teacher logits (N(0, 3))")
    x = torch.from_numpy(WL.teacher_logits(R, V, seed=1)).to("cuda:0").to(torch.bfloat16).contiguous()
    ids = torch.empty((R, K), dtype=torch.int32, device=x.device)
    vals = torch.empty((R, K), dtype=torch.float32, device=x.device)
    for _ in range(args.warmup):
        binding.topk(x, K, ids, vals)
    torch.cuda.synchronize()
    binding.timing_enable(True)
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        binding.topk(x, K, ids, vals)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    k_ms, k_n = binding.timing_query("topk")
    binding.timing_enable(False)
    launch_ms = k_ms / max(k_n, 1)
    alg_bytes = R * V * 2 + R * K * 8  # logits read once, ids and values written once
    gbs = alg_bytes / (launch_ms / 1e3) / 1e9
    log(f"[bench] top-K: {ms:.3f} ms/step, {R / (ms / 1e3):.0f} rows/s, {gbs:.0f} GB/s algorithmic")
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import topk_rows

        n = 256
        xs = x[:n].float().cpu().numpy()
        t0 = time.perf_counter()
        topk_rows(xs, K)
        dt = time.perf_counter() - t0
        cpu = {"value": n / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
               "sample": f"first {n} rows, float64 NumPy stable argsort per row, {dt:.2f} s wall"}
        log(f"[bench] oracle {cpu['value']:.1f} rows/s")
    out = {
        "metric": "teacher top-K cache writer rows/s (HBM-bound)",
        "value": round(R / (ms / 1e3), 1),
        "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "teacher-logits-gpt-oss-vocab", "rows": R, "V": V, "K": K, "parallelism": "none"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile("topk"), "kernel": "top-K",
                     "launch_avg_ms": round(launch_ms, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_sweep_rows(args):
    """Workspace against sequence length: the fused call on the first R
    positions of one workload for each R, with the library's workspace released
    before each size, so that each size makes its own single allocation.  The
    pages' point is that the fused loss's memory barely grows with the input
    grows ("A New Trick...", section "Does this matter for longer documents?")."""
    import torch

    from chunked_kl_loss_seq_amd import binding
    from chunked_kl_loss_seq_amd import workloads as WL

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    binding.lib()
    sizes = sorted(int(x) for x in args.sweep_rows.split(","))
    wl = WL.WORKLOADS[args.workload]
    if sizes[-1] > wl.N:
        raise SystemExit(f"workload {args.workload} has {wl.N} positions")
    log(f"[sweep] generating the first {sizes[-1]} positions of {wl.name}")
    inp = WL.make(args.workload, rows=sizes[-1])
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    H = torch.from_numpy(inp["H"]).to(dev).to(tdt)
    W = torch.from_numpy(inp["W"]).to(dev).to(tdt)
    ids = torch.from_numpy(inp["ids"]).to(dev)
    T = torch.from_numpy(inp["tlogit"]).to(dev)
    mask = torch.from_numpy(inp["mask"]).to(dev) if wl.mask != "none" else None
    del inp
    d, V, K = wl.d, wl.V, wl.K
    loss = torch.empty((), dtype=torch.float32, device=dev)
    dH = torch.empty_like(H)
    dW = torch.empty((V, d), dtype=torch.float32, device=dev)
    rows_out = []
    for R in sizes:
        C, plan_bytes = binding.plan(R, d, V, K, wl.dtype)
        binding.release_workspace()
        torch.cuda.synchronize()
        free0, _ = torch.cuda.mem_get_info(dev)
        m = mask[:R] if mask is not None else None
        binding.fwd_bwd(H[:R], W, ids[:R], T[:R], m, 0, out_loss=loss, dH=dH[:R], dW=dW)
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info(dev)
        held = binding.workspace_bytes_held()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(args.steps):
            binding.fwd_bwd(H[:R], W, ids[:R], T[:R], m, 0, out_loss=loss, dH=dH[:R], dW=dW)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / args.steps
        rec = {"tokens": R, "chunk": C, "chunks": -(-R // C), "plan_bytes": plan_bytes, "held_bytes": held,
               "mem_get_info_drop_bytes": free0 - free1, "ms_per_call": round(ms, 3),
               "tokens_per_s": round(R / (ms / 1e3), 1), "dense_fp32_logit_grid_bytes": R * V * 4}
        log(f"[sweep] N={R}: chunk {C} x {rec['chunks']}, plan {plan_bytes / 2**30:.3f} GiB, held "
            f"{held / 2**30:.3f} GiB, free-memory drop {(free0 - free1) / 2**30:.3f} GiB, {ms:.1f} ms/call")
        rows_out.append(rec)
    print(json.dumps({"metric": "fused KL workspace bytes vs sequence length", "workload": wl.name,
                      "d": d, "V": V, "K": K, "steps": args.steps, "rows": rows_out}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=4, help="named workload number (4 = gpt-oss head, 32K tokens)")
    ap.add_argument("--chunk", type=int, default=-1, help="rows per chunk (default: the workload's own)")
    ap.add_argument("--dtype", choices=["bf16", "f32"], default=None,
                    help="type of H, W and dH in place of the workload's own (fused and two-pass runs)")
    ap.add_argument("--variant", choices=["fused", "two-pass", "topk"], default="fused",
                    help="fused: one ckl_fwd_bwd call per step; two-pass: ckl_fwd then ckl_bwd (logits recomputed); "
                         "topk: the teacher top-K cache writer (ckl_topk) over --topk-rows rows")
    ap.add_argument("--topk-rows", type=int, default=8192, help="rows of teacher logits for --variant topk")
    ap.add_argument("--sweep-rows", default="",
                    help="comma-separated position counts: run the fused call on that many first positions of "
                         "--workload for each, the workspace released in between (memory against N)")
    ap.add_argument("--cpu-rows", type=int, default=-1,
                    help="positions in the oracle's timed sample (default: the whole workload up to 8192 "
                         "positions, else 4096)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (reference for HBM byte counters)")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="host only: turn rocprofv3 --pmc counter files into the per-GEMM traffic records")
    ap.add_argument("--traffic-commands", default="", help="the profiling commands, stored with the records")
    args = ap.parse_args()

    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, commands=args.traffic_commands)
        return

    if args.copy_calibration:
        import torch

        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": 1 << 30, "launches": 5}))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    if args.variant == "topk":
        bench_topk(args)
        return
    if args.sweep_rows:
        bench_sweep_rows(args)
        return

    import numpy as np
    import torch

    from chunked_kl_loss_seq_amd import binding
    from chunked_kl_loss_seq_amd import workloads as WL

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    binding.lib()
    wl = resolve_workload(args.workload, args.dtype)
    chunk = wl.chunk if args.chunk < 0 else args.chunk
    log(f"[bench] generating {wl.name}: N={wl.N} d={wl.d} V={wl.V} K={wl.K} {wl.dtype}")
    inp = WL.make_custom(wl, args.workload)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    H = torch.from_numpy(inp["H"]).to(dev).to(tdt)
    W = torch.from_numpy(inp["W"]).to(dev).to(tdt)
    ids = torch.from_numpy(inp["ids"]).to(dev)
    T = torch.from_numpy(inp["tlogit"]).to(dev)
    mask = torch.from_numpy(inp["mask"]).to(dev) if wl.mask != "none" else None
    n_valid = int(inp["mask"].sum())
    N, d, V, K = wl.N, wl.d, wl.V, wl.K
    C, ws_plan = binding.plan(N, d, V, K, wl.dtype, chunk)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    dH = torch.empty_like(H)
    dW = torch.empty((V, d), dtype=torch.float32, device=dev)
    del inp["H"], inp["W"]

    two_pass = args.variant == "two-pass"
    row_lse = torch.empty((N,), dtype=torch.float32, device=dev)
    if two_pass:
        C1, ws1 = binding.plan(N, d, V, K, wl.dtype, chunk, pass_="fwd")
        C, ws_plan = binding.plan(N, d, V, K, wl.dtype, chunk, pass_="bwd")
        ws_plan = max(ws_plan, ws1)
        log(f"[bench] two-pass: forward chunk {C1} rows, backward chunk {C} rows")

    def step():
        if two_pass:
            binding.fwd(H, W, ids, T, mask, chunk, out_loss=loss, row_lse=row_lse)
            binding.bwd(H, W, ids, T, row_lse, mask, chunk=chunk, dH=dH, dW=dW)
        else:
            binding.fwd_bwd(H, W, ids, T, mask, chunk, out_loss=loss, dH=dH, dW=dW)

    log(f"[bench] chunk {C} rows, planned workspace {ws_plan / 2**30:.3f} GiB; warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warm, loss {loss.item():.6f}; timing {args.steps} steps")

    binding.timing_enable(True)
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    kinds = {}
    for k in ("logits", "rows", "dh", "dh_reduce", "dw", "other"):
        t, n = binding.timing_query(k)
        kinds[k] = (t, n)
    binding.timing_enable(False)
    ws_held = binding.workspace_bytes_held()

    flop_gemm_launch_total = 2.0 * n_valid * d * V * args.steps  # per GEMM kind (and pass) over the timed region
    logits_passes = 2 if two_pass else 1  # the two-pass backward recomputes the logits
    gemm = {k: kinds[k] for k in ("logits", "dh", "dw")}
    dom = max(gemm, key=lambda k: gemm[k][0] / (logits_passes if k == "logits" else 1))
    dom_ms, dom_n = gemm[dom]
    achieved = flop_gemm_launch_total * (logits_passes if dom == "logits" else 1) / (dom_ms / 1e3) / 1e12
    total_tflops = (6.0 + 2.0 * (logits_passes - 1)) * n_valid * d * V / (ms / 1e3) / 1e12
    peak = BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS
    per_kernel = {k: {"ms_per_step": kinds[k][0] / args.steps, "launches_per_step": kinds[k][1] / args.steps}
                  for k in kinds}
    for k in ("logits", "dh", "dw"):
        f = flop_gemm_launch_total * (logits_passes if k == "logits" else 1)
        per_kernel[k]["tflops"] = f / (kinds[k][0] / 1e3) / 1e12 if kinds[k][0] else None
    traffic = traffic_from_profile(dom)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": f"{dom} GEMM",
                "launch_avg_ms": round(dom_ms / max(dom_n, 1), 4)}
    log(f"[bench] {ms:.2f} ms/step, {N / (ms / 1e3):.0f} tokens/s, {total_tflops:.1f} TFLOP/s whole step")
    for k, v in per_kernel.items():
        log(f"[bench]   {k:10s} {v['ms_per_step']:8.3f} ms/step  launches {v['launches_per_step']:.0f}"
            + (f"  {v['tflops']:.1f} TFLOP/s" if v.get("tflops") else ""))

    cpu = None
    if not args.no_cpu_baseline:
        rows = args.cpu_rows if args.cpu_rows > 0 else (N if N <= 8192 else 4096)
        log(f"[bench] timing the oracle on {rows} positions")
        cpu = cpu_baseline(args.workload, rows, wl)
        log(f"[bench] oracle {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    metric = "fused KL fwd+bwd tokens/s + MFMA TFLOP/s % peak; peak workspace GiB"
    if two_pass:
        metric = "chunked KL forward + recomputing backward (two calls) tokens/s; MFMA TFLOP/s % peak; workspace GiB"
    out = {
        "metric": metric,
        "value": round(N / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "variant": args.variant, "N": N, "valid_tokens": n_valid, "d": d, "V": V,
                   "K": K, "chunk": C,
                   "global_batch": N // (wl.seq_len or N), "seq_len": wl.seq_len or N, "parallelism": "none"},
        "tokens_per_s_valid": round(n_valid / (ms / 1e3), 1),
        "tflops": round(total_tflops, 2),
        "pct_bf16_peak": round(100 * total_tflops / BF16_PEAK_TFLOPS, 2),
        "workspace_gib": round(ws_plan / 2**30, 4),
        "workspace_held_gib": round(ws_held / 2**30, 4),
        "per_kernel": per_kernel,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
