"""Benchmark of the FlashAttention-2 forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload train] [--splits S]

A step is one fa2_fwd call (the whole hot path: one kernel launch) over the
workload's inputs (with --splits: one fa2_fwd_splitkv call, the split kernel and
the merge kernel), which are generated with the seeded recipe and copied to
HBM before timing starts.  W untimed steps, then exactly K timed steps
bracketed by torch.cuda.synchronize(); the launches are also bracketed by HIP
events recorded on the stream the kernel is enqueued on, which gives the
average kernel duration used for the roofline figure.

Prints one JSON line.  ``value`` is TFLOP/s by the metric's count
(4*B*H*N^2*d, halved with the causal mask); ``roofline`` compares the same
algorithmic flops per launch against MI355X's dense bf16 MFMA peak;
``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of the same
workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (4BHN²d, causal halved) and % of bf16 MFMA peak"
METRIC_BWD = "attention bwd TFLOP/s (2.5 x 4BHN²d, causal halved) and % of bf16 MFMA peak"
# MI355X published dense peaks (256 CUs at 2.4 GHz): bf16 MFMA 2.5 PFLOP/s
# (256 * 4096 flop/clk * 2.4 GHz = 2516.6 TFLOP/s); fp32 vector 157.3 TFLOP/s.
PEAK_TFLOPS = {"bf16": 2516.6, "fp32": 157.3}
KERNEL_SOURCES = {"bf16": "exact_attention_62_amd/csrc/fa2_fwd_bf16.hip",
                  "fp32": "exact_attention_62_amd/csrc/fa2_fwd_f32.hip"}


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="train", help="tiny, small, train, long or ragged")
    p.add_argument("--causal", type=int, choices=(0, 1), default=None,
                   help="override the workload's first mask setting")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--backward", action="store_true",
                   help="time the backward pass (fa2_bwd) instead; flops = 2.5 x the forward's")
    p.add_argument("--splits", type=int, default=None, metavar="S",
                   help="time the split-KV path (fa2_fwd_splitkv) with S splits; 0 = the pages' rule")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target duration of the CPU-oracle baseline sample (0 disables it)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="instead of the benchmark, run a plain device-to-device copy of MIB MiB "
                        "(--steps times): the reference for scaling FETCH_SIZE / WRITE_SIZE")
    return p.parse_args(argv)


def copy_calibration(mib: int, steps: int) -> int:
    """A plain copy kernel of known size, for calibrating the HBM byte counters."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                      "steps": steps}), flush=True)
    return 0


def kernel_source_hash(dtype: str) -> str:
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES[dtype], "exact_attention_62_amd/csrc/fa2_internal.h"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, causal: bool, dtype: str):
    """HBM bytes per launch from the committed counter summary, if it still applies.

    The summary records the kernel-source hash it was measured on; after any
    change to the kernel the figure no longer applies and None is returned.
    """
    path = os.path.join(ROOT, "profiles", f"fa2_fwd_{dtype}_{workload}_{'causal' if causal else 'full'}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(dtype):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, q, k, v, causal: bool, target_s: float):
    """Time the fp64 oracle on whole (batch, head) slices until ~target_s seconds pass.

    q, k, v are the CPU copies of the very inputs the GPU run used.
    """
    from threadpoolctl import threadpool_info

    from oracle import attention_fp64

    attention_fp64(q[:1, :1, :64], k[:1, :1, :64], v[:1, :1, :64], causal=causal)  # warm-up
    heads = 0
    t0 = time.perf_counter()
    elapsed = 0.0
    while heads < w.B * w.H and (heads == 0 or elapsed < target_s):
        b, h = divmod(heads, w.H)
        attention_fp64(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                       causal=causal, scale=w.scale)
        heads += 1
        elapsed = time.perf_counter() - t0
    flops = 4.0 * heads * w.N * w.N * w.d / (2.0 if causal else 1.0)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{heads} of the {w.B * w.H} (batch, head) slices of the {w.name} workload "
                   f"(all {w.N} rows each, fp64 numpy, full N^2 work even with the mask), "
                   f"{elapsed:.1f} s; throughput by the metric's flop count"),
        "seconds": elapsed,
        "blas_threads": int(threads),
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def main(argv=None) -> int:
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        return 2

    if args.copy_calibration:
        return copy_calibration(args.copy_calibration, args.steps)

    import torch

    from exact_attention_62_amd import (fa2_bwd, fa2_bwd_workspace_size, fa2_fwd,
                                        fa2_fwd_splitkv, fa2_num_splits,
                                        fa2_splitkv_workspace_size, load_library)
    from exact_attention_62_amd.inputs import WORKLOADS, make, make_upstream

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    load_library()
    w = WORKLOADS[args.workload]
    causal = bool(w.causal[0] if args.causal is None else args.causal)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    q_cpu, k_cpu, v_cpu = make(w, args.seed)
    q, k, v = (t.to(dev) for t in (q_cpu, k_cpu, v_cpu))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    flops = w.flops(causal)
    splits = None
    if args.backward:
        if w.dtype != "bf16" or w.d not in (64, 128):
            print("the backward pass is bf16 with d = 64 or 128", file=sys.stderr)
            return 1
        fa2_fwd(q, k, v, o, lse, causal=causal, scale=w.scale)
        do = make_upstream(w.B, w.H, w.N, w.d, args.seed).to(dev)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        bws = torch.empty(fa2_bwd_workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8,
                          device=dev)
        flops = 2.5 * flops  # five products to the forward's two

        def step():
            fa2_bwd(q, k, v, o, do, lse, dq, dk, dv, bws, causal=causal, scale=w.scale)
    elif args.splits is not None:
        if w.dtype != "bf16":
            print("the split-KV path is bf16 only", file=sys.stderr)
            return 1
        splits = args.splits if args.splits > 0 else fa2_num_splits(w.B, w.H, w.N, w.d)
        ws = torch.empty(fa2_splitkv_workspace_size(w.B, w.H, w.N, w.d, splits), dtype=torch.uint8,
                         device=dev)

        def step():
            fa2_fwd_splitkv(q, k, v, o, lse, ws, num_splits=splits, causal=causal, scale=w.scale)
    else:
        def step():
            fa2_fwd(q, k, v, o, lse, causal=causal, scale=w.scale)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps  # average launch duration on the stream
    ms_per_step = wall * 1e3 / args.steps
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]

    traffic = (measured_traffic(w.name, causal, w.dtype)
               if splits is None and not args.backward else None)
    kname = f"fa2_fwd_{w.dtype}_kernel<{w.d},{'true' if causal else 'false'}" + (
        ",false>" if w.dtype == "bf16" else ">")
    if splits is not None:
        kname = (f"fa2_fwd_bf16_kernel<{w.d},{'true' if causal else 'false'},true> + "
                 f"fa2_combine_kernel<{w.d}> (both per step; kernel_ms covers the two)")
    if args.backward:
        kname = (f"fa2_bwd_prep_kernel<{w.d}> + fa2_bwd_dkdv_kernel<{w.d},{'true' if causal else 'false'}> + "
                 f"fa2_bwd_dq_kernel<{w.d},{'true' if causal else 'false'}> (all per step; kernel_ms covers the three)")
    out = {
        "metric": METRIC if not args.backward else METRIC_BWD,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal Q, K, V; see exact_attention_62_amd/inputs.py)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": causal, "scale": w.scale, "kBlockM": 128,
                   "flops_per_step": flops,
                   **({"path": "split-KV", "num_splits": splits} if splits is not None else {}),
                   **({"path": "backward"} if args.backward else {})},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic,
                     "kernel": kname,
                     "kernel_ms": round(kernel_ms, 5),
                     "kernel_source_hash": kernel_source_hash(w.dtype)},
    }
    if args.cpu_seconds > 0 and not args.backward:
        out["cpu_baseline"] = cpu_baseline(w, q_cpu, k_cpu, v_cpu, causal, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
