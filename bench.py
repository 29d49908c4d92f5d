"""Benchmark of the FlashAttention-2 forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload train] [--splits S]
                    [--dtype bf16|fp16] [--B B] [--H H] [--d D] [--q-len NQ] [--kv-len NK]

A step is one fa2_fwd call (the whole hot path: one kernel launch) over the
workload's inputs (with --splits: one fa2_fwd_splitkv call, the split kernel and
the merge kernel), which are generated with the seeded recipe and copied to
HBM before timing starts.  First a settle phase (untimed steps for at least
--settle-seconds and until the launch rate of two consecutive quarter seconds
agrees within 2%, at most --settle-max-seconds; reported in the line as
"settle"), so that a GPU that was idle reaches its sustained clocks (a box's
first run can take a few seconds), then W untimed warm-up steps, then exactly K timed steps
bracketed by torch.cuda.synchronize().  An event recorded on the stream the
kernels are enqueued on separates consecutive launches, so every launch is
timed on its own: the roofline uses their mean, and the line gives their
median, min and max.  The device's name, compute units and graphics clock are
reported beside it; the clock is sampled through amdsmi during the settle phase
and over --clock-seconds of untimed steps right after the timed region, never
during it (a sampling thread's driver calls can delay launches, and a delayed
launch counts as idle time in the events and the wall clock).

Prints one JSON line.  ``value`` is TFLOP/s by the metric's count
(4*B*H*N^2*d, halved with the causal mask); ``roofline`` compares the same
algorithmic flops per launch against MI355X's dense bf16 MFMA peak;
``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of the same
workload on this host's cores, and ``parity`` compares the outputs of the last
timed step with the oracle's on the slices of that sample.

Variants: --dtype, --B, --H, --d, --q-len and --kv-len override the named
workload's type and shape (same seeded recipe).  With query and key lengths
that differ, the flop count is 4*d per visible (query, key) pair (the causal
mask aligned bottom-right), and a problem whose arithmetic intensity is below
MI355X's ridge point (peak flops / 8 TB/s) is reported against HBM bandwidth
instead: algorithmic bytes (Q, K, V read once, O and L written once) per
launch over the kernel time.
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
PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp32": 157.3}
PEAK_HBM_GBS = 8000.0
_FWD16 = ["exact_attention_62_amd/csrc/fa2_fwd_kernel.h", "exact_attention_62_amd/csrc/fa2_device.h"]
KERNEL_SOURCES = {"bf16": _FWD16 + ["exact_attention_62_amd/csrc/fa2_fwd_bf16.hip"],
                  "fp16": _FWD16 + ["exact_attention_62_amd/csrc/fa2_fwd_fp16.hip"],
                  "fp32": ["exact_attention_62_amd/csrc/fa2_fwd_f32.hip"]}
KERNEL_TYPE = {"bf16": "__bf16", "fp16": "_Float16"}


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="train", help="tiny, small, train, long or ragged")
    p.add_argument("--causal", type=int, choices=(0, 1), default=None,
                   help="override the workload's first mask setting")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--dtype", choices=("bf16", "fp16", "fp32"), default=None,
                   help="override the workload's element type")
    p.add_argument("--B", type=int, default=None, help="override the batch size")
    p.add_argument("--H", type=int, default=None, help="override the head count")
    p.add_argument("--d", type=int, default=None, help="override the head dimension")
    p.add_argument("--q-len", type=int, default=None, help="override the query length")
    p.add_argument("--kv-len", type=int, default=None,
                   help="key/value length (default: the query length)")
    p.add_argument("--backward", action="store_true",
                   help="time the backward pass (fa2_bwd) instead; flops = 2.5 x the forward's")
    p.add_argument("--ring", type=int, default=None, metavar="G",
                   help="time one GPU's share of attention with the key/value sequence in G shards "
                        "(the last query shard: G fa2_fwd_partial calls and one fa2_merge)")
    p.add_argument("--ring-streams", type=int, default=1, metavar="K",
                   help="with --ring: spread the partial-result launches over K streams")
    p.add_argument("--splits", type=int, default=None, metavar="S",
                   help="time the split-KV path (fa2_fwd_splitkv) with S splits; 0 = the pages' rule")
    p.add_argument("--clock-seconds", type=float, default=0.5,
                   help="untimed launches after the timed region while the shader clock is "
                        "sampled (0: no clock sampling)")
    p.add_argument("--settle-seconds", type=float, default=1.0,
                   help="before the warm-up steps, run steps for at least this many seconds, and "
                        "on until the launch rate is steady, so the clocks reach their sustained "
                        "level (reported as 'settle'; 0 disables it)")
    p.add_argument("--settle-max-seconds", type=float, default=8.0,
                   help="upper bound of the settle phase")
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
    for rel in KERNEL_SOURCES[dtype] + ["exact_attention_62_amd/csrc/fa2_internal.h"]:
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


def metric_flops(B: int, H: int, Nq: int, Nk: int, d: int, causal: bool) -> float:
    """The metric's flop count: 4*B*H*N^2*d (halved when causal) for equal lengths; otherwise
    4*d per visible (query, key) pair, the causal mask aligned bottom-right."""
    if Nq == Nk:
        return 4.0 * B * H * Nq * Nq * d / (2.0 if causal else 1.0)
    if not causal:
        return 4.0 * B * H * Nq * Nk * d
    off = Nk - Nq
    pairs = sum(min(Nk, max(0, i + 1 + off)) for i in range(Nq))
    return 4.0 * B * H * pairs * d


def cpu_baseline(w, q, k, v, o_gpu, l_gpu, causal: bool, scale: float, target_s: float):
    """Time the fp64 oracle on whole (batch, head) slices until ~target_s seconds pass.

    q, k, v are the CPU copies of the very inputs the GPU run used; o_gpu and
    l_gpu are the CPU copies of the outputs of the last timed step.  The oracle's
    results for the slices it computed are compared with those outputs element
    by element, which gives the parity of the timed run (returned separately).
    """
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention_fp64

    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    attention_fp64(q[:1, :1, :64], k[:1, :1, :64], v[:1, :1, :64], causal=causal)  # warm-up
    heads = 0
    err_o = err_l = 0.0
    finite = True
    t0 = time.perf_counter()
    elapsed = 0.0
    spent = 0.0  # oracle time only (the comparison is not timed)
    while heads < B * H and (heads == 0 or spent < target_s):
        b, h = divmod(heads, H)
        t1 = time.perf_counter()
        O, L = attention_fp64(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                              causal=causal, scale=scale)
        spent += time.perf_counter() - t1
        og = o_gpu[b, h].double().numpy()
        lg = l_gpu[b, h].double().numpy()
        finite = finite and bool(np.isfinite(og).all())
        err_o = max(err_o, float(np.abs(og - O[0, 0]).max(initial=0.0)))
        seen = np.isfinite(L[0, 0])
        if seen.any():
            err_l = max(err_l, float(np.abs(lg[seen] - L[0, 0][seen]).max()))
        if not np.array_equal(np.isfinite(lg), seen):
            finite = False
        heads += 1
    elapsed = spent
    flops = metric_flops(1, heads, Nq, Nk, d, causal)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    base = {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{heads} of the {B * H} (batch, head) slices of the {w.name} workload "
                   f"(all {Nq} rows each over {Nk} keys, fp64 numpy, full work even with the "
                   f"mask), {elapsed:.1f} s; throughput by the metric's flop count"),
        "seconds": elapsed,
        "blas_threads": int(threads),
        "host_cpus": len(os.sched_getaffinity(0)),
    }
    tol_o, tol_l = TOLERANCE[q_dtype_name(q)]
    parity = {"slices": heads, "of": B * H, "rows": heads * Nq,
              "max_abs_err_O": err_o, "max_abs_err_L": err_l, "tol_O": tol_o, "tol_L": tol_l,
              "ok": bool(finite and err_o <= tol_o and err_l <= tol_l),
              "compared": "the outputs of the last timed step, element by element, against "
                          "the fp64 oracle on the slices of the CPU baseline"}
    return base, parity


def q_dtype_name(q) -> str:
    import torch

    return {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[q.dtype]


# Parity tolerances (max-abs on O, max-abs on L): bf16 as the target states;
# fp16 half of it (a finer output rounding); fp32 the exact mode's bound.
TOLERANCE = {"bf16": (2e-2, 1e-3), "fp16": (1e-2, 1e-3), "fp32": (1e-5, 1e-5)}


class ClockSampler:
    """Samples the GPU's current graphics (shader) clock and socket power from a
    host thread, through the amdsmi library, while the benchmark runs.

    The device is matched to torch's device 0 by PCI bus address.  Any failure
    (no amdsmi, no permission) leaves the samples empty and records why.
    """

    def __init__(self, dev_index: int = 0, period_s: float = 0.001):
        import threading

        self.samples = []  # (perf_counter seconds, MHz, watts or None)
        self.error = None
        self.period = period_s
        self._stop = threading.Event()
        self._thread = None
        self._handle = None
        try:
            import amdsmi
            import torch

            self._amdsmi = amdsmi
            amdsmi.amdsmi_init()
            props = torch.cuda.get_device_properties(dev_index)
            want = (props.pci_domain_id, props.pci_bus_id, props.pci_device_id)
            for hnd in amdsmi.amdsmi_get_processor_handles():
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(hnd)  # "dddd:bb:dd.f"
                dom, bus, rest = bdf.split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self._handle = hnd
                    break
            if self._handle is None:
                self.error = f"no amdsmi device at PCI {want}"
        except Exception as e:  # noqa: BLE001 - any failure only disables sampling
            self.error = f"{type(e).__name__}: {e}"

    def _read(self):
        a = self._amdsmi
        clk = a.amdsmi_get_clock_info(self._handle, a.AmdSmiClkType.SYS)
        mhz = clk.get("clk") if isinstance(clk, dict) else None
        watts = None
        try:
            pw = a.amdsmi_get_power_info(self._handle)
            for key in ("current_socket_power", "average_socket_power"):
                if isinstance(pw.get(key), (int, float)):
                    watts = float(pw[key])
                    break
        except Exception:  # noqa: BLE001
            pass
        return mhz, watts

    def _run(self):
        while not self._stop.is_set():
            try:
                mhz, watts = self._read()
                if isinstance(mhz, (int, float)):
                    self.samples.append((time.perf_counter(), float(mhz), watts))
            except Exception as e:  # noqa: BLE001
                self.error = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self.period)

    def start(self):
        import threading

        if self._handle is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def halt(self):
        """Stop sampling (the thread ends after its current reading)."""
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
            self._thread = None

    def stop(self):
        self.halt()
        try:
            if self._handle is not None:
                self._amdsmi.amdsmi_shut_down()
                self._handle = None
        except Exception:  # noqa: BLE001
            pass

    def window(self, t0: float, t1: float):
        """Clock statistics of the samples taken between perf_counter times t0 and t1."""
        xs = [(mhz, w) for (t, mhz, w) in self.samples if t0 <= t <= t1]
        if not xs:
            return {"samples": 0, "error": self.error}
        mhz = sorted(x[0] for x in xs)
        watts = [x[1] for x in xs if x[1] is not None]
        out = {"samples": len(mhz), "mean_mhz": round(sum(mhz) / len(mhz), 1),
               "min_mhz": mhz[0], "max_mhz": mhz[-1]}
        if watts:
            out["mean_socket_w"] = round(sum(watts) / len(watts), 1)
        return out


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

    from exact_attention_62_amd import (fa2_bwd, fa2_bwd_workspace_size, fa2_fwd, fa2_fwd_cross,
                                        fa2_fwd_partial, fa2_fwd_splitkv, fa2_launch_shape,
                                        fa2_merge,
                                        fa2_num_splits, fa2_splitkv_workspace_size, load_library)
    from exact_attention_62_amd.inputs import WORKLOADS, make, make_upstream

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    load_library()
    w = WORKLOADS[args.workload]
    causal = bool(w.causal[0] if args.causal is None else args.causal)
    dtype = args.dtype or w.dtype
    B = w.B if args.B is None else args.B
    H = w.H if args.H is None else args.H
    d = w.d if args.d is None else args.d
    Nq = w.N if args.q_len is None else args.q_len
    Nk = Nq if args.kv_len is None else args.kv_len
    scale = 1.0 / d ** 0.5
    overridden = (dtype, B, H, d, Nq, Nk) != (w.dtype, w.B, w.H, w.d, w.N, w.N)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    q_cpu, k_cpu, v_cpu = make(w, args.seed, B=B, H=H, N=Nq, d=d, dtype=dtype, Nk=Nk)
    q, k, v = (t.to(dev) for t in (q_cpu, k_cpu, v_cpu))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    flops = metric_flops(B, H, Nq, Nk, d, causal)
    esize = q.element_size()
    # Algorithmic bytes per launch: Q, K, V read once, O and L written once.
    alg_bytes = float(B * H * (2 * Nq * d + 2 * Nk * d) * esize + B * H * Nq * 4)
    splits = None
    if args.backward:
        if dtype == "fp32":
            print("the backward pass is bf16 or fp16", file=sys.stderr)
            return 1
        if Nq == Nk:
            fa2_fwd(q, k, v, o, lse, causal=causal, scale=scale)
        else:
            fa2_fwd_cross(q, k, v, o, lse, causal=causal, scale=scale)
        do = make_upstream(B, H, Nq, d, args.seed, dtype=dtype).to(dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bws = torch.empty(fa2_bwd_workspace_size(B, H, Nq, d), dtype=torch.uint8, device=dev)
        flops = 2.5 * flops  # five products to the forward's two

        def step():
            fa2_bwd(q, k, v, o, do, lse, dq, dk, dv, bws, causal=causal, scale=scale)
    elif args.ring is not None:
        G = args.ring
        if dtype == "fp32" or Nq != Nk or Nq % G:
            print("--ring needs a 16-bit type and equal lengths divisible by G", file=sys.stderr)
            return 1
        S = Nq // G
        r = G - 1  # the last query shard: the heaviest share under the causal mask
        qs = q[:, :, r * S:].contiguous()
        shards = [(k[:, :, s * S:(s + 1) * S].contiguous(), v[:, :, s * S:(s + 1) * S].contiguous())
                  for s in range(G if not causal else r + 1)]
        o_parts = torch.empty((len(shards),) + tuple(qs.shape), dtype=torch.float32, device=dev)
        l_parts = torch.empty((len(shards),) + tuple(qs.shape[:3]), dtype=torch.float32, device=dev)
        o = torch.empty_like(qs)
        lse = torch.empty(qs.shape[:3], dtype=torch.float32, device=dev)
        flops = sum(metric_flops(B, H, S, S, d, causal and s == r) for s in range(len(shards)))
        alg_bytes = float(B * H * (2 * S * d + 2 * S * d * len(shards)) * esize + B * H * S * 4)

        # Partials of different shards are independent: with K streams they run side by side
        # (default stream priority), and the merge waits for all of them.
        side = [torch.cuda.Stream(device=dev) for _ in range(max(0, args.ring_streams - 1))]

        def step():
            start = torch.cuda.Event()
            start.record(stream)
            for st in side:
                st.wait_event(start)
            for s, (ks, vs) in enumerate(shards):
                st = ([stream] + side)[s % (len(side) + 1)]
                fa2_fwd_partial(qs, ks, vs, o_parts[s], l_parts[s], causal=causal and s == r,
                                scale=scale, stream=st)
            for st in side:
                done = torch.cuda.Event()
                done.record(st)
                stream.wait_event(done)
            fa2_merge(o_parts, l_parts, o, lse, stream=stream)
    elif args.splits is not None:
        if dtype == "fp32":
            print("the split-KV path is for bf16 and fp16", file=sys.stderr)
            return 1
        splits = args.splits if args.splits > 0 else fa2_num_splits(B, H, Nq, Nk, d)
        ws = torch.empty(fa2_splitkv_workspace_size(B, H, Nq, Nk, d, splits), dtype=torch.uint8,
                         device=dev)

        def step():
            fa2_fwd_splitkv(q, k, v, o, lse, ws, num_splits=splits, causal=causal, scale=scale)
    elif Nq != Nk:
        def step():
            fa2_fwd_cross(q, k, v, o, lse, causal=causal, scale=scale)
    else:
        def step():
            fa2_fwd(q, k, v, o, lse, causal=causal, scale=scale)

    props = torch.cuda.get_device_properties(dev)
    # One event between consecutive timed launches, all on the stream the kernels
    # are enqueued on: launch i runs between events i and i+1.  Created before
    # the settle phase: creating them between the warm-up and the timed region
    # left the GPU idle long enough, on a box's first run, for the next launches
    # to run up to a third slower for some 30 ms.
    events = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    clock = ClockSampler(0).start()
    t_settle = time.perf_counter()
    settled = 0
    t_sampled = t_settle
    steady, rate_prev, rate_last = False, None, None
    if args.settle_seconds > 0:
        # Untimed, reported: enough launches for the clocks to reach their sustained
        # level (a fresh GPU starts from idle clocks).  Synchronised every 16 launches
        # so that the queue stays short.  The clock is sampled over the first 70% of
        # the phase only: no sampling while timed (a sampling thread's calls into the
        # driver can delay launches, and a delayed launch shows up as idle time in the
        # events), and the launches go on while the sampler stops, because even a
        # short idle gap drops the clock again (after 3 s idle the next 20 launches
        # took 20% longer).
        # After the minimum, the phase goes on until two consecutive quarter-second
        # windows run launches at rates within 2% of each other (a box's first run
        # has taken seconds to reach its clocks).
        t_win, n_win = t_settle, 0
        while True:
            for _ in range(16):
                step()
            settled += 16
            n_win += 16
            torch.cuda.synchronize()
            now = time.perf_counter()
            elapsed = now - t_settle
            if t_sampled == t_settle and elapsed >= 0.7 * args.settle_seconds:
                clock.halt()
                t_sampled = time.perf_counter()
            if now - t_win >= 0.25:
                rate_prev, rate_last = rate_last, (now - t_win) / n_win
                t_win, n_win = now, 0
                steady = rate_prev is not None and abs(rate_last - rate_prev) <= 0.02 * rate_prev
            if elapsed >= args.settle_seconds and (steady or elapsed >= args.settle_max_seconds):
                break
    settle_s = time.perf_counter() - t_settle
    clock.halt()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    events[0].record(stream)
    for i in range(args.steps):
        step()
        events[i + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    # The timed step's outputs, kept for the parity check before the clock phase
    # below overwrites them (with the same values: the kernels are deterministic).
    o_timed, lse_timed = o.clone(), lse.clone()
    # The clock the timed launches ran at: sampled over untimed launches of the
    # same step right after the timed region.
    after = ClockSampler(0).start() if args.clock_seconds > 0 else None
    t_after = time.perf_counter()
    after_launches = 0
    while after is not None:
        for _ in range(16):
            step()
        after_launches += 16
        torch.cuda.synchronize()
        if time.perf_counter() - t_after >= args.clock_seconds:
            break
    t_after_end = time.perf_counter()
    if after is not None:
        after.stop()
    clock.stop()
    launch_ms = [events[i].elapsed_time(events[i + 1]) for i in range(args.steps)]
    kernel_ms = sum(launch_ms) / len(launch_ms)  # average launch duration on the stream
    srt = sorted(launch_ms)
    median_ms = (srt[(len(srt) - 1) // 2] + srt[len(srt) // 2]) / 2
    ms_per_step = wall * 1e3 / args.steps
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype]
    # Below the ridge point (peak flops per HBM byte) the roofline is bandwidth.
    hbm_bound = not args.backward and flops / alg_bytes < peak * 1e12 / (PEAK_HBM_GBS * 1e9)

    block_m = fa2_launch_shape(B, H, Nq, d, {"bf16": torch.bfloat16, "fp16": torch.float16,
                                              "fp32": torch.float32}[dtype])[0]
    traffic = (measured_traffic(w.name, causal, dtype)
               if splits is None and not args.backward and not overridden else None)
    c = "true" if causal else "false"
    if dtype == "fp32":
        kname = f"fa2_fwd_f32_kernel<{d}, {c}>"
    elif Nq == 1 and d in (64, 128, 256):  # one query row per head: the decoding kernel
        kname = f"fa2_decode_kernel<{KERNEL_TYPE[dtype]}, {d}>"
    else:
        # Wavefronts per workgroup: kBlockM / 32 (the split kernel always has
        # four); wavefronts per SIMD: 2, or 1 for d = 256 with splits or on a
        # grid of fewer than two items per CU.
        waves = 4 if splits is not None else block_m // 32
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        items = B * H * ((Nq + block_m - 1) // block_m)
        # The same rule as the library's dispatch: without splits four per SIMD
        # for d = 32 (128 VGPRs) and three for d = 64 (168); with splits three
        # for d = 32; one for d = 256 with splits or on small grids; two otherwise.
        if d == 32:
            occ = 4 if splits is None else 3
        elif d == 64 and splits is None:
            occ = 3
        else:
            occ = 1 if d == 256 and (splits is not None or items < 2 * cus) else 2
        kname = (f"fa2_fwd_kernel<{KERNEL_TYPE[dtype]}, {d}, {c}, "
                 f"{'true' if splits is not None else 'false'}, {waves}, {occ}>")
    if splits is not None:
        kname += (f" + fa2_combine_kernel<{KERNEL_TYPE[dtype]}, {d}> (both per step; kernel_ms "
                  f"covers the two)")
    if args.ring is not None:
        kname = (f"{G} x fa2_fwd_kernel<{KERNEL_TYPE[dtype]}, {d}, *, true, 4, "
                 f"{1 if d == 256 else 2}> + "
                 f"fa2_combine_kernel<{KERNEL_TYPE[dtype]}, {d}> (all per step; kernel_ms covers them)")
    if args.backward:
        T = KERNEL_TYPE[dtype]
        kname = (f"fa2_bwd_prep_kernel<{T}, {d}> + fa2_bwd_dkdv_kernel<{T}, {d}, {c}> + "
                 f"fa2_bwd_dq_kernel<{T}, {d}, {c}> (all per step; kernel_ms covers the three)")
    if hbm_bound:
        gbs = alg_bytes / (kernel_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "algorithmic_bytes": alg_bytes, "mfma_tflops": round(achieved, 2)}
    else:
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic}
    roofline.update({"kernel": kname, "kernel_ms": round(kernel_ms, 5),
                     "launch_ms": {"mean": round(kernel_ms, 5), "median": round(median_ms, 5),
                                   "min": round(srt[0], 5), "max": round(srt[-1], 5),
                                   "n": len(srt)},
                     "achieved_at_median": round(flops / (median_ms * 1e-3) / 1e12, 2),
                     "kernel_source_hash": kernel_source_hash(dtype)})
    name = w.name if not overridden else f"{w.name}-variant"
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
        "dtype": dtype,
        "data": "synthetic (seeded normal Q, K, V; see exact_attention_62_amd/inputs.py)",
        "config": {"workload": name, "B": B, "H": H, "N": Nq, "d": d,
                   **({"Nk": Nk} if Nk != Nq else {}),
                   "causal": causal, "scale": scale, "kBlockM": block_m,
                   "flops_per_step": flops,
                   **({"path": "split-KV", "num_splits": splits} if splits is not None else {}),
                   **({"path": f"one GPU's share of {args.ring} key/value shards (the last query "
                               f"shard)", "shard_len": Nq // args.ring,
                       "streams": args.ring_streams} if args.ring else {}),
                   **({"path": "backward"} if args.backward else {})},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "roofline": roofline,
        "device": {"name": props.name, "arch": props.gcnArchName,
                   "compute_units": props.multi_processor_count,
                   "gfx_clock_after_timed": (
                       {**after.window(t_after, t_after_end), "launches": after_launches,
                        "note": "amdsmi samples over untimed launches of the same step right "
                                "after the timed region (nothing samples while timed)"}
                       if after is not None else None),
                   "gfx_clock_settle": clock.window(t_settle, t_sampled)},
        "settle": {"seconds": round(settle_s, 3), "launches": settled, "steady": steady,
                   "ms_per_launch_last_windows": (
                       [round(1e3 * x, 5) for x in (rate_prev, rate_last) if x is not None]),
                   "note": "untimed launches before the warm-up, at least --settle-seconds and "
                           "until two consecutive quarter-second windows agree within 2% on "
                           "the launch rate (wall clock, 16 launches per synchronisation), "
                           "so the clocks reach their sustained level; the clock is sampled "
                           "over the first 70% of the minimum only"},
    }
    if args.cpu_seconds > 0 and not args.backward and not args.ring:
        out["cpu_baseline"], out["parity"] = cpu_baseline(
            w, q_cpu, k_cpu, v_cpu, o_timed.cpu(), lse_timed.cpu(), causal, scale,
            args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
