"""Benchmark of the MoE dispatch+combine hot path on one MI355X.

One step = one call of moe_dispatch_combine (gate -> layout -> pack ->
combine, the combine reading the packed rows back) over one batch of
synthetic, seeded inputs already resident in HBM.  Prints one JSON line:
tokens/s of the whole path, achieved HBM GB/s against the algorithmic bytes,
a roofline entry for the dominant kernel (per-launch duration measured live
with HIP events on the launch stream) and the CPU oracle timed on a bounded
sample of the same workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--workload deepseek_v3] [--no-cpu-baseline]
                       [--path flat|two_leg|fp8|capacity|assign]
                       [--gamma 1.25] [--rho 0.5]
                       [--part-dtype bf16|f32]

--path two_leg times moe_dispatch_combine_nodes instead: the node-level
two-leg dispatch (one row per (token, node) crossing, then forwarded to the
experts) and the hierarchical combine (per-node partial sums, then their sum
at the source).  --path fp8 times moe_dispatch_combine_fp8: the pack
quantises each row to E4M3 codes with one fp32 scale per 128 elements and the
combine gathers and dequantises those rows.  --path capacity times
moe_dispatch_combine_capacity with one level C = ceil(gamma*T*K/E): every
expert's segment padded to C rows, overflow dropped.  --path assign times
the gate and moe_assign_tasks on a seeded replica layout (rho*E extra
replicas), tokens from rank 0, and reports remote-node crossings with and
without the replicas.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moe_inputs as mi  # noqa: E402

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, 8 TB/s
METRIC = "dispatch+combine tokens/s and achieved HBM GB/s (% of peak), 1 MI355X"
# sources whose text decides each kernel's memory traffic
KERNEL_SOURCES = {
    "pack": ["combine_moe_topk_amd/csrc/pack.hip"],
    "combine": ["combine_moe_topk_amd/csrc/combine.hip",
                "combine_moe_topk_amd/csrc/row_io.h"],
    "assign": ["combine_moe_topk_amd/csrc/assign.hip"],
    "gate": ["combine_moe_topk_amd/csrc/gate.hip"],
    "pack_nodes": ["combine_moe_topk_amd/csrc/pack.hip"],
    "forward": ["combine_moe_topk_amd/csrc/nodes.hip"],
    "partial": ["combine_moe_topk_amd/csrc/nodes.hip",
                "combine_moe_topk_amd/csrc/row_io.h"],
    "sum_nodes": ["combine_moe_topk_amd/csrc/nodes.hip",
                  "combine_moe_topk_amd/csrc/row_io.h"],
    "pack_capacity": ["combine_moe_topk_amd/csrc/pack.hip",
                      "combine_moe_topk_amd/csrc/capacity.hip"],
    "combine_capacity": ["combine_moe_topk_amd/csrc/combine.hip",
                         "combine_moe_topk_amd/csrc/row_io.h"],
    "pack_fp8": ["combine_moe_topk_amd/csrc/fp8.hip",
                 "combine_moe_topk_amd/csrc/row_io.h"],
    "combine_fp8": ["combine_moe_topk_amd/csrc/fp8.hip",
                    "combine_moe_topk_amd/csrc/row_io.h"],
}
# int32 vector ALU issue rate: 256 CUs x 64 lanes x 2.4 GHz (lane-ops/s)
ALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12


def kernel_bytes(w: mi.Workload) -> dict:
    """Algorithmic bytes one launch of each row kernel must move."""
    b, ob = w.elem_bytes, w.out_elem_bytes
    T, H, K, E = w.T, w.H, w.K, w.E
    return {
        # x read once, K rows written, slot positions read
        "pack": T * H * b + T * K * H * b + 4 * T * K,
        # K rows read, one row written, slot/weight/expert id read, scales
        "combine": T * K * H * b + T * H * ob + 12 * T * K + 4 * E,
    }


def fp8_kernel_bytes(w: mi.Workload, B: int = 128) -> dict:
    """Algorithmic bytes per launch of the FP8 pack and combine.  A row's
    payload is its H codes and H/B fp32 scales; the padding up to the
    128-byte row stride is not part of what the method moves."""
    b, ob = w.elem_bytes, w.out_elem_bytes
    T, H, K = w.T, w.H, w.K
    pay = H + 4 * (H // B)
    return {
        # x read once, K quantised rows written, slot positions read
        "pack_fp8": T * H * b + T * K * pay + 4 * T * K,
        # K quantised rows read, one row written, routing read, scales
        "combine_fp8": T * K * pay + T * H * ob + 12 * T * K + 4 * w.E,
    }


def capacity_kernel_bytes(w: mi.Workload, C: int, dropped: int) -> dict:
    """Algorithmic bytes per launch of the capacity path's pack (its used
    rows and its zeroed padding rows, two kernels) and combine; C = rows a
    segment holds, dropped = (token, slot) pairs over capacity."""
    b, ob = w.elem_bytes, w.out_elem_bytes
    T, H, K = w.T, w.H, w.K
    n_rows, kept = w.E * C, T * K - dropped
    return {
        # x read once, every padded row written, slots and row sources read
        "pack_capacity": T * H * b + n_rows * H * b + 4 * T * K + 4 * n_rows,
        # kept rows read, one row written, routing read
        "combine_capacity": kept * H * b + T * H * ob + 12 * T * K,
    }


def two_leg_kernel_bytes(w: mi.Workload, D: int, pb: int) -> dict:
    """Algorithmic bytes per launch of the two-leg kernels; D = crossings."""
    b, ob = w.elem_bytes, w.out_elem_bytes
    T, H, K, N = w.T, w.H, w.K, w.N
    return {
        # x read once, one row per crossing written, node slots read
        "pack_nodes": T * H * b + D * H * b + 4 * T * N,
        # each crossing row read once, K rows written, routing read
        "forward": D * H * b + T * K * H * b + T * (8 * K + 4 * N),
        # K rows read, one partial row per crossing written, routing read
        "partial": T * K * H * b + D * H * pb + T * (12 * K + 4 * N),
        # partial rows read, one output row written, node slots read
        "sum_nodes": D * H * pb + T * H * ob + 4 * T * N,
    }


def copy_calibration(mib: int, dev) -> None:
    """Three device copies of mib MiB: under rocprofv3 --pmc they give the
    counters' reading for a known number of bytes read and written."""
    import torch

    src = torch.ones(mib << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(os.path.join(ROOT, path), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries.

    Null when no summary exists or the kernel source changed since the
    counters were taken."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        data = json.load(open(p))
        ent = data[f"{kernel}/{workload}"]
    except (KeyError, ValueError):
        return None
    if ent.get("source_sha") != source_digest(KERNEL_SOURCES[kernel]):
        return None
    return ent.get("bytes_per_launch")


def traffic_source(kernel: str, workload: str, traffic) -> str:
    """Where roofline.traffic comes from: it is not measured in this run."""
    if traffic is None:
        return ("none: no committed counters for this kernel and workload, "
                "or its source changed since they were taken")
    return (f"profiles/traffic.json entry {kernel}/{workload}: rocprofv3 "
            f"FETCH_SIZE + WRITE_SIZE per launch from committed runs, "
            f"scaled by a plain copy's reading; kernel source sha "
            f"{source_digest(KERNEL_SOURCES[kernel])} unchanged since")


def load_valu(workload: str):
    """Vector instructions one moe_assign_tasks call issues, from committed
    rocprofv3 counters; null when absent or the source changed since."""
    p = os.path.join(ROOT, "profiles", "valu.json")
    try:
        ent = json.load(open(p))[f"assign/{workload}"]
    except (OSError, KeyError, ValueError):
        return None
    if ent.get("source_sha") != source_digest(KERNEL_SOURCES["assign"]):
        return None
    return ent.get("valu_insts_per_call")


def cpu_baseline(w: mi.Workload, d: dict, sample_tokens: int) -> dict:
    """The CPU oracle (single-threaded C) on the first tokens of the workload."""
    import oracle

    Ts = min(sample_tokens, w.T)
    x = np.ascontiguousarray(d["x"][:Ts])
    lg = np.ascontiguousarray(d["logits"][:Ts])
    oracle.gate(lg[:2], w.K)  # load the library outside the timing
    # whole passes of the oracle over the sample until about 10 s of CPU
    # work (at most 8 passes); throughput over all passes
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.dispatch_combine(x, lg, w.K, w.R, w.N, d["expert_scale"],
                                w.out_dtype)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps >= 8:
            break
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f
                        if ln.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": reps * Ts / dt, "unit": "tokens/s", "cores": 1,
            "kind": "oracle", "cpu": cpu, "host_cpus": os.cpu_count(),
            "sample": f"first {Ts} of {w.T} tokens of {w.name}, whole path "
                      f"(gate, layout, pack, combine), one thread, {reps} "
                      f"passes in {dt:.2f} s"}


def _pct(a, q):
    return float(np.percentile(np.asarray(a), q))


def _timed(fn, n, stream, before=None):
    """Per-call durations (ms) of n calls of fn, HIP events on stream."""
    import torch

    evs = []
    for _ in range(n):
        if before is not None:
            before()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def _timed_b2b(fn, n, stream) -> float:
    """Mean duration (ms) of n calls of fn enqueued back to back between
    one pair of HIP events: the GPU's time per call whenever the host
    enqueues faster than the GPU runs them."""
    import torch

    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def _gate_split(gate, step, n, stream):
    """(gate ms, step ms) on the GPU for a decode-sized step.  A gate call
    alone is enqueued about as slowly as the GPU runs it, so timing it
    back to back measures the host; instead the gate is timed as the extra
    time of back-to-back [gate, step] pairs over back-to-back steps, which
    the GPU paces."""
    def both():
        gate()
        step()
    alone = _timed_b2b(step, n, stream)
    pair = _timed_b2b(both, n, stream)
    return pair - alone, alone


def sequential_bounds(w, dev, stream, n=20) -> dict:
    """The pack and the combine on the same buffers and bytes as the step,
    with the slot table k*T + t instead of the expert-major permutation: every
    destination (pack) or source (combine) row stream runs sequentially.
    Same kernels, same byte counts and read:write mix; only the row order
    differs, so this is the rate the order-free access pattern allows."""
    import torch

    import combine_moe_topk_amd as moe

    if w.T * w.K * w.H * w.elem_bytes < (1 << 20):
        return None
    rows = torch.float32 if w.x_dtype == mi.F32 else torch.bfloat16
    odt = torch.float32 if w.out_dtype == mi.F32 else torch.bfloat16
    cfg = moe.make_cfg(w.T, w.H, w.E, w.K, w.R, w.N, w.x_dtype, w.out_dtype,
                       w.renorm)
    T, K = w.T, w.K
    slots = (torch.arange(K, dtype=torch.int32, device=dev)[None, :] * T +
             torch.arange(T, dtype=torch.int32, device=dev)[:, None])
    slots = slots.contiguous().view(-1)
    x = torch.randn((T, w.H), device=dev).to(rows)
    send = torch.empty((T * K, w.H), dtype=rows, device=dev)
    out = torch.empty((T, w.H), dtype=odt, device=dev)
    wt = torch.full((T * K,), 1.0 / K, dtype=torch.float32, device=dev)
    idx = torch.zeros(T * K, dtype=torch.int32, device=dev)
    for _ in range(3):
        moe.moe_dispatch_pack(cfg, x, slots, send, stream)
        moe.moe_combine(cfg, send, slots, wt, idx, None, out, stream)
    pk, cb = [], []
    for _ in range(n):  # pack then combine, as in a step
        pk += _timed(lambda: moe.moe_dispatch_pack(cfg, x, slots, send,
                                                   stream), 1, stream)
        cb += _timed(lambda: moe.moe_combine(cfg, send, slots, wt, idx, None,
                                             out, stream), 1, stream)
    kb = kernel_bytes(w)
    kb["combine"] -= 4 * w.E  # no expert scales read here
    return {"slots": "k*T + t",
            "pack_gbps": kb["pack"] / (_pct(pk, 50) * 1e-3) / 1e9,
            "combine_gbps": kb["combine"] / (_pct(cb, 50) * 1e-3) / 1e9,
            "pack_ms": _pct(pk, 50), "combine_ms": _pct(cb, 50)}


# The fused call takes the one-launch decode kernel after the gate for
# batches of at most 1024 tokens and 4096 (token, slot) pairs (the
# library's rule, stated in its decode kernel source).
DECODE_MAX_T, DECODE_MAX_TK = 1024, 4096


def config_line(w, dev, n=20) -> dict:
    """One workload through moe_dispatch_combine: warm and cold-clean step
    times, tokens/s, whole-path GB/s, and the dominant kernel's rate."""
    import torch

    import combine_moe_topk_amd as moe

    d = mi.make_inputs(w)
    rows = torch.float32 if w.x_dtype == mi.F32 else torch.bfloat16
    odt = torch.float32 if w.out_dtype == mi.F32 else torch.bfloat16

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    cfg = moe.make_cfg(w.T, w.H, w.E, w.K, w.R, w.N, w.x_dtype, w.out_dtype,
                       w.renorm)
    x, lg = to_dev(d["x"]), to_dev(d["logits"])
    del d["x"]
    scale = None if d["expert_scale"] is None else to_dev(d["expert_scale"])
    idx = torch.empty(w.T * w.K, dtype=torch.int32, device=dev)
    wt = torch.empty(w.T * w.K, dtype=torch.float32, device=dev)
    lay = moe.alloc_layout(cfg, dev)
    send = torch.empty((w.T * w.K, w.H), dtype=rows, device=dev)
    out = torch.empty((w.T, w.H), dtype=odt, device=dev)
    ws = moe.alloc_workspace(cfg, dev)
    stream = torch.cuda.current_stream()

    def step():
        moe.moe_dispatch_combine(cfg, x, lg, scale, idx, wt, lay, send, out,
                                 ws)

    for _ in range(5):
        step()
    torch.cuda.synchronize()
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    warm = _timed(step, n, stream)
    clean = _timed(step, n, stream,
                   before=lambda: flush.sum(dtype=torch.int64))
    del flush
    alg = w.algorithmic_bytes()
    ms = _pct(warm, 50)
    line = {"T": w.T, "H": w.H, "E": w.E, "K": w.K, "R": w.R, "N": w.N,
            "ms_warm": ms, "ms_cold_clean": _pct(clean, 50),
            "tokens_per_s": w.T / (ms * 1e-3),
            "gbps": alg / (ms * 1e-3) / 1e9,
            "frac_of_peak": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "frac_of_peak_cold_clean":
                alg / (_pct(clean, 50) * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    if w.T <= DECODE_MAX_T and w.T * w.K <= DECODE_MAX_TK:
        # gate, then one decode kernel: its time is the step less the gate
        gate, b2b = _gate_split(
            lambda: moe.moe_topk_gate(cfg, lg, idx, wt, stream), step, 4 * n,
            stream)
        dk = b2b - gate
        by = alg - w.T * (4 * w.E + 8 * w.K)  # less the gate's own bytes
        line["ms_back_to_back"] = b2b
        line["dominant"] = {"kernel": "decode (layout+pack+combine)",
                            "ms": dk, "gbps": by / (dk * 1e-3) / 1e9,
                            "frac": by / (dk * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        line["gate_ms"] = gate
    else:
        gate = _pct(_timed(lambda: moe.moe_topk_gate(cfg, lg, idx, wt,
                                                     stream), n, stream), 50)
        lay_ms = _pct(_timed(lambda: moe.moe_dispatch_layout(
            cfg, idx, lay, ws, stream), n, stream), 50)
        pk, cb = [], []
        for _ in range(n):  # in step order, so the cache state is a step's
            pk += _timed(lambda: moe.moe_dispatch_pack(cfg, x, lay.slot_pos,
                                                       send, stream), 1, stream)
            cb += _timed(lambda: moe.moe_combine(cfg, send, lay.slot_pos, wt,
                                                 idx, scale, out, stream),
                         1, stream)
        kb = kernel_bytes(w)
        t = {"pack": _pct(pk, 50), "combine": _pct(cb, 50)}
        dom = max(t, key=t.get)
        line["steps_ms"] = {"gate": gate, "layout": lay_ms, **t}
        line["dominant"] = {"kernel": dom, "ms": t[dom],
                            "gbps": kb[dom] / (t[dom] * 1e-3) / 1e9,
                            "frac": kb[dom] / (t[dom] * 1e-3) / 1e9 /
                            HBM_PEAK_GBPS}
    del x, lg, send, out, lay, ws, idx, wt
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return line


def extras(w, step, stream, alg, dev) -> dict:
    """Outside the timed region: per-step spread (warm), steps after flushing
    the last-level cache (cold), a device-to-device copy ceiling, and the
    clocks and versions of this run."""
    import subprocess

    import torch

    n = 20
    # warm: back-to-back steps, one event pair each
    warm = []
    for _ in range(n):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        warm.append((a, b))
    torch.cuda.synchronize()
    warm = [a.elapsed_time(b) for a, b in warm]
    # cold: 1 GiB written between steps evicts the 256 MB last-level cache
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(n):
        flush.fill_(1)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        cold.append((a, b))
    torch.cuda.synchronize()
    cold = [a.elapsed_time(b) for a, b in cold]
    # cold, clean: 1 GiB read between steps evicts the cache without leaving
    # dirty lines (after the write flush above, their write-back to HBM runs
    # inside the next step)
    clean = []
    for _ in range(n):
        flush.sum(dtype=torch.int64)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        clean.append((a, b))
    torch.cuda.synchronize()
    clean = [a.elapsed_time(b) for a, b in clean]
    del flush
    seq = sequential_bounds(w, dev, stream)
    # a plain 2 GiB device-to-device copy (torch), for context only: it
    # moves bytes 1:1, a mix the pack and combine do not have
    src = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 31) * 5 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst

    def run(cmd):
        try:
            return subprocess.run(cmd, capture_output=True, text=True,
                                  timeout=20).stdout.strip()
        except (OSError, subprocess.SubprocessError):
            return None

    clocks = run(["rocm-smi", "--showclocks", "--json"])
    try:  # keep the current engine and memory clocks of card 0 only
        card = next(iter(json.loads(clocks).values()))
        clocks = {k: v for k, v in card.items()
                  if k.startswith(("sclk", "mclk", "fclk"))}
    except (TypeError, ValueError, StopIteration, AttributeError):
        pass
    ver = None
    try:
        ver = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    driver = None
    try:
        driver = open("/sys/module/amdgpu/version").read().strip()
    except OSError:
        drv = run(["rocm-smi", "--showdriverversion", "--json"])
        try:
            driver = next(iter(json.loads(drv).values())).get("Driver version")
        except (TypeError, ValueError, StopIteration, AttributeError):
            driver = None
    med_w = _pct(warm, 50)
    return {
        "warm_ms": {"p10": _pct(warm, 10), "p50": med_w, "p90": _pct(warm, 90)},
        "cold_ms": {"p10": _pct(cold, 10), "p50": _pct(cold, 50),
                    "p90": _pct(cold, 90)},
        "cold_clean_ms": {"p10": _pct(clean, 10), "p50": _pct(clean, 50),
                          "p90": _pct(clean, 90)},
        "sequential_bound": seq,
        "device_copy_gbps": copy_gbps,
        "rocm": ver, "driver": driver, "torch": torch.__version__,
        "clocks": clocks,
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="deepseek_v3",
                    choices=sorted(mi.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=16384)
    ap.add_argument("--fused-only", action="store_true",
                    help="time only the fused call (for profiler runs)")
    ap.add_argument("--layout-tile", type=int, default=0,
                    help="tokens per layout workgroup (0: library default)")
    ap.add_argument("--path", default="flat",
                    choices=("flat", "two_leg", "fp8", "capacity", "assign",
                             "pack_orders"))
    ap.add_argument("--rho", type=float, default=0.5,
                    help="replica budget of --path assign")
    ap.add_argument("--gamma", type=float, default=1.25,
                    help="capacity factor of --path capacity")
    ap.add_argument("--part-dtype", default="bf16", choices=("bf16", "f32"))
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time replays")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the per-step distribution, cold-cache steps "
                         "and the copy ceiling")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run 3 plain device copies of this many MiB "
                         "(calibrates rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this library does one GPU's "
              "share of the dispatch/combine and uses no collectives; "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import combine_moe_topk_amd as moe

    w = mi.WORKLOADS[args.workload]
    print(f"bench: workload {w.name} T={w.T} H={w.H} E={w.E} K={w.K} "
          f"R={w.R} N={w.N}", file=sys.stderr, flush=True)
    moe.lib()
    d = mi.make_inputs(w)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    rows = torch.float32 if w.x_dtype == mi.F32 else torch.bfloat16
    odt = torch.float32 if w.out_dtype == mi.F32 else torch.bfloat16
    cfg = moe.make_cfg(w.T, w.H, w.E, w.K, w.R, w.N, w.x_dtype, w.out_dtype,
                       w.renorm, args.layout_tile)
    x, lg = to_dev(d["x"]), to_dev(d["logits"])
    scale = None if d["expert_scale"] is None else to_dev(d["expert_scale"])
    idx = torch.empty(w.T * w.K, dtype=torch.int32, device=dev)
    wt = torch.empty(w.T * w.K, dtype=torch.float32, device=dev)
    lay = moe.alloc_layout(cfg, dev)
    send = torch.empty((w.T * w.K, w.H), dtype=rows, device=dev)
    out = torch.empty((w.T, w.H), dtype=odt, device=dev)
    ws = moe.alloc_workspace(cfg, dev)
    stream = torch.cuda.current_stream()
    if args.path == "two_leg":
        return two_leg(args, w, d, cfg, x, lg, scale, idx, wt, lay, send, out,
                       ws, stream)
    if args.path == "assign":
        del send
        return assign_path(args, w, d, cfg, lg, idx, wt, stream)
    if args.path == "pack_orders":
        return pack_orders(args, w, cfg, x, lg, idx, wt, lay, send, ws, stream)
    if args.path == "capacity":
        del send
        return capacity_path(args, w, cfg, x, lg, scale, idx, wt, out, stream)
    if args.path == "fp8":
        del send
        return fp8_path(args, w, cfg, x, lg, scale, idx, wt, lay, out, ws,
                        stream)

    def step():
        # current stream: the launch stream, or the capture stream of --graph
        moe.moe_dispatch_combine(cfg, x, lg, scale, idx, wt, lay, send, out,
                                 ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if moe.moe_read_device_error(ws) != 0:
        raise RuntimeError("device reported an input error")
    eager_step = step
    if args.graph:
        # the library enqueues kernel launches only, so a step captures
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            step()
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eager_step()
        torch.cuda.synchronize()

        def step():
            graph.replay()

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()

    # ---- timed region: exactly K fused steps --------------------------------
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_host0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host0
    ms = ev0.elapsed_time(ev1) / args.steps
    print(f"bench: fused {ms:.4f} ms/step (host clock {1e3 * t_host / args.steps:.4f})",
          file=sys.stderr, flush=True)

    tokens_per_s = w.T / (ms * 1e-3)
    alg = w.algorithmic_bytes()
    gbps = alg / (ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.x_dtype == mi.BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "E": w.E,
                   "K": w.K, "R": w.R, "N": w.N, "rows": w.x_dtype,
                   "accumulate": "f32", "seed": w.seed,
                   "launch": "hip-graph" if args.graph else "stream"},
        "hbm": {"alg_bytes": alg, "gbps": gbps,
                "frac_of_peak": gbps / HBM_PEAK_GBPS},
    }

    decode_sized = w.T <= DECODE_MAX_T and w.T * w.K <= DECODE_MAX_TK
    if not args.fused_only and decode_sized:
        # ---- decode-sized: the gate, then one decode kernel ----------------
        # The fused call runs layout, pack and combine as one kernel here, so
        # the separate calls would time other kernels (and, at a few
        # microseconds each, the host's launch gaps).  The decode kernel's
        # time is the fused step less the gate, as in extras.configs.
        gate, b2b = _gate_split(
            lambda: moe.moe_topk_gate(cfg, lg, idx, wt, stream), step,
            max(args.steps, 50), stream)
        dk = b2b - gate
        by = alg - w.T * (4 * w.E + 8 * w.K)  # less the gate's own bytes
        result["steps_ms"] = {"gate": gate, "decode": dk}
        result["roofline"] = {
            "kernel": "decode", "bound": "hbm",
            "achieved": by / (dk * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": by / (dk * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "traffic": None,
            "traffic_source": traffic_source("decode", w.name, None),
            "alg_bytes_per_launch": by, "launch_ms": dk,
            "timing": "back-to-back fused steps less the gate, the gate "
                      "timed as the extra time of back-to-back [gate, "
                      "step] pairs",
        }
    elif not args.fused_only:
        # ---- per-kernel durations inside a real step ------------------------
        # The four calls below launch exactly the kernels of one fused step,
        # in the same order on the same stream; HIP events between them give
        # each step's duration in the cache state a real step leaves behind.
        n = max(args.steps, 5)
        names = ("gate", "layout", "pack", "combine")
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
               for _ in range(n)]
        for i in range(n):
            e = evs[i]
            e[0].record(stream)
            moe.moe_topk_gate(cfg, lg, idx, wt, stream)
            e[1].record(stream)
            moe.moe_dispatch_layout(cfg, idx, lay, ws, stream)
            e[2].record(stream)
            moe.moe_dispatch_pack(cfg, x, lay.slot_pos, send, stream)
            e[3].record(stream)
            moe.moe_combine(cfg, send, lay.slot_pos, wt, idx, scale, out, stream)
            e[4].record(stream)
        torch.cuda.synchronize()
        per = {nm: [evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(n)]
               for j, nm in enumerate(names)}
        steps_ms = {nm: float(np.mean(v)) for nm, v in per.items()}
        result["steps_ms"] = steps_ms
        result["steps_pct_ms"] = {nm: {"p10": _pct(v, 10), "p50": _pct(v, 50),
                                       "p90": _pct(v, 90)}
                                  for nm, v in per.items()}
        kb = kernel_bytes(w)
        dom = max(("pack", "combine"), key=lambda k: steps_ms[k])
        achieved = kb[dom] / (steps_ms[dom] * 1e-3) / 1e9
        traffic = load_traffic(dom, w.name)
        result["roofline"] = {
            "kernel": dom, "bound": "hbm", "achieved": achieved,
            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
            "traffic_source": traffic_source(dom, w.name, traffic),
            "alg_bytes_per_launch": kb[dom],
            "launch_ms": steps_ms[dom],
        }
        for k in ("pack", "combine"):
            result["roofline"][f"{k}_gbps"] = kb[k] / (steps_ms[k] * 1e-3) / 1e9

    if args.copy_calib_mib > 0:
        copy_calibration(args.copy_calib_mib, dev)
        result["copy_calib_bytes"] = args.copy_calib_mib << 20

    if not args.fused_only and not args.no_extras:
        result["extras"] = extras(w, step, stream, alg, dev)
        # every workload through the same fused call, measured in this run
        del send, out, lay, ws
        torch.cuda.empty_cache()
        configs = {}
        for name in ("tiny", "mixtral", "qwen3_skewed", "deepseek_v3",
                     "deepseek_v3_decode", "kimi"):
            print(f"bench: config {name}", file=sys.stderr, flush=True)
            configs[name] = config_line(mi.WORKLOADS[name], dev)
        result["extras"]["configs"] = configs

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, d, args.cpu_sample_tokens)

    print(json.dumps(result), flush=True)
    return 0


def pack_orders(args, w, cfg, x, lg, idx, wt, lay, send, ws, stream) -> int:
    """The pack kernel on the step's buffers with two destination orders:
    args.warmup launches of each, then args.steps launches with the
    layout's expert-major slots, then args.steps with slot k*T + t (every
    destination stream sequential).  Under rocprofv3 the dispatches come in
    that order (bench_profile.py pack_orders splits them).  One JSON line."""
    import torch

    import combine_moe_topk_amd as moe

    moe.moe_topk_gate(cfg, lg, idx, wt, stream)
    moe.moe_dispatch_layout(cfg, idx, lay, ws, stream)
    T, K = w.T, w.K
    seq = (torch.arange(K, dtype=torch.int32, device=x.device)[None, :] * T +
           torch.arange(T, dtype=torch.int32, device=x.device)[:, None])
    seq = seq.contiguous().view(-1)
    orders = {"expert_major": lay.slot_pos, "sequential": seq}
    for _ in range(args.warmup):
        for sl in orders.values():
            moe.moe_dispatch_pack(cfg, x, sl, send, stream)
    res = {}
    for name, sl in orders.items():
        ms = _pct(_timed(lambda: moe.moe_dispatch_pack(cfg, x, sl, send,
                                                       stream),
                         args.steps, stream), 50)
        res[name] = {"ms": ms,
                     "gbps": kernel_bytes(w)["pack"] / (ms * 1e-3) / 1e9}
    print(json.dumps({"path": "pack_orders", "workload": w.name,
                      "steps": args.steps, "warmup": args.warmup, **res}),
          flush=True)
    return 0


def two_leg(args, w, d, cfg, x, lg, scale, idx, wt, lay, send, out, ws,
            stream) -> int:
    """Time moe_dispatch_combine_nodes (the two-leg path); one JSON line."""
    import torch

    import combine_moe_topk_amd as moe

    dev = x.device
    pdt = torch.bfloat16 if args.part_dtype == "bf16" else torch.float32
    pb = 2 if args.part_dtype == "bf16" else 4
    cap = moe.moe_node_rows_max(cfg)
    ns = torch.empty((cap, w.H), dtype=x.dtype, device=dev)
    part = torch.empty((cap, w.H), dtype=pdt, device=dev)

    def step():
        moe.moe_dispatch_combine_nodes(cfg, x, lg, scale, idx, wt, lay, ns,
                                       send, part, out, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if moe.moe_read_device_error(ws) != 0:
        raise RuntimeError("device reported an input error")
    D = int(lay.node_off[-1].item())  # crossings (outside the timed region)

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    print(f"bench: two-leg {ms:.4f} ms/step, {D} crossings for "
          f"{w.T * w.K} slots", file=sys.stderr, flush=True)

    kb = two_leg_kernel_bytes(w, D, pb)
    meta = w.T * (4 * w.E + 32 * w.K + 8 + 4 * w.N) + 8 * (w.E + w.R + w.N)
    alg = sum(kb.values()) + meta
    # per-kernel durations inside real steps (same launches, same order)
    n = max(args.steps, 5)
    names = ("gate", "layout", "pack_nodes", "forward", "partial", "sum_nodes")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)]
           for _ in range(n)]
    for i in range(n):
        e = evs[i]
        e[0].record(stream)
        moe.moe_topk_gate(cfg, lg, idx, wt, stream)
        e[1].record(stream)
        moe.moe_dispatch_layout(cfg, idx, lay, ws, stream)
        e[2].record(stream)
        moe.moe_dispatch_pack_nodes(cfg, x, lay.node_slot, ns, stream)
        e[3].record(stream)
        moe.moe_dispatch_forward(cfg, ns, lay.node_slot, idx, lay.slot_pos,
                                 send, stream)
        e[4].record(stream)
        moe.moe_combine_partial(cfg, send, lay.slot_pos, wt, idx, scale,
                                lay.node_slot, part, stream)
        e[5].record(stream)
        moe.moe_combine_nodes(cfg, part, lay.node_slot, out, stream)
        e[6].record(stream)
    torch.cuda.synchronize()
    steps_ms = {nm: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1])
                                   for i in range(n)]))
                for j, nm in enumerate(names)}
    dom = max(kb, key=lambda k: steps_ms[k])
    achieved = kb[dom] / (steps_ms[dom] * 1e-3) / 1e9
    gbps = alg / (ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": w.T / (ms * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.x_dtype == mi.BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "path": "two_leg", "T": w.T, "H": w.H,
                   "E": w.E, "K": w.K, "R": w.R, "N": w.N, "rows": w.x_dtype,
                   "partials": args.part_dtype, "accumulate": "f32",
                   "seed": w.seed},
        "hbm": {"alg_bytes": alg, "gbps": gbps,
                "frac_of_peak": gbps / HBM_PEAK_GBPS},
        "dedup": {"crossing_rows": D, "slot_rows": w.T * w.K,
                  "inter_node_row_ratio": D / (w.T * w.K)},
        "steps_ms": steps_ms,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": load_traffic(dom, w.name),
                     "alg_bytes_per_launch": kb[dom],
                     "launch_ms": steps_ms[dom],
                     **{f"{k}_gbps": kb[k] / (steps_ms[k] * 1e-3) / 1e9
                        for k in kb}},
    }
    if args.copy_calib_mib > 0:
        copy_calibration(args.copy_calib_mib, dev)
        result["copy_calib_bytes"] = args.copy_calib_mib << 20
    print(json.dumps(result), flush=True)
    return 0


def fp8_path(args, w, cfg, x, lg, scale, idx, wt, lay, out, ws,
             stream) -> int:
    """Time moe_dispatch_combine_fp8 (E4M3 rows, scale per 128); JSON line."""
    import torch

    import combine_moe_topk_amd as moe

    B = 128
    rb = moe.moe_fp8_row_bytes(w.H, B)
    if rb == 0:
        raise SystemExit(f"H={w.H} does not split into blocks of {B}")
    send = torch.empty((w.T * w.K, rb), dtype=torch.uint8, device=x.device)

    def step():
        moe.moe_dispatch_combine_fp8(cfg, x, lg, scale, idx, wt, lay, send,
                                     out, ws, B, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if moe.moe_read_device_error(ws) != 0:
        raise RuntimeError("device reported an input error")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    print(f"bench: fp8 {ms:.4f} ms/step", file=sys.stderr, flush=True)

    T, H, K = w.T, w.H, w.K
    kb = fp8_kernel_bytes(w, B)
    meta = T * (4 * w.E + 32 * K + 8) + 8 * (w.E + w.R + w.N)
    alg = kb["pack_fp8"] + kb["combine_fp8"] + meta - 4 * T * K - 12 * T * K
    n = max(args.steps, 5)
    names = ("gate", "layout", "pack_fp8", "combine_fp8")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
           for _ in range(n)]
    for i in range(n):
        e = evs[i]
        e[0].record(stream)
        moe.moe_topk_gate(cfg, lg, idx, wt, stream)
        e[1].record(stream)
        moe.moe_dispatch_layout(cfg, idx, lay, ws, stream)
        e[2].record(stream)
        moe.moe_dispatch_pack_fp8(cfg, x, lay.slot_pos, send, B, stream)
        e[3].record(stream)
        moe.moe_combine_fp8(cfg, send, lay.slot_pos, wt, idx, scale, out, B,
                            stream)
        e[4].record(stream)
    torch.cuda.synchronize()
    steps_ms = {nm: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1])
                                   for i in range(n)]))
                for j, nm in enumerate(names)}
    dom = max(kb, key=lambda k: steps_ms[k])
    achieved = kb[dom] / (steps_ms[dom] * 1e-3) / 1e9
    gbps = alg / (ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8-e4m3",
        "data": "synthetic",
        "config": {"workload": w.name, "path": "fp8", "T": T, "H": H,
                   "E": w.E, "K": K, "R": w.R, "N": w.N, "rows": w.x_dtype,
                   "payload": "e4m3+f32 scale/128", "accumulate": "f32",
                   "seed": w.seed},
        "hbm": {"alg_bytes": alg, "gbps": gbps,
                "frac_of_peak": gbps / HBM_PEAK_GBPS},
        "steps_ms": steps_ms,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": load_traffic(dom, w.name),
                     "alg_bytes_per_launch": kb[dom],
                     "launch_ms": steps_ms[dom],
                     **{f"{k}_gbps": kb[k] / (steps_ms[k] * 1e-3) / 1e9
                        for k in kb}},
    }
    if args.copy_calib_mib > 0:
        copy_calibration(args.copy_calib_mib, x.device)
        result["copy_calib_bytes"] = args.copy_calib_mib << 20
    print(json.dumps(result), flush=True)
    return 0


def capacity_path(args, w, cfg, x, lg, scale, idx, wt, out, stream) -> int:
    """Time moe_dispatch_combine_capacity (one capacity level); JSON line."""
    import torch

    import combine_moe_topk_amd as moe

    C = int(np.ceil(args.gamma * w.T * w.K / w.E))
    levels = [C]
    n_rows = w.E * C
    lay = moe.alloc_capacity_layout(cfg, levels, x.device)
    ws = moe.alloc_capacity_workspace(cfg, x.device)
    send = torch.empty((n_rows, w.H), dtype=x.dtype, device=x.device)

    def step():
        moe.moe_dispatch_combine_capacity(cfg, x, lg, scale, idx, wt, levels,
                                          lay, send, out, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    dropped = int(lay.dropped[0].item())
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    print(f"bench: capacity {ms:.4f} ms/step, C={C}, dropped {dropped}",
          file=sys.stderr, flush=True)

    T, H, K = w.T, w.H, w.K
    kb = capacity_kernel_bytes(w, C, dropped)
    meta = T * (4 * w.E + 32 * K + 8) + 8 * w.E
    alg = kb["pack_capacity"] + kb["combine_capacity"] + meta
    n = max(args.steps, 5)
    names = ("gate", "layout_capacity", "pack_capacity", "combine_capacity")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
           for _ in range(n)]
    for i in range(n):
        e = evs[i]
        e[0].record(stream)
        moe.moe_topk_gate(cfg, lg, idx, wt, stream)
        e[1].record(stream)
        moe.moe_dispatch_layout_capacity(cfg, idx, levels, lay, ws, stream)
        e[2].record(stream)
        moe.moe_dispatch_pack_capacity(cfg, x, lay.slot_pos, lay.row_src,
                                       send, stream)
        e[3].record(stream)
        moe.moe_combine_capacity(cfg, send, lay.slot_pos, wt, idx, scale, out,
                                 stream)
        e[4].record(stream)
    torch.cuda.synchronize()
    steps_ms = {nm: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1])
                                   for i in range(n)]))
                for j, nm in enumerate(names)}
    dom = max(kb, key=lambda k: steps_ms[k])
    achieved = kb[dom] / (steps_ms[dom] * 1e-3) / 1e9
    gbps = alg / (ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.x_dtype == mi.BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "path": "capacity", "T": T, "H": H,
                   "E": w.E, "K": K, "R": w.R, "N": w.N, "gamma": args.gamma,
                   "capacity": C, "rows": w.x_dtype, "accumulate": "f32",
                   "seed": w.seed},
        "hbm": {"alg_bytes": alg, "gbps": gbps,
                "frac_of_peak": gbps / HBM_PEAK_GBPS},
        "capacity": {"rows": n_rows, "slots": T * K, "dropped": dropped,
                     "pad_ratio": n_rows / (T * K),
                     "drop_rate": dropped / (T * K)},
        "steps_ms": steps_ms,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": load_traffic(dom, w.name),
                     "alg_bytes_per_launch": kb[dom],
                     "launch_ms": steps_ms[dom],
                     **{f"{k}_gbps": kb[k] / (steps_ms[k] * 1e-3) / 1e9
                        for k in kb}},
    }
    if args.copy_calib_mib > 0:
        copy_calibration(args.copy_calib_mib, x.device)
        result["copy_calib_bytes"] = args.copy_calib_mib << 20
    print(json.dumps(result), flush=True)
    return 0


def assign_path(args, w, d, cfg, lg, idx, wt, stream) -> int:
    """Time gate + moe_assign_tasks; report crossings; JSON line."""
    import torch

    import combine_moe_topk_amd as moe

    dev = lg.device
    holds = torch.from_numpy(mi.replica_layout(w.E, w.R, args.rho, 0)).to(dev)
    un, ur = mi.assign_draws(w.T, w.K, 0)
    un = torch.from_numpy(un.view(np.int32)).to(dev)
    ur = torch.from_numpy(ur.view(np.int32)).to(dev)
    src = torch.zeros(w.T, dtype=torch.int32, device=dev)
    ar = torch.empty(w.T * w.K, dtype=torch.int32, device=dev)
    rm = torch.empty(w.T, dtype=torch.int64, device=dev)
    ws = moe.alloc_assign_workspace(cfg, dev)

    def step():
        moe.moe_topk_gate(cfg, lg, idx, wt, stream)
        moe.moe_assign_tasks(cfg, idx, src, holds, un, ur, ar, rm, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if moe.moe_read_device_error(ws) != 0:
        raise RuntimeError("device reported an input error")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    t_gate = t_assign = 0.0
    for _ in range(args.steps):
        ev[0].record(stream)
        moe.moe_topk_gate(cfg, lg, idx, wt, stream)
        ev[1].record(stream)
        moe.moe_assign_tasks(cfg, idx, src, holds, un, ur, ar, rm, ws, stream)
        ev[2].record(stream)
        torch.cuda.synchronize()
        t_gate += ev[0].elapsed_time(ev[1])
        t_assign += ev[1].elapsed_time(ev[2])
    ms_gate, ms_assign = t_gate / args.steps, t_assign / args.steps
    ms = ms_gate + ms_assign
    masks = rm.cpu().numpy().view(np.uint64)
    with_rep = int(sum(bin(int(v)).count("1") for v in masks))
    # the same tokens with home placement only (no replicas): the remote
    # nodes of the token's experts
    per_rank, per_node = w.E // w.R, w.R // w.N
    home = (idx.view(w.T, w.K).cpu().numpy() // per_rank) // per_node
    without = int(sum(len(set(r.tolist()) - {0}) for r in home))
    print(f"bench: assign {ms_assign * 1e3:.1f} us, crossings {with_rep} "
          f"with replicas vs {without} without", file=sys.stderr, flush=True)
    T, K = w.T, w.K
    by = T * (4 * K + 8 * K + 4 + 4 * K + 8) + w.R * w.E + 8 * w.E
    # issued vector instructions x 64 lanes (an upper bound on lane-ops:
    # inactive lanes count) per second, against the int32 issue rate
    valu_insts = load_valu(w.name)
    achieved = (None if valu_insts is None
                else valu_insts * 64 / (ms_assign * 1e-3) / 1e12)
    result = {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": w.name, "path": "assign", "T": T, "E": w.E,
                   "K": K, "R": w.R, "N": w.N, "rho": args.rho,
                   "src_rank": 0, "seed": w.seed},
        "steps_ms": {"gate": ms_gate, "assign": ms_assign},
        "crossings": {"with_replicas": with_rep, "home_only": without,
                      "ratio": with_rep / max(without, 1)},
        "roofline": {"kernel": "assign", "bound": "alu",
                     "achieved": achieved, "peak": ALU_PEAK_TOPS,
                     "unit": "Tops/s",
                     "frac": None if achieved is None
                     else achieved / ALU_PEAK_TOPS,
                     "traffic": None, "alg_bytes_per_launch": by,
                     "valu_insts_per_launch": valu_insts,
                     "mtokens_per_s": T / (ms_assign * 1e-3) / 1e6,
                     "launch_ms": ms_assign},
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
