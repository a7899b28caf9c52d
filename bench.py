"""Benchmark of the KDA recurrent prefill forward on one MI355X.

One step = one kda_fwd launch over the whole workload (every chunk of every
(sequence, head)), inputs already resident in device memory.  Prints one JSON
line.  The default workload is B=2, T=1024, H=96, D=128 with a bf16 initial
state ~ N(0, 0.1^2) and a bf16 final state.

Roofline accounting (per launch):
  algorithmic bytes = token-heads * (8 D + 2 + 2 D)   (q, k, v, g, beta in; out)
                    + states in and out + A_log + dt_bias
  counted FLOP      = token-heads * 7 * D * D          (the per-token recurrence:
                      decay D^2, S k 2 D^2, rank-1 update 2 D^2, S q 2 D^2)
The kernel is HBM-bound at this arithmetic intensity (about 85 FLOP/B against a
ridge of about 315), so the roofline object reports bytes against 8 TB/s; the
fraction of the bf16 MFMA peak (2.5 PFLOP/s dense) is reported beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6
METRIC = "prefill tokens/sec (H=96,D=128) + % of MI355X bf16 MFMA peak"
PMC_PROFILE_FMT = os.path.join(ROOT, "profiles", "kda_fwd_{}_pmc.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "gated_delta_rule_62_amd", "csrc", f)
                  for f in ("kda_kernel.hip", "kda_params.h")]


def kernel_source_hash() -> str:
    """Hash of the kernel's code: the sources with // comments, trailing blanks and
    empty lines removed, so that a comment edit does not orphan the counters."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def algorithmic_bytes(inp) -> int:
    B, T, H, D = inp["q"].shape
    th = B * T * H
    b = th * (8 * D + 2 + 2 * D)
    for s in (inp["initial_state"], inp["final_state"]):
        if s is not None:
            b += s.numel() * s.element_size()
    b += inp["A_log"].numel() * 4 + inp["dt_bias"].numel() * 4
    return int(b)


def counted_flops(inp) -> int:
    B, T, H, D = inp["q"].shape
    return int(B * T * H * 7 * D * D)


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none or the kernel source changed since it was taken."""
    path = PMC_PROFILE_FMT.format(workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*(\w+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def gpu_clocks():
    """The GPU's current shader (sclk) and memory (mclk) clock levels, read from the amdgpu
    driver's sysfs files of this device (the ones rocm-smi reports), or None when they are
    not readable.  No other program is started."""
    import torch
    try:
        pr = torch.cuda.get_device_properties(torch.cuda.current_device())
        dev = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (pr.pci_domain_id, pr.pci_bus_id,
                                                         pr.pci_device_id)
    except (AttributeError, RuntimeError):
        return None
    found = {}
    for name in ("sclk", "mclk"):
        try:
            text = open(os.path.join(dev, "pp_dpm_" + name)).read()
        except OSError:
            continue
        for line in text.splitlines():
            m = re.search(r"([0-9.]+\s*[MG]hz)\s*\*\s*$", line, flags=re.I)
            if m:
                found[name] = m.group(1)
    return found or None


def cpu_baseline(inp, min_wall: float):
    """Times the fp64 oracle (the test suite's reference, unchanged) on the same
    workload on the host cores: whole runs repeated until min_wall seconds passed."""
    import numpy as np
    import torch

    import oracle
    if oracle.override_active():
        raise RuntimeError("KDA_ORACLE_LIB_OVERRIDE is set: the CPU baseline would time a "
                           "swapped oracle")
    B, T, H, D = inp["q"].shape
    oracle._load()
    # widen to fp64 outside the timed region, exactly as the oracle would
    wide = [np.ascontiguousarray(inp[n].to("cpu", torch.float64).numpy())
            for n in ("q", "k", "v", "g", "beta")]
    s0 = inp["initial_state"]
    s0w = None if s0 is None else np.ascontiguousarray(s0.to("cpu", torch.float64).numpy())
    A_log = inp["A_log"].to("cpu", torch.float64).numpy()
    dt_bias = inp["dt_bias"].to("cpu", torch.float64).numpy()
    cu = inp["cu_seqlens"].cpu() if inp["cu_seqlens"] is not None else None
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.kda_fwd(*wide, inp["scale"], A_log, dt_bias, inp["lower_bound"], s0w, cu,
                       nthreads=threads)
        reps += 1
        wall = time.perf_counter() - t0
        if wall >= min_wall:
            break
    result = {"value": reps * B * T / wall, "unit": "tokens/s", "cores": threads, "kind": "oracle",
              "sample": "fp64 per-token recurrence over the whole workload (%d tokens x %d heads), "
                        "%d run(s) in %.2f s wall on %d threads" % (B * T, H, reps, wall, threads)}
    # one core: the first few heads of the same workload, scaled to all heads
    hs = min(H, 8)
    sub = [np.ascontiguousarray(x[:, :, :hs]) for x in wide]
    s0s = None if s0w is None else np.ascontiguousarray(s0w[:, :hs])
    reps1 = 0
    t0 = time.perf_counter()
    while True:
        oracle.kda_fwd(*sub, inp["scale"], A_log[:hs], dt_bias[:hs], inp["lower_bound"], s0s, cu,
                       nthreads=1)
        reps1 += 1
        wall1 = time.perf_counter() - t0
        if wall1 >= min_wall / 2:
            break
    result["per_core_value"] = reps1 * B * T * hs / H / wall1
    result["per_core_sample"] = ("the same recurrence on heads 0..%d of the workload, %d run(s) in "
                                 "%.2f s on 1 thread, scaled to all %d heads" % (hs - 1, reps1, wall1, H))
    return result


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # The default warm-up runs long enough (about 0.25 s on the batched workload) for the
    # GPU clocks to settle: after 100 launches the timed mean is 2-3% slower than after 3000.
    ap.add_argument("--warmup", type=int, default=3000)
    ap.add_argument("--workload", default="batched")
    ap.add_argument("--chunk", type=int, default=None, help="force the chunk size")
    ap.add_argument("--v-tile", type=int, default=0, help="force the value tile")
    ap.add_argument("--path", choices=("fused", "split", "lds_state"), default="fused",
                    help="fused: the one-kernel forward (kda_fwd_sched); split: the prep and "
                         "recurrent kernels with a workspace (kda_fwd_split), both timed; "
                         "lds_state: the opt-in bf16 LDS state mode (kda_fwd_bf16_state)")
    ap.add_argument("--longest-first", action="store_true",
                    help="packed workloads: dispatch sequences longest first (kda_fwd_ordered); "
                         "the order is computed once, before the timed launches")
    ap.add_argument("--cpu-seconds", type=float, default=1.0,
                    help="minimum wall time of the CPU oracle baseline (whole-workload runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="after the timed launches, this many single launches each preceded by "
                         "a 1 GiB read sweep that evicts the L2s and the Infinity Cache (and as "
                         "many after a 1 GiB fill)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a known-size "
                         "kernel for scaling HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs one GPU's share of the work and "
              "has no multi-GPU path (heads or sequences would be sharded across GPUs with no "
              "exchange). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_62_amd as kda
    from gated_delta_rule_62_amd.workloads import WORKLOADS, make_inputs, token_heads

    w = WORKLOADS[args.workload]
    chunk = w.chunk_size if args.chunk is None else args.chunk
    inp = make_inputs(w, device="cuda")
    B, T, H, D = inp["q"].shape
    stream = torch.cuda.current_stream()

    order = None
    if args.longest_first:
        if inp["cu_seqlens"] is None or chunk or args.v_tile:
            print("--longest-first needs a packed workload and the automatic schedule",
                  file=sys.stderr)
            sys.exit(2)
        order = kda.kda_longest_first(inp["cu_seqlens"], stream=stream)

    # The binding checks and marshals the arguments once; the timed loop then calls
    # the C ABI directly, so host-side Python work never gaps the launches.
    lib = kda.load_library()
    args_c = kda.c_args(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["scale"],
                        inp["out"], inp["A_log"], inp["dt_bias"], inp["lower_bound"],
                        inp["initial_state"], inp["final_state"], inp["cu_seqlens"], stream)
    if args.path == "split":
        if order is not None or args.chunk is not None or w.chunk_size:
            print("--path split takes the automatic chunk length and the index order",
                  file=sys.stderr)
            sys.exit(2)
        ws_bytes = kda.kda_split_workspace_bytes(B * T, args_c[15], H, D, w.lower_bound, 0)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        call = lambda: lib.kda_fwd_split(*args_c, ws.data_ptr(), ws_bytes, 0, int(args.v_tile))
    elif args.path == "lds_state":
        if order is not None:
            print("--path lds_state takes the index order", file=sys.stderr)
            sys.exit(2)
        call = lambda: lib.kda_fwd_bf16_state(*args_c, int(chunk), int(args.v_tile))
    elif order is not None:
        call = lambda: lib.kda_fwd_ordered(*args_c, order.data_ptr())
    else:
        call = lambda: lib.kda_fwd_sched(*args_c, int(chunk), int(args.v_tile))

    def step():
        st = call()
        if st != kda.KDA_OK:
            raise kda.KdaError(st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    clocks_before = gpu_clocks()  # after the warm-up, right before the timed launches
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_launch = ev0.elapsed_time(ev1) / args.steps
    # a second pass with an event between consecutive launches gives the median and
    # minimum single launch (the event packets add a little time between launches,
    # so the mean above is taken without them)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    singles = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    clocks = gpu_clocks()  # after the timed launches, while the clocks are still up

    # The in-place state update (initial_state == final_state), timed as the pages time
    # it: K launches rotating over three state buffers, each pre-initialised with the
    # workload's initial state, so no launch reads the state the previous one wrote.
    inplace = None
    if args.path == "fused" and order is None and inp["final_state"] is not None:
        s0 = inp["initial_state"]
        if s0 is None:
            s0 = torch.zeros_like(inp["final_state"])
        bufs = [s0.to(inp["final_state"].dtype).clone() for _ in range(3)]
        calls_ip = [kda.c_args(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["scale"],
                               inp["out"], inp["A_log"], inp["dt_bias"], inp["lower_bound"], b, b,
                               inp["cu_seqlens"], stream) for b in bufs]
        torch.cuda.synchronize()
        i0 = torch.cuda.Event(enable_timing=True)
        i1 = torch.cuda.Event(enable_timing=True)
        i0.record(stream)
        for i in range(args.steps):
            st = lib.kda_fwd_sched(*calls_ip[i % 3], int(chunk), int(args.v_tile))
            if st != kda.KDA_OK:
                raise kda.KdaError(st)
        i1.record(stream)
        torch.cuda.synchronize()
        ms_ip = i0.elapsed_time(i1) / args.steps
        inplace = {"kernel_ms": ms_ip, "tokens_per_s": B * T / (ms_ip * 1e-3),
                   "state_buffers": 3,
                   "note": "initial_state and final_state the same buffer, three buffers "
                           "pre-initialised with the initial state used in turn"}

    cold = cold_dirty = None
    if args.cold_reps > 0:
        # Cold caches, two ways.  Each timed launch follows a 1 GiB sweep that evicts
        # the L2s and the 256 MB Infinity Cache.  A read sweep (a sum) leaves clean
        # lines behind, so the launch pays only for its own misses.  A write sweep
        # (a fill) leaves dirty lines, whose write-back the launch then also pays for.
        flush = torch.empty(1 << 28, dtype=torch.int32, device="cuda")
        flush.fill_(1)
        flush.sum()
        torch.cuda.synchronize()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)

        def timed_after(sweep):
            ms = []
            for _ in range(args.cold_reps):
                sweep()
                c0.record(stream)
                step()
                c1.record(stream)
                torch.cuda.synchronize()
                ms.append(c0.elapsed_time(c1))
            return sorted(ms)

        cold = timed_after(lambda: flush.sum())
        cold_dirty = timed_after(lambda: flush.fill_(1))
        del flush
    tokens = B * T
    value = tokens * args.steps / wall

    nbytes = algorithmic_bytes(inp)
    flops = counted_flops(inp)
    achieved = nbytes / (ms_per_launch * 1e-3) / 1e9
    tflops = flops / (ms_per_launch * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "kda_fwd %s: B=%d T=%d H=%d D=%d, bf16 q/k/v/g/beta ~N(0,1), "
                               "lower_bound=%g, state %s->%s" % (
                                   w.name, B, T, H, D, w.lower_bound, w.state_in, w.state_out),
                   "B": B, "T": T, "H": H, "D": D, "token_heads": token_heads(inp),
                   "chunk": chunk or "auto", "v_tile": args.v_tile or "auto",
                   "num_seqs": inp["N"],
                   "lengths": inp["lengths"] if inp["lengths"] is not None else None,
                   "sequence_order": "longest first" if order is not None else "index",
                   "path": args.path},
        "mfma_pct_of_bf16_peak": 100.0 * tflops / MFMA_BF16_PEAK_TFLOPS,
        # the most any kernel could reach: counted FLOP over the time the algorithmic bytes
        # take at the full HBM bandwidth
        "mfma_pct_ceiling_at_hbm_peak":
            100.0 * flops / (nbytes / (HBM_PEAK_GBS * 1e9)) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "kernel_ms": ms_per_launch,
        "kernel_ms_median": singles[len(singles) // 2],
        "kernel_ms_min": singles[0],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(w.name) if args.path == "fused" else None,
                     "algorithmic_bytes": nbytes, "counted_tflops": tflops},
        "kernel_source_hash": kernel_source_hash(),
        "gpu_clocks": {"before_timed": clocks_before, "after_timed": clocks},
    }
    if inplace is not None:
        result["inplace"] = inplace
    if cold is not None:
        med = cold[len(cold) // 2]
        med_d = cold_dirty[len(cold_dirty) // 2]
        result["cold_cache"] = {
            "reps": len(cold), "kernel_ms_median": med, "kernel_ms_min": cold[0],
            "hbm_frac_median": nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "note": "each launch after a 1 GiB read sweep that evicts the L2s and the "
                    "Infinity Cache and leaves clean lines",
            "after_write_sweep": {"kernel_ms_median": med_d, "kernel_ms_min": cold_dirty[0],
                                  "hbm_frac_median": nbytes / (med_d * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                  "note": "each launch after a 1 GiB fill: the launch also "
                                          "writes back the fill's dirty lines"}}
    if args.calib_copy_mb:
        # One elementwise kernel of known traffic (torch.neg: reads and writes every
        # byte once) over a source evicted from the caches by a 1 GiB fill first.
        n = args.calib_copy_mb * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        flush.fill_(1)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = {"read": n * 2, "write": n * 2}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
