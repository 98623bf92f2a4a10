#!/usr/bin/env python3
"""Throughput of the chunked KDA forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1] [--no-cpu]
                    [--path chunked|recurrent] [--gate safe|unbounded]
    python bench.py --copy-calibration      # plain 1 GiB device copy, for HBM counter scaling

A step is one kda_fwd call (the whole hot path: varlen scheduler when
cu_seqlens is given, intra-chunk kernel, state-chain/output kernel) over one
batch of synthetic inputs already resident in HBM. The default workload is the
fixed-length prefill B=1, T=8192, H=64, K=V=128 (bf16 inputs, stateless,
fp32 final state). Prints ONE JSON line.

  value       tokens/s = tokens per step / mean step time (HIP events)
  roofline    HBM roofline of the dominant kernel (longest average launch):
              its algorithmic bytes per launch / its average launch duration
              (HIP events recorded by libkda on the launch stream around each
              kernel, over the timed steps) against 8 TB/s. Algorithmic bytes
              are the kernel's share of the path's 1,282 B per token-head: the
              intra kernel reads q, k, v, g, beta (1,026 B), the chain kernel
              writes out (256 B) and reads/writes the states (64 KiB fp32 or
              32 KiB bf16 per sequence-head). "traffic" is the measured HBM
              bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a
              plain-copy calibration) recorded in profiles/traffic.json for the
              current kernel-source hash, else null.
  path        the same for the whole call: 1,282 B per token-head + state bytes
              over the call's duration, and the bf16 MFMA fraction at
              180,224 FLOP per token-head
  kernels     per-kernel average duration, algorithmic bytes and the bytes the
              design moves (including the per-chunk records written by the
              intra kernel and read back by the chain kernel)
  cpu_baseline the fp64 CPU oracle timed on the host cores over the same
              workload (bounded: see "sample"), with a one-thread figure

Timing: about 50 ms of plain device copies first (--settle-ms; no step of the
method, reported as clock_settle_ms: an idle GPU takes some milliseconds to
raise its clocks, and without it the first tens of calls run up to 12% slower),
then W warm-up steps (default 50), then K timed
steps between two HIP events on the launch stream, with nothing recorded
between the calls; the steps alternate between two input sets (distinct
tensors, the second drawn with the next seed) so that no step finds its inputs
in the last-level cache from the step before. The per-kernel durations come
from K further steps with libkda's per-kernel events (created without a
system-scope fence), kept out of the headline span.

  extra_workloads  the uniform varlen workload (8 sequences of 1024 tokens,
              fp32 initial and final state) timed the same way, after the
              headline one (--no-extra skips it)
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/sec at T=8192,H=64,K=V=128 bf16; % of MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FLOP_PER_TOKEN_HEAD = 180224          # dense C=64 chunk form, 2C(3K+2V) + 6KV
BYTES_PER_TOKEN_HEAD = 1282           # q, k, v, g (4 x 256) + beta 2 + out 256
IN_BYTES_PER_TOKEN_HEAD = 1026        # read by the intra kernel: q, k, v, g, beta
OUT_BYTES_PER_TOKEN_HEAD = 256        # written by the chain kernel: out
CHUNK = 64


def kernel_source_hash():
    from gated_delta_rule_87_amd.rocprof_summary import kernel_source_hash as h
    return h()


def recorded_traffic(workload_name, kernel):
    """Measured HBM bytes per launch of `kernel`, if recorded for the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = rec.get("workloads", {}).get(workload_name)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    k = ent.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def copy_calibration(steps):
    """Plain device-to-device copy of 1 GiB: the counter-scaling reference."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    src.fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"copy_calibration": True, "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                      "launches": steps + 1, "ms_per_launch": ms, "GBps_read_plus_write": 2 * n / ms / 1e6}),
          flush=True)


def settle_clocks(dev, ms):
    """Keep the GPU busy with plain device copies for about `ms` milliseconds, so that the
    warm-up and timed steps that follow run at the clocks a busy GPU holds (an idle GPU
    takes some milliseconds to raise them). Nothing of the method runs here."""
    import torch
    if ms <= 0:
        return 0.0
    a = torch.empty(64 << 20, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    a.fill_(1.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    t = time.perf_counter()
    while True:
        for _ in range(8):
            b.copy_(a)
        e1.record()
        e1.synchronize()
        if e0.elapsed_time(e1) >= ms or time.perf_counter() - t > 5.0:
            break
    del a, b
    return e0.elapsed_time(e1)


def cpu_threads():
    n = os.environ.get("OMP_NUM_THREADS")
    if n and n.isdigit():
        return int(n)
    try:
        return min(16, len(os.sched_getaffinity(0)))
    except AttributeError:
        return min(16, os.cpu_count() or 1)


def host_cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=1, help="workload index (kda_inputs.workload)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--path", choices=["chunked", "recurrent"], default="chunked")
    ap.add_argument("--gate", choices=["safe", "unbounded"], default="safe",
                    help="safe: lower_bound * sigmoid gate (the default); unbounded: the gate without the "
                         "safe bound, -exp(A_log) * softplus(g + dt_bias)")
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="plain device copies for this long before the warm-up steps (clock settle)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra workload (uniform varlen 8 x 1024) timed after the headline one")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 1 GiB device copy instead (HBM counter scaling reference)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this implementation runs on exactly one GPU (asked for --gpus {args.gpus}); "
              "sharding over several GPUs is a design, not built", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.steps)
        return

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    res = measure(args.workload, args, headline=True)
    if args.workload == 1 and args.path == "chunked" and not args.no_extra:
        # the pages' best case (uniform varlen, 8 sequences of 1024 tokens), same timing
        ex = measure(2, args, headline=False)
        res["extra_workloads"] = {ex["config"]["workload"]: ex}
    print(json.dumps(res), flush=True)


def measure(widx, args, headline):
    """Time workload ``widx``: W warm-up steps, K timed steps between two events with
    nothing recorded in between, then K more steps with libkda's per-kernel events."""
    import torch
    import kda_inputs
    import gated_delta_rule_87_amd as kda

    dev = torch.device("cuda:0")
    w = kda_inputs.workload(widx)
    d = kda_inputs.make_inputs(w)
    x = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    w2 = kda_inputs.Workload(**{**w.__dict__, "seed": w.seed + 1})
    x2 = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in kda_inputs.make_inputs(w2).items()}
    sets = [x, x2]
    B, T, H = w.B, w.T, w.H
    tokens = B * T
    nseq = w.n_seqs
    out = torch.empty(B, T, H, 128, dtype=torch.bfloat16, device=dev)
    fin = None
    if w.final is not None:
        fin = torch.empty(nseq, H, 128, 128, dtype=torch.float32 if w.final == 'fp32' else torch.bfloat16,
                          device=dev)
    N = nseq if x['cu_seqlens'] is not None else 0
    ws = torch.empty(max(1, kda.workspace_size(B, T, H, N)), dtype=torch.uint8, device=dev)

    safe = args.gate == "safe"
    nstep = [0]

    def step():
        x = sets[nstep[0] & 1]
        nstep[0] += 1
        if args.path == "chunked":
            kda.fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out, x['A_log'], x['dt_bias'],
                    x['lower_bound'], initial_state=x['initial_state'], final_state=fin,
                    cu_seqlens=x['cu_seqlens'], workspace=ws, safe_gate=safe)
        else:
            kda.fwd_recurrent(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out, x['A_log'],
                              x['dt_bias'], x['lower_bound'], initial_state=x['initial_state'],
                              final_state=fin, cu_seqlens=x['cu_seqlens'], safe_gate=safe)

    settled_ms = settle_clocks(dev, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    span_ms = start.elapsed_time(end)
    ms_per_step = span_ms / args.steps
    call_ms = ms_per_step
    # per-kernel durations: a second pass of K steps with libkda's own events on the launch
    # stream around each kernel (kept out of the headline span above, whose steps have none)
    per_kernel = {}
    prof_ms = None
    if args.path == "chunked":
        kda.profile_start(args.steps)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        per_kernel = kda.profile_stop()
        prof_ms = e0.elapsed_time(e1) / args.steps

    state_in = state_out = 0
    if w.state is not None:
        state_in = nseq * H * 128 * 128 * (4 if w.state == 'fp32' else 2)
    if w.final is not None:
        state_out = nseq * H * 128 * 128 * (4 if w.final == 'fp32' else 2)
    alg_bytes = BYTES_PER_TOKEN_HEAD * tokens * H + state_in + state_out
    flops = FLOP_PER_TOKEN_HEAD * tokens * H
    achieved = alg_bytes / (call_ms * 1e-3) / 1e9
    if N:
        lens = [int(a) for a in w.lengths]
        chunks = sum((n + CHUNK - 1) // CHUNK for n in lens)
    else:
        chunks = B * ((T + CHUNK - 1) // CHUNK)
    rec_bytes = chunks * H * kda.record_bytes()
    alg = {"kda_sched_kernel": (0, 0),
           "kda_intra_kernel": (IN_BYTES_PER_TOKEN_HEAD * tokens * H, rec_bytes),
           "kda_chain_kernel": (OUT_BYTES_PER_TOKEN_HEAD * tokens * H + state_in + state_out, rec_bytes)}
    kernels = {}
    if args.path == "recurrent":   # one kernel per call: its time is the call's, on the same stream
        per_kernel = {"kda_recurrent_kernel": (call_ms * args.steps, args.steps)}
        alg["kda_recurrent_kernel"] = (alg_bytes, 0)
    for name, (tot_ms, launches) in per_kernel.items():
        if launches == 0 or name not in alg:
            continue
        ms = tot_ms / launches
        a, r = alg[name]
        kernels[name] = {"avg_ms": ms, "launches": launches, "alg_bytes": a, "alg_GBps": a / (ms * 1e-3) / 1e9,
                         "design_bytes": a + r, "design_GBps": (a + r) / (ms * 1e-3) / 1e9}
    res = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "T": T, "H": H, "K": 128, "V": 128,
                   "varlen_seqs": N or None, "initial_state": w.state, "final_state": w.final,
                   "lower_bound": w.lower_bound if safe else None, "gate": args.gate, "path": args.path},
    }
    if not headline:   # an extra workload: only what differs from the headline line
        res = {k: res[k] for k in ("value", "unit", "ms_per_step", "config")}
    if kernels:
        dom = max(kernels, key=lambda k: kernels[k]["avg_ms"])
        kd = kernels[dom]
        res["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": kd["alg_GBps"], "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": kd["alg_GBps"] / HBM_PEAK_GBS,
                           "traffic": recorded_traffic(w.name, dom) if safe else None,
                           "alg_bytes_per_launch": kd["alg_bytes"], "avg_launch_ms": kd["avg_ms"]}
    res["path"] = {"achieved_GBps": achieved, "frac_hbm": achieved / HBM_PEAK_GBS, "alg_bytes_per_call": alg_bytes,
                   "call_ms": call_ms, "input_sets": 2, "mfma_tflops": flops / (call_ms * 1e-3) / 1e12,
                   "frac_mfma_bf16": flops / (call_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
    if prof_ms is not None:
        res["path"]["profiled_call_ms"] = prof_ms
    res["clock_settle_ms"] = settled_ms
    res["kernels"] = kernels
    if headline:
        res["wall_s_timed"] = t_wall

    if headline and not args.no_cpu:
        from oracle import kda_oracle
        nthr = cpu_threads()
        t = time.perf_counter()
        kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'], d['dt_bias'],
                   d['lower_bound'], initial_state=d['initial_state'], cu_seqlens=d['cu_seqlens'],
                   want_final=True, nthreads=nthr, safe_gate=safe)
        dt = time.perf_counter() - t
        chains = nseq * H
        # one thread on one head, scaled to the whole workload
        t1 = time.perf_counter()
        kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'], d['dt_bias'],
                   d['lower_bound'], initial_state=d['initial_state'], cu_seqlens=d['cu_seqlens'],
                   heads=[0], want_final=True, nthreads=1, safe_gate=safe)
        dt1 = (time.perf_counter() - t1) * H
        try:
            affinity = len(os.sched_getaffinity(0))
        except AttributeError:
            affinity = None
        res["cpu_baseline"] = {
            "value": tokens / dt,
            "unit": "tokens/s",
            "cores": min(nthr, chains),
            "kind": "oracle",
            "sample": f"whole workload ({tokens} tokens x {H} heads, fp64, {min(nthr, chains)} OpenMP "
                      f"threads over {chains} independent chains), {dt:.2f} s",
            "one_thread_value": tokens / dt1,
            "one_thread_sample": f"head 0 of the same workload on one thread, {dt1 / H:.2f} s, scaled to {H} heads",
            "host": host_cpu_model(),
            "host_nproc": os.cpu_count(),
            "host_affinity_cpus": affinity,
            "threads_note": "OpenMP threads = OMP_NUM_THREADS if set, else min(16, affinity CPUs): a one-GPU "
                            "job's CPU share on the GPU host is 16 CPUs, whatever nproc shows",
        }
        res["gpu_over_cpu"] = res["value"] / res["cpu_baseline"]["value"]
    return res


if __name__ == "__main__":
    main()
