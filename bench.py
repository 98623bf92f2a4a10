#!/usr/bin/env python3
"""Throughput of the chunked KDA forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1] [--no-cpu]

A step is one kda_fwd call (the whole hot path: varlen scheduler when
cu_seqlens is given, intra-chunk kernel, state-chain/output kernel) over one
batch of synthetic inputs already resident in HBM. The default workload is the
fixed-length prefill B=1, T=8192, H=64, K=V=128 (bf16 inputs, stateless,
fp32 final state). Prints ONE JSON line.

  value       tokens/s = tokens per step / mean step time (HIP events)
  roofline    whole-call HBM roofline: algorithmic bytes per call / mean call
              duration against 8 TB/s; algorithmic bytes = 1,282 B per
              token-head (q, k, v, g, beta, out) + 64 KiB per fp32 state read
              or written per (sequence, head); "traffic" is the measured HBM
              bytes per call from rocprofv3 FETCH_SIZE/WRITE_SIZE (recorded in
              profiles/traffic.json for a given kernel-source hash; null when the
              kernels changed since)
  cpu_baseline the fp64 CPU oracle timed on the host cores over the same
              workload (bounded: see "sample")
"""
import argparse
import hashlib
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


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_87_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload_name):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = rec.get(workload_name)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_call")


def cpu_threads():
    n = os.environ.get("OMP_NUM_THREADS")
    if n and n.isdigit():
        return int(n)
    try:
        return min(16, len(os.sched_getaffinity(0)))
    except AttributeError:
        return min(16, os.cpu_count() or 1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=1, help="workload index (kda_inputs.workload)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--path", choices=["chunked", "recurrent"], default="chunked")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU (asked for --gpus {args.gpus}); "
              "multi-GPU sharding is design-only here", file=sys.stderr)
        sys.exit(2)

    import torch
    import kda_inputs
    import gated_delta_rule_87_amd as kda

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = kda_inputs.workload(args.workload)
    d = kda_inputs.make_inputs(w)
    x = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
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

    def step():
        if args.path == "chunked":
            kda.fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out, x['A_log'], x['dt_bias'],
                    x['lower_bound'], initial_state=x['initial_state'], final_state=fin,
                    cu_seqlens=x['cu_seqlens'], workspace=ws)
        else:
            kda.fwd_recurrent(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out, x['A_log'],
                              x['dt_bias'], x['lower_bound'], initial_state=x['initial_state'],
                              final_state=fin, cu_seqlens=x['cu_seqlens'])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    per_call_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    span_ms = starts[0].elapsed_time(ends[-1])
    ms_per_step = span_ms / args.steps
    call_ms = sum(per_call_ms) / len(per_call_ms)

    state_bytes = 0
    sbytes = 4 if (w.state == 'fp32' or w.final == 'fp32') else 2
    if w.state is not None:
        state_bytes += nseq * H * 128 * 128 * sbytes
    if w.final is not None:
        state_bytes += nseq * H * 128 * 128 * (4 if w.final == 'fp32' else 2)
    alg_bytes = BYTES_PER_TOKEN_HEAD * tokens * H + state_bytes
    flops = FLOP_PER_TOKEN_HEAD * tokens * H
    achieved = alg_bytes / (call_ms * 1e-3) / 1e9
    traffic = recorded_traffic(w.name)
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
                   "lower_bound": w.lower_bound, "path": args.path},
        "roofline": {
            "kernel": "kda_fwd (all kernels of one call)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "alg_bytes_per_call": alg_bytes,
            "call_ms": call_ms,
            "mfma_tflops": flops / (call_ms * 1e-3) / 1e12,
            "mfma_frac": flops / (call_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        },
        "wall_s_timed": t_wall,
    }

    if not args.no_cpu:
        import numpy as np
        from oracle import kda_oracle
        nthr = cpu_threads()
        t = time.perf_counter()
        kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'], d['dt_bias'],
                   d['lower_bound'], initial_state=d['initial_state'], cu_seqlens=d['cu_seqlens'],
                   want_final=True, nthreads=nthr)
        dt = time.perf_counter() - t
        chains = nseq * H
        res["cpu_baseline"] = {
            "value": tokens / dt,
            "unit": "tokens/s",
            "cores": min(nthr, chains),
            "kind": "oracle",
            "sample": f"whole workload ({tokens} tokens x {H} heads, fp64, {min(nthr, chains)} OpenMP "
                      f"threads over {chains} independent chains), {dt:.2f} s",
        }
        res["gpu_over_cpu"] = res["value"] / res["cpu_baseline"]["value"]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
