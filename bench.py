"""Benchmark of the verification step on one MI355X.

One step = one sdv_verify call (row pass, accept scan, terminal draw) over one ragged batch whose
inputs are already resident in HBM.  Default workload: B = 256 requests, K_i ~ U{0..8},
V = 128256, bf16 logits, T = 1 (target ~ N(0, 3^2), draft = target + N(0, s_i^2), s_i ~ U[0.5, 3]).
Two independently drawn input sets (about 1.2 GB together) alternate so that the memory-side
cache cannot serve a call from the previous one.

Prints one JSON line: verified draft positions per second (sum K_i per call / time per call), the
call's algorithmic HBM bandwidth, the row-pass kernel's roofline fraction (algorithmic bytes of
one launch / its mean duration from HIP events recorded on the library's stream), and the CPU
oracle's rate on the host.
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

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
METRIC = "verified draft positions/sec and achieved HBM GB/s (% of peak) at B=256, V=128256"
KERNEL_SOURCES = ["lossless_draft_verification_online_amd/csrc/sdv.hip",
                  "lossless_draft_verification_online_amd/csrc/sdv_device.hpp"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def make_workload(name: str, set_index: int):
    import workloads as W
    if name == "ragged_b256":
        return W.ragged_b256(data_seed=W.DATA_SEED_BASE + 4 + 1000 * set_index, verify_seed=4000)
    if name == "greedy_b512":
        return W.greedy_b512(data_seed=W.DATA_SEED_BASE + 5 + 1000 * set_index, verify_seed=5000)
    if name == "uniform_b64":
        return W.uniform_b64(data_seed=W.DATA_SEED_BASE + 3 + 1000 * set_index, verify_seed=3000)
    raise SystemExit(f"unknown workload {name}")


def traffic_from_profile(workload: str):
    """HBM bytes per row_records launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"row_records_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_baseline(batch, budget_s: float):
    from oracle import oracle
    times = []
    t_end = time.perf_counter() + budget_s
    while True:
        t0 = time.perf_counter()
        oracle.verify(batch.target, batch.draft, batch.tokens, batch.cu, batch.temperature, batch.seed)
        times.append(time.perf_counter() - t0)
        if len(times) >= 3 or time.perf_counter() > t_end:
            break
    t = float(np.median(times))
    pos = int(batch.cu[-1])
    return {"value": pos / t, "unit": "positions/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{len(times)} oracle calls on one full {batch.name} batch (sum K_i = {pos}), median "
                      f"{t * 1e3:.1f} ms per call, fp64 C with OpenMP"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="ragged_b256", choices=["ragged_b256", "greedy_b512", "uniform_b64"])
    ap.add_argument("--sets", type=int, default=2, help="input sets rotated through the timed steps")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle timing (0 = skip)")
    ap.add_argument("--no-check", action="store_true", help="skip the oracle comparison of one call")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        raise SystemExit("bench.py measures one GPU: the verification step is built and measured on a single "
                         "MI355X; requests shard across GPUs with no exchange (see the design notes), and "
                         "no multi-GPU figure is produced.")

    import torch

    import lossless_draft_verification_online_amd as sdv
    from oracle.compare import compare_verdicts

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] generating {args.sets} input set(s) of {args.workload}")
    batches = [make_workload(args.workload, s) for s in range(args.sets)]

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    sets = []
    for b in batches:
        sets.append(dict(target=up(b.target), draft=up(b.draft), tokens=torch.from_numpy(b.tokens).to(dev),
                         cu=torch.from_numpy(b.cu).to(dev), batch=b))
    B0 = batches[0]
    positions = [int(b.cu[-1]) for b in batches]
    alg_bytes = [b.algorithmic_bytes() for b in batches]
    ws = torch.empty(max(sdv.workspace_bytes(b.B, b.n_draft_rows, b.V, sets[0]["target"].dtype) for b in batches),
                     dtype=torch.uint8, device=dev)
    outs = [(torch.empty(b.B, dtype=torch.int32, device=dev),
             torch.empty(b.n_draft_rows + b.B, dtype=torch.int32, device=dev)) for b in batches]

    def step(k, events=None):
        s = sets[k % len(sets)]
        b = s["batch"]
        sdv.verify_ex(s["target"], s["draft"], s["tokens"], s["cu"], b.temperature, b.seed + k,
                      out=outs[k % len(sets)], workspace=ws, events=events)

    # correctness of the timed configuration, once, against the oracle
    parity = None
    if not args.no_check:
        from oracle import oracle
        log("[bench] checking one call against the oracle")
        step(0)
        torch.cuda.synchronize()
        ref = oracle.verify(B0.target, B0.draft, B0.tokens, B0.cu, B0.temperature, B0.seed, diag=True)
        cmp = compare_verdicts(outs[0][0].cpu().numpy(), outs[0][1].cpu().numpy(), ref, B0.cu, B0.temperature)
        parity = {"requests": cmp["requests"], "hard_mismatches": cmp["n_hard"], "near_tie_excused": cmp["n_excused"]}
        if cmp["n_hard"]:
            raise SystemExit(f"GPU verdicts differ from the oracle: {cmp['hard'][:5]}")

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    log(f"[bench] warmup {args.warmup} steps")
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + k)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # a second pass with HIP events that the library records on its stream before the first kernel
    # and after each kernel: per-kernel durations for the roofline
    greedy = B0.temperature == 0
    n_kernels = 2
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_kernels + 1)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record()  # instantiate the handles
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(args.warmup + k, events=evs[k])
    torch.cuda.synchronize()
    per_kernel = [float(np.mean([evs[k][j].elapsed_time(evs[k][j + 1]) for k in range(args.steps)]))
                  for j in range(n_kernels)]
    ms_step = elapsed * 1e3 / args.steps
    mean_pos = float(np.mean([positions[(args.warmup + k) % len(sets)] for k in range(args.steps)]))
    mean_bytes = float(np.mean([alg_bytes[(args.warmup + k) % len(sets)] for k in range(args.steps)]))
    value = mean_pos / (ms_step * 1e-3)
    call_gbps = mean_bytes / (ms_step * 1e-3) / 1e9
    rowpass_gbps = mean_bytes / (per_kernel[0] * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if B0.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": B0.name, "B": B0.B, "V": B0.V, "temperature": B0.temperature,
                   "sum_K_per_call": positions, "input_sets": len(sets),
                   "algorithmic_bytes_per_call": alg_bytes},
        "hbm_gbps": call_gbps,
        "hbm_frac_of_peak": call_gbps / PEAK_HBM_GBPS,
        "kernel_ms": dict(zip(["row_records", "verdicts"], per_kernel)),
        "roofline": {"bound": "hbm", "achieved": rowpass_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": rowpass_gbps / PEAK_HBM_GBPS, "traffic": traffic_from_profile(args.workload),
                     "kernel": "row_records", "algorithmic_bytes_per_launch": mean_bytes},
        "parity": parity,
        "kernel_source_hash": kernel_source_hash(),
    }
    if args.cpu_budget > 0:
        log("[bench] timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(B0, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
