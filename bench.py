"""Benchmark of the verification step on one MI355X.

One step = one sdv_verify call (the row pass, then the per-request verdict kernel) over one ragged
batch whose inputs are already resident in HBM.  Default workload: B = 256 requests,
K_i ~ U{0..8}, V = 128256, bf16 logits, T = 1 (target ~ N(0, 3^2), draft = target + N(0, s_i^2),
s_i ~ U[0.5, 3]).  Independently drawn input sets rotate, enough of them for about 1 GB of inputs
(at least 2, at most 32), so that the 256 MB memory-side cache cannot serve a call from an earlier
one.

Prints one JSON line: verified draft positions per second (sum K_i per call / wall time per call),
the call's algorithmic HBM bandwidth, the row-pass kernel's roofline fraction (algorithmic bytes of
one launch / its mean duration from HIP events recorded on the library's stream), the bandwidth of
a plain read of the same size with the row pass's loads, per-call percentiles, accepted-length
statistics and the CPU oracle's rate on the host.

  python bench.py [--workload ragged_b256|greedy_b512|uniform_b64|small_b1|small_b1_v128256|
                              ragged_b256_profiled|ragged_b256_qrows|ragged_b256_topk50_topp900]
                  [--steps K] [--warmup W]

Profile summaries (rocprofv3 output -> text under profiles/):

  python bench.py --summarize-trace KERNEL_STATS_CSV --bench-json OUT --command "..."
  python bench.py --summarize-pmc FETCH_CSV WRITE_CSV --copy-mib 512 --command "..."
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
METRIC = "verified draft positions/sec and achieved HBM GB/s (% of peak) at B=256, V=128256"
KERNEL_SOURCES = ["lossless_draft_verification_online_amd/csrc/sdv.hip",
                  "lossless_draft_verification_online_amd/csrc/sdv_device.hpp",
                  "lossless_draft_verification_online_amd/csrc/split.hpp"]
KERNELS = ["row_records", "verdicts"]
TRUNCATION_KERNELS = ["row_records", "cuts", "verdicts"]  # "cuts": row_cuts_counted, then row_cuts
TRACE_KERNELS = ["row_records", "row_cuts_counted", "row_cuts", "tree_verdicts", "verdicts", "read_reg_kernel", "read_lds_kernel",
                 "read_strided_kernel", "philox_kernel"]
CHUNK_BYTES = 16384


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the kernels' code: line comments and blank lines are left out, so a profile stays
    valid across changes to comments alone (the sources hold no '//' inside a string literal)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        for line in open(os.path.join(ROOT, p), encoding="utf-8"):
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


WORKLOADS = ["ragged_b256", "greedy_b512", "uniform_b64", "small_b1", "small_b1_v128256", "ragged_b256_profiled",
             "ragged_b256_qrows", "ragged_b256_topk50_topp900", "tree_b64_v128256"]


def make_workload(name: str, set_index: int):
    import workloads as W
    if name == "ragged_b256":
        return W.ragged_b256(data_seed=W.DATA_SEED_BASE + 4 + 1000 * set_index, verify_seed=4000)
    if name == "greedy_b512":
        return W.greedy_b512(data_seed=W.DATA_SEED_BASE + 5 + 1000 * set_index, verify_seed=5000)
    if name == "uniform_b64":
        return W.uniform_b64(data_seed=W.DATA_SEED_BASE + 3 + 1000 * set_index, verify_seed=3000)
    if name == "small_b1":
        return W.small_b1(set_index)
    if name == "small_b1_v128256":
        return W.small_b1_v128256(data_seed=W.DATA_SEED_BASE + 8 + 1000 * set_index, verify_seed=8000)
    if name == "ragged_b256_qrows":  # the draft side as distributions (SDCP q_rows), float32
        return W.with_qrows(W.ragged_b256(data_seed=W.DATA_SEED_BASE + 4 + 1000 * set_index, verify_seed=4000))
    if name == "ragged_b256_topk50_topp900":  # top-k 50, then top-p 0.9, on every request
        return W.with_truncation(W.ragged_b256(data_seed=W.DATA_SEED_BASE + 4 + 1000 * set_index, verify_seed=4000),
                                 50, 900)
    if name == "ragged_b256_profiled":  # one sampling profile per request: a quarter greedy
        base = W.ragged_b256(data_seed=W.DATA_SEED_BASE + 4 + 1000 * set_index, verify_seed=4000)
        t, s = W.mixed_profiles(base.B, np.random.default_rng(W.DATA_SEED_BASE + 6 + set_index))
        return W.with_profiles(base, t, s, token_seed=W.DATA_SEED_BASE + 7 + set_index)
    if name == "tree_b64_v128256":  # token trees: 64 random trees of 8 to 24 nodes
        sizes = np.random.default_rng(W.DATA_SEED_BASE + 9 + 1000 * set_index).integers(8, 25, size=64)
        return W.make_tree("tree_b64_n8to24_v128256_bf16", sizes, "random", 128256, "bf16", 1.0, 3.0, 1.5,
                           data_seed=W.DATA_SEED_BASE + 10 + 1000 * set_index, verify_seed=9000, shared=True)
    raise SystemExit(f"unknown workload {name}")


def pmc_path(workload: str, kernel: str = "row_records") -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json")


def traffic_from_profile(workload: str, kernel: str = "row_records"):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; else None."""
    path = pmc_path(workload, kernel)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get(kernel, {}).get("traffic_bytes_per_launch")


def truncated_bytes(b) -> int:
    """Algorithmic bytes of the truncation kernel: every logit of every row it cuts, read once (the
    target and draft rows of each request that samples with a profile that truncates)."""
    if b.top_k is None:
        return 0
    T = b.temp_each if b.temp_each is not None else np.full(b.B, b.temperature)
    cuts = (T > 0) & (((b.top_k > 0) & (b.top_k < b.V)) | ((b.top_p_milli >= 0) & (b.top_p_milli < 1000)))
    rows = np.sum((b.depths + 1)[cuts]) + (0 if b.qrows is not None else np.sum(b.depths[cuts]))
    return int(rows) * b.V * b.elem_bytes


def oracle_profile(b):
    """(temperature, seed) as the oracle takes them: scalars, or one value per request."""
    if b.temp_each is not None:
        return b.temp_each.astype(np.float64), b.seed_each
    return b.temperature, b.seed


def oracle_options(b) -> dict:
    """The batch's other per-request inputs, as the oracle takes them."""
    kw = {}
    if b.qrows is not None:
        kw["draft_probs"] = b.qrows
    if b.top_k is not None:
        kw["top_k"], kw["top_p_milli"] = b.top_k, b.top_p_milli
    return kw


def cpu_baseline(batch, budget_s: float):
    """The oracle on all host threads (median of up to 3 calls), then once on a single thread."""
    from oracle import oracle

    def timed(budget):
        times = []
        t_end = time.perf_counter() + budget
        while True:
            t0 = time.perf_counter()
            if batch.parents is not None:
                oracle.verify_tree(batch.target, batch.draft, batch.tokens, batch.parents, batch.cu, batch.temperature,
                                   batch.seed, draft_row=batch.draft_row)
            else:
                oracle.verify(batch.target, batch.draft, batch.tokens, batch.cu, *oracle_profile(batch),
                              **oracle_options(batch))
            times.append(time.perf_counter() - t0)
            if len(times) >= 3 or time.perf_counter() > t_end:
                return float(np.median(times)), len(times)

    cores = oracle.num_threads()
    t, n = timed(budget_s)
    oracle.set_num_threads(1)
    t1, _ = timed(0.0)
    oracle.set_num_threads(cores)
    pos = int(batch.cu[-1])
    what = "nodes" if batch.parents is not None else "sum K_i"
    return {"value": pos / t, "unit": "positions/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} oracle calls on one full {batch.name} batch ({what} = {pos}), median "
                      f"{t * 1e3:.1f} ms per call, fp64 C with OpenMP",
            "single_thread_value": pos / t1}


def reread_bytes(batch, acc: np.ndarray) -> int:
    """Bytes the verdict kernel reads again beyond the algorithmic bytes: a correction re-reads its
    target and draft rows for the residual chunk masses and then one chunk of each for the search;
    a bonus re-reads one chunk of its target row; greedy terminals read nothing again."""
    sampling = batch.temp_each > 0 if batch.temp_each is not None else np.full(batch.B, batch.temperature > 0)
    K = batch.depths
    row = batch.V * batch.elem_bytes
    chunk = min(CHUNK_BYTES, row)
    resid = int(np.sum(sampling & (acc >= 0) & (acc < K)))
    bonus = int(np.sum(sampling & (acc == K)))
    if batch.qrows is not None:  # the q row of a correction is algorithmic; its target row is read again
        return resid * (row + chunk) + bonus * chunk
    return resid * (2 * row + 2 * chunk) + bonus * chunk


def qrow_bytes(batch, acc: np.ndarray) -> int:
    """Algorithmic bytes of the draft side when it comes as q rows: the row of every correction."""
    if batch.qrows is None:
        return 0
    K = batch.depths
    sampling = batch.temp_each > 0 if batch.temp_each is not None else np.full(batch.B, batch.temperature > 0)
    return int(np.sum(sampling & (acc >= 0) & (acc < K))) * batch.V * 4


def acceptance_stats(batch, accs):
    """Mean accepted length, committed tokens per call and the acceptance rate by depth
    (accepts at j / requests that reached j with a draft there; linear drafts only)."""
    K = batch.depths
    a = np.stack(accs)                      # calls x B
    ok = a >= 0
    committed = float(np.mean(np.sum(np.where(ok, a + 1, 0), axis=1)))
    by_depth = []
    for j in range(int(K.max()) if K.size and batch.parents is None else 0):
        reach = ok & (K[None, :] > j) & (a >= j)
        by_depth.append(float(np.sum(reach & (a > j)) / max(1, np.sum(reach))))
    return {"mean_accepted_len": float(np.mean(a[ok])), "committed_tokens_per_call": committed,
            "alpha_hat_by_depth": [round(x, 4) for x in by_depth], "calls": int(a.shape[0])}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="ragged_b256", choices=WORKLOADS)
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets rotated through the timed steps (0: enough for 1 GB, at least 2, at most 32)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle timing (0 = skip)")
    ap.add_argument("--no-check", action="store_true", help="skip the oracle comparison of one call")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--bench-json", help="bench output of the profiled run (for --summarize-trace)")
    ap.add_argument("--copy-mib", type=int, default=512, help="size of the calibration copy (--summarize-pmc)")
    ap.add_argument("--kernel", default="row_records", help="the kernel a counter summary is for (--summarize-pmc)")
    ap.add_argument("--command", default="", help="the command that produced the profile")
    ap.add_argument("--summary-name", default="", help="file name (no suffix) of a --summarize-trace summary")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph holding one step per input set (no host work between calls)")
    ap.add_argument("--yardsticks", action="store_true",
                    help="time the read yardsticks (three read shapes) and torch's fill_ at the workload's size")
    args = ap.parse_args()
    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_pmc:
        return summarize_pmc(args)
    if args.yardsticks:
        return yardsticks(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        raise SystemExit("bench.py measures one GPU: the verification step is built and measured on a single "
                         "MI355X. Requests are independent and would shard across GPUs by request with no "
                         "exchange, each GPU running this same step on its share; no multi-GPU figure is "
                         "produced.")

    import torch

    import lossless_draft_verification_online_amd as sdv
    from oracle.compare import compare_verdicts

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    first = make_workload(args.workload, 0)
    if args.sets <= 0:  # rotate past the 256 MB memory-side cache: about 1 GB of inputs in all
        per_set = first.target.nbytes + sum(x.nbytes for x in (first.draft, first.qrows) if x is not None)
        args.sets = int(min(32, max(2, -(-(1 << 30) // per_set))))
    log(f"[bench] generating {args.sets} input set(s) of {args.workload}")
    batches = [first] + [make_workload(args.workload, s) for s in range(1, args.sets)]

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
        if b.qrows is not None:
            sets[-1]["qrows"] = torch.from_numpy(b.qrows).to(dev)
        if b.temp_each is not None:  # one sampling profile per request, as device arrays
            sets[-1]["temp"] = torch.from_numpy(b.temp_each.astype(np.float32)).to(dev)
            sets[-1]["seeds"] = torch.from_numpy(b.seed_each.astype(np.uint64).view(np.int64)).to(dev)
        if b.top_k is not None:
            sets[-1]["top_k"] = torch.from_numpy(b.top_k).to(dev)
            sets[-1]["top_p_milli"] = torch.from_numpy(b.top_p_milli).to(dev)
        if b.parents is not None:
            sets[-1]["parents"] = torch.from_numpy(b.parents).to(dev)
            if b.draft_row is not None:
                sets[-1]["draft_row"] = torch.from_numpy(b.draft_row).to(dev)
    B0 = batches[0]
    tree = B0.parents is not None
    truncating = B0.top_k is not None
    kernels = TRUNCATION_KERNELS if truncating else KERNELS
    positions = [int(b.cu[-1]) for b in batches]
    rows = [int(b.cu[-1]) + b.B for b in batches]
    alg_bytes = [b.algorithmic_bytes() for b in batches]
    stream_bytes = list(alg_bytes)  # what the row pass reads: every row it streams, once
    ws = torch.empty(max(sdv.workspace_bytes(b.B, b.n_draft_rows, b.V, sets[0]["target"].dtype) for b in batches),
                     dtype=torch.uint8, device=dev)
    outs = [(torch.empty(b.B, dtype=torch.int32, device=dev),
             torch.empty(b.n_draft_rows + b.B, dtype=torch.int32, device=dev),
             torch.empty(b.n_draft_rows, dtype=torch.int32, device=dev)) for b in batches]

    def step(k, events=None):
        s = sets[k % len(sets)]
        b = s["batch"]
        temperature, seed = (s["temp"], s["seeds"]) if "temp" in s else (b.temperature, b.seed + k)
        if tree:
            sdv.verify_tree(s["target"], s["draft"], s["tokens"], s["parents"], s["cu"], temperature, seed,
                            draft_row=s.get("draft_row"), out=outs[k % len(sets)], workspace=ws, events=events)
            return
        sdv.verify_ex(s["target"], s["draft"], s["tokens"], s["cu"], temperature, seed,
                      out=outs[k % len(sets)][:2], workspace=ws, events=events, draft_probs=s.get("qrows"),
                      top_k=s.get("top_k"), top_p_milli=s.get("top_p_milli"))

    # correctness of the timed configuration, once, against the oracle
    parity = None
    if not args.no_check:
        from oracle import oracle
        log("[bench] checking one call against the oracle")
        step(0)
        torch.cuda.synchronize()
        if tree:
            from oracle.compare import compare_tree_verdicts
            ref = oracle.verify_tree(B0.target, B0.draft, B0.tokens, B0.parents, B0.cu, B0.temperature, B0.seed,
                                     diag=True, draft_row=B0.draft_row)
            cmp = compare_tree_verdicts(outs[0][0].cpu().numpy(), outs[0][1].cpu().numpy(), outs[0][2].cpu().numpy(),
                                        ref, B0.cu, B0.parents, B0.temperature)
        else:
            ref = oracle.verify(B0.target, B0.draft, B0.tokens, B0.cu, *oracle_profile(B0), diag=True,
                                **oracle_options(B0))
            cmp = compare_verdicts(outs[0][0].cpu().numpy(), outs[0][1].cpu().numpy(), ref, B0.cu,
                                   oracle_profile(B0)[0])
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

    if args.graph:  # one step per input set, captured once and replayed: every kernel of every step runs
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for k in range(len(sets)):
                step(k)
        torch.cuda.synchronize()
        replays = max(1, args.steps // len(sets))
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        log(f"[bench] timing {replays} replays of {len(sets)} steps")
        t0 = time.perf_counter()
        for _ in range(replays):
            graph.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        args.steps = replays * len(sets)
    else:
        log(f"[bench] timing {args.steps} steps")
        t0 = time.perf_counter()
        for k in range(args.steps):
            step(args.warmup + k)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0

    # a second pass with HIP events that the library records on its stream: [0] before the first
    # kernel, [1] after the row pass, [3] after the truncation kernel (when it runs), [2] after the
    # verdicts; per-kernel and per-call durations
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record()  # instantiate the handles
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(args.warmup + k, events=evs[k])
    torch.cuda.synchronize()
    order = [0, 1, 3, 2] if truncating else [0, 1, 2]
    per_kernel = [float(np.mean([evs[k][order[j]].elapsed_time(evs[k][order[j + 1]]) for k in range(args.steps)]))
                  for j in range(len(kernels))]
    per_call = np.array([evs[k][0].elapsed_time(evs[k][2]) for k in range(args.steps)])

    # the bandwidth yardstick: the row pass's loads with no arithmetic over buffers of the call's size
    n_chunks = int(np.mean(alg_bytes)) // CHUNK_BYTES
    bufs = [torch.empty(n_chunks * CHUNK_BYTES, dtype=torch.uint8, device=dev) for _ in range(len(sets))]
    for buf in bufs:
        buf.fill_(1)
    folded = torch.empty(n_chunks, dtype=torch.int32, device=dev)
    for k in range(10):
        sdv.read_ceiling(bufs[k % len(bufs)], folded)
    reps = 100
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record()
    for k in range(reps):
        sdv.read_ceiling(bufs[k % len(bufs)], folded)
    r1.record()
    torch.cuda.synchronize()
    read_gbps = n_chunks * CHUNK_BYTES / (r0.elapsed_time(r1) / reps * 1e-3) / 1e9
    del bufs

    # verdict statistics over a few more calls (untimed)
    accs, rereads, qbytes = [], [], [[] for _ in sets]
    for k in range(16):
        step(k)
        acc = outs[k % len(sets)][0].cpu().numpy()
        if k % len(sets) == 0:
            accs.append(acc)
        rereads.append(0 if tree else reread_bytes(batches[k % len(sets)], acc))
        qbytes[k % len(sets)].append(qrow_bytes(batches[k % len(sets)], acc))
    stats = acceptance_stats(B0, accs)
    if B0.qrows is not None:  # q rows read at the corrections are part of each call's algorithmic bytes
        alg_bytes = [a + int(np.mean(q)) if q else a for a, q in zip(alg_bytes, qbytes)]

    ms_step = elapsed * 1e3 / args.steps
    mean_pos = float(np.mean([positions[(args.warmup + k) % len(sets)] for k in range(args.steps)]))
    mean_rows = float(np.mean([rows[(args.warmup + k) % len(sets)] for k in range(args.steps)]))
    mean_bytes = float(np.mean([alg_bytes[(args.warmup + k) % len(sets)] for k in range(args.steps)]))
    mean_stream = float(np.mean([stream_bytes[(args.warmup + k) % len(sets)] for k in range(args.steps)]))
    value = mean_pos / (ms_step * 1e-3)
    call_gbps = mean_bytes / (ms_step * 1e-3) / 1e9
    rowpass_gbps = mean_stream / (per_kernel[0] * 1e-3) / 1e9
    # the roofline object describes the longest kernel with algorithmic bytes of its own: the row
    # pass, or the truncation kernel when it takes longer
    roof_kernel, roof_bytes, roof_ms = "row_records", mean_stream, per_kernel[0]
    if truncating and per_kernel[1] > per_kernel[0]:
        roof_bytes = float(np.mean([truncated_bytes(batches[(args.warmup + k) % len(sets)]) for k in range(args.steps)]))
        roof_kernel, roof_ms = "cuts", per_kernel[1]
    roof_gbps = roof_bytes / (roof_ms * 1e-3) / 1e9

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
        "config": {"workload": B0.name, "B": B0.B, "V": B0.V, "timing": "hip_graph_replay" if args.graph else "eager",
                   "temperature": B0.temperature if B0.temp_each is None else
                   {f"{t:g}": int(n) for t, n in zip(*np.unique(B0.temp_each, return_counts=True))},
                   **({} if B0.top_k is None else {"top_k": int(B0.top_k[0]), "top_p_milli": int(B0.top_p_milli[0]),
                                                    "drafts": "argmax of the draft row"}),
                   "sum_K_per_call": positions, "input_sets": len(sets),
                   "algorithmic_bytes_per_call": alg_bytes},
        "hbm_gbps": call_gbps,
        "hbm_frac_of_peak": call_gbps / PEAK_HBM_GBPS,
        "read_ceiling_gbps": read_gbps,
        "hbm_frac_of_read_ceiling": call_gbps / read_gbps,
        "rows_per_s": mean_rows / (ms_step * 1e-3),
        "committed_tokens_per_s": stats["committed_tokens_per_call"] / (ms_step * 1e-3),
        "call_ms_events": {"median": float(np.median(per_call)), "p5": float(np.percentile(per_call, 5)),
                           "p95": float(np.percentile(per_call, 95)), "n": int(per_call.size)},
        "kernel_ms": dict(zip(kernels, per_kernel)),
        "terminal_reread_bytes_per_call": None if tree else float(np.mean(rereads)),
        "terminal_reread_frac_of_algorithmic": None if tree else float(np.mean(rereads)) / mean_bytes,
        "acceptance": stats,
        "roofline": {"bound": "hbm", "achieved": roof_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": roof_gbps / PEAK_HBM_GBPS, "traffic": traffic_from_profile(args.workload, roof_kernel),
                     "kernel": roof_kernel, "algorithmic_bytes_per_launch": roof_bytes,
                     "frac_of_read_ceiling": roof_gbps / read_gbps,
                     "call_frac": call_gbps / PEAK_HBM_GBPS},
        "row_pass": {"achieved_gbps": rowpass_gbps, "frac": rowpass_gbps / PEAK_HBM_GBPS,
                     "algorithmic_bytes_per_launch": mean_stream},
        "parity": parity,
        "kernel_source_hash": kernel_source_hash(),
    }
    if args.cpu_budget > 0:
        log("[bench] timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(B0, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def yardsticks(args):
    """Reads with no arithmetic in three shapes (sdv_read_yardstick: 0 the row pass's loads, 1
    direct-to-LDS loads in two-wave workgroups, 2 a persistent grid with two chunks in flight per
    wave) and torch's fill_ (writes), each over two rotated buffers of the workload's algorithmic
    bytes; one JSON line of mean event times and rates."""
    import torch

    import lossless_draft_verification_online_amd as sdv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n_chunks = make_workload(args.workload, 0).algorithmic_bytes() // CHUNK_BYTES
    nbytes = n_chunks * CHUNK_BYTES
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(2)]
    for b in bufs:
        b.fill_(1)
    folded = torch.empty(n_chunks, dtype=torch.int32, device=dev)
    reps = max(args.steps, 10)
    out = {"yardsticks": args.workload, "bytes": nbytes, "reps": reps}
    runs = {f"read_shape{s}": (lambda k, s=s: sdv.read_ceiling(bufs[k % 2], folded, shape=s)) for s in range(3)}
    runs["torch_fill"] = lambda k: bufs[k % 2].fill_(k & 0xff)
    for name, fn in runs.items():
        for k in range(10):
            fn(k)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for k in range(reps):
            fn(k)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        out[name] = {"us": us, "gbps": nbytes / (us * 1e-6) / 1e9}
        log(f"[yardsticks] {name}: {us:.2f} us, {nbytes / (us * 1e-6) / 1e9:.0f} GB/s")
    print(json.dumps(out), flush=True)


# ----------------------------------------------------------------------------- profile summaries

def _short(name: str) -> str:
    for k in TRACE_KERNELS:  # longer names first where one name starts another
        if re.search(rf"(sdv{len(k)}{k}[EI])|(::{k}[(<])|(^{k}[(<])", name):
            return k
    return name.split("(")[0][:48]


def summarize_trace(args):
    """rocprofv3 --kernel-trace --stats kernel_stats.csv -> profiles/kernels_<workload>_trace.md."""
    rows = list(csv.DictReader(open(args.summarize_trace)))
    bench = None
    if args.bench_json and os.path.exists(args.bench_json):
        for line in open(args.bench_json):
            if line.startswith("{"):
                bench = json.loads(line)
                if "yardsticks" in bench:
                    bench["config"] = {"workload": f"read shapes at the size of {bench['yardsticks']}"}
    workload = bench["config"]["workload"] if bench else args.workload
    lines = [f"# Kernel durations: {workload}", "", "Command ($REPO is the repository root):", "", "```",
             args.command, "```", "",
             "| kernel | calls | total ms | mean us | min us | max us | share |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        n = int(r["Calls"])
        lines.append(f"| {_short(r['Name'])} | {n} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    if bench and "yardsticks" in bench:
        lines += ["", "The same run's event timings (mean per launch over two rotated buffers of "
                  f"{bench['bytes']} bytes):", ""]
        lines += [f"- {k}: {v['us']:.2f} us, {v['gbps']:.0f} GB/s" for k, v in bench.items() if isinstance(v, dict) and "us" in v]
        lines += ["", "Shapes: read_reg_kernel = shape 0 (the row pass's loads: one wave per 16 KiB chunk, 16 "
                  "non-temporal 16-byte loads per lane, four waves per workgroup); read_lds_kernel = shape 1 "
                  "(direct-to-LDS loads, two waves per workgroup); read_strided_kernel = shape 2 (a persistent "
                  "grid, two chunks in flight per wave); vectorized_elementwise_kernel = torch's fill_ (writes)."]
    elif bench:
        lines += ["", "The same run's bench line (HIP events on the library's stream):", "",
                  f"- kernel_ms: {json.dumps({k: round(v * 1e3, 2) for k, v in bench['kernel_ms'].items()})} (us)",
                  f"- ms_per_step: {bench['ms_per_step'] * 1e3:.2f} us; roofline frac of "
                  f"{bench['roofline'].get('kernel', 'row_records')}: {bench['roofline']['frac']:.4f}; "
                  f"kernel_source_hash {bench['kernel_source_hash']}"]
    out = os.path.join(ROOT, "profiles", f"{args.summary_name or f'kernels_{args.workload}_trace'}.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_pmc(args):
    """Two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) -> HBM bytes per launch,
    each counter scaled by what it reads for one plain device copy of --copy-mib MiB."""
    copy_kib = args.copy_mib * 1024

    def per_kernel(path, counter):
        vals, copies = {}, []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            name = r["Kernel_Name"]
            if "copyBuffer" in name:
                copies.append(v)
            else:
                vals.setdefault(_short(name), []).append(v)
        big = max(copies) if copies else 0.0
        if not (0.25 * copy_kib <= big <= 2.0 * copy_kib):
            raise SystemExit(f"{counter}: no calibration copy of about {copy_kib} KiB found (largest {big} KiB)")
        return {k: float(np.mean(v)) for k, v in vals.items()}, copy_kib / big, big

    fetch, f_fac, f_copy = per_kernel(args.summarize_pmc[0], "FETCH_SIZE")
    write, w_fac, w_copy = per_kernel(args.summarize_pmc[1], "WRITE_SIZE")
    batches = [make_workload(args.workload, s) for s in range(2)]
    kern = args.kernel
    alg = float(np.mean([truncated_bytes(b) if kern == "row_cuts" else b.algorithmic_bytes() for b in batches]))
    rec = {"kernel_source_hash": kernel_source_hash(), "workload": args.workload, "command": args.command,
           "calibration": {"copy_bytes": copy_kib * 1024, "fetch_kib_read": f_copy, "write_kib_read": w_copy,
                           "fetch_factor": f_fac, "write_factor": w_fac},
           f"algorithmic_bytes_per_{kern}_launch": alg}
    lines = [f"# HBM traffic per launch: {args.workload}", "", "Commands ($REPO is the repository root):", "",
             "```", args.command, "```", "",
             f"Calibration: a {args.copy_mib} MiB device copy reads FETCH_SIZE {f_copy:.0f} KiB "
             f"(factor {f_fac:.3f}) and WRITE_SIZE {w_copy:.0f} KiB (factor {w_fac:.3f}).", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched bytes (scaled) | written bytes (scaled) |",
             "|---|---|---|---|---|"]
    for k in sorted(set(fetch) | set(write)):
        fb = fetch.get(k, 0.0) * 1024 * f_fac
        wb = write.get(k, 0.0) * 1024 * w_fac
        rec[k] = {"fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb, "traffic_bytes_per_launch": fb + wb}
        lines.append(f"| {k} | {fetch.get(k, 0):.0f} | {write.get(k, 0):.0f} | {fb:.4g} | {wb:.4g} |")
    if kern in rec:
        lines += ["", f"{kern}: traffic {rec[kern]['traffic_bytes_per_launch']:.4g} B against "
                      f"{alg:.4g} algorithmic bytes per launch "
                      f"(ratio {rec[kern]['traffic_bytes_per_launch'] / alg:.4f})."]
    json.dump(rec, open(pmc_path(args.workload, kern), "w"), indent=1)
    out = os.path.join(ROOT, "profiles", f"{kern}_{args.workload}_pmc.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
