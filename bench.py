"""Benchmark: batched lossless draft verification on one MI355X.

One step = one sv_verify_chain call (the whole hot path: streaming row
statistics, per-request decisions, residual/bonus sampling) over one batch
of the chain workload bs=64, k=7, V=128256, bf16 target logits, half the
requests greedy and half at T=0.8 with fp32 draft probabilities.  Inputs
are resident in HBM before the timed region; the timed steps rotate over
several input sets whose total size exceeds the 256 MB Infinity Cache, so
the stream really comes from HBM.

The call is two stream-ordered kernels: the row-statistics pass (streams
every logit row once; the dominant kernel) and the decision/sampling pass.
Two timed passes over the same K steps:
  1. throughput: K plain calls between two events -> value, ms_per_step;
  2. kernels: the same K calls, split into their two phases
     (FLAG_STATS_ONLY, FLAG_DECIDE_ONLY) and grouped by input set: the
     row-statistics launches of all sets between one event pair, then their
     decision launches between the next (each set has its own workspace)
     -> each kernel's mean launch duration, and the roofline of the
     row-statistics kernel (its algorithmic bytes / that duration, against
     the 8 TB/s HBM peak).
The fused schedule is one launch; there the roofline covers the whole call.

Prints one JSON line, with the oracle timed on the host as a CPU baseline.
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

HBM_PEAK_GBS = 8000.0
WORKLOADS = {
    "chain_bf16_mixed": "chain verify bs=64 k=7 V=128256, bf16 target logits, half greedy, half T=0.8 with fp32 draft probs",
    "chain_fp32": "chain verify bs=8 k=3 V=128256, fp32 target logits, T=1, fp32 draft probs",
    "onehot_bf16": "one-hot (target-only) chain verify bs=256 k=3 V=151936, bf16 target logits, T=1",
}
KERNEL_SOURCE = os.path.join(ROOT, "lossless_draft_verification_amd", "csrc", "specverify.hip")


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def filter_bytes(inp, top_k, top_p):
    """Bytes the top-k / top-p thresholds must move at least: one read of
    every filtered row (rows 0..k_b of each stochastic request, when a filter
    is on) and its 16-byte record."""
    bs, R, V = inp.logits.shape
    k = R - 1
    if not ((0 < top_k < V) or (0.0 < top_p < 1.0)):
        return 0
    bl = inp.logits.dtype.itemsize
    ids = inp.draft_ids
    kb = np.where((ids == -1).any(axis=1), np.argmax(ids == -1, axis=1), k) if k else np.zeros(bs, np.int64)
    stoch = (inp.temperature > 0) & np.isfinite(inp.temperature)
    return int(((kb + 1) * stoch).sum() * (V * bl + 16))


def algorithmic_bytes(inp, accept_len, block=False):
    """Bytes the method must move for one call, from the actual outcomes,
    split by phase.  Row statistics: every read logit row (rows 0..k_b of
    each request) once, the gathers at the draft ids (logit, id, q value)
    and the temperature.  Decision/sampling: per-request scalars, the
    re-read of the one sampled row per stochastic request (its logits, plus
    its q row after a rejection), and the outputs; under the block rule
    with draft probabilities also the residual-mass pass over target and q
    rows 1..k_b-1 of each stochastic request.  Returns (stats_bytes,
    decide_bytes)."""
    bs, R, V = inp.logits.shape
    k = R - 1
    bl = inp.logits.dtype.itemsize
    ids = inp.draft_ids
    kb = np.where((ids == -1).any(axis=1), np.argmax(ids == -1, axis=1), k) if k else np.zeros(bs, np.int64)
    stoch = (inp.temperature > 0) & np.isfinite(inp.temperature)
    stats = decide = 0
    for b in range(bs):
        stats += (kb[b] + 1) * V * bl                                         # streamed rows
        stats += kb[b] * (bl + 4 + (0 if inp.onehot else 4))                  # gathers at the draft ids
        stats += 4                                                            # temperature
        decide += 4 + 8 + 4 * k                                               # temperature, seed, ids
        if stoch[b]:
            reject = accept_len[b] < kb[b]
            decide += V * bl + (V * 4 if (reject and not inp.onehot) else 0)  # sampled row (+ q row)
            if block and not inp.onehot and kb[b] >= 2:
                decide += (kb[b] - 1) * V * (bl + 4)                          # residual masses
        decide += 4 + 4 * R + 4                                               # accept_len, tokens, status
    return int(stats), int(decide)


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` measured with rocprofv3 counters for
    this kernel source (committed under profiles/), or None if there is no
    record or the kernel changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("kernels", {}).get(kernel, {}).get("bytes_per_launch")


def cpu_baseline(inputs, seconds: float, rule: str = "standard", top_k: int = 0, top_p: float = 1.0):
    import oracle

    inp = inputs[0]
    bs = inp.batch
    filt = {}
    if top_k or top_p != 1.0:
        filt = dict(top_k=np.full(bs, top_k, np.int32), top_p=np.full(bs, top_p, np.float32))
    positions = int((inp.draft_ids >= 0).cumprod(axis=1).sum()) if inp.max_draft else 0
    calls = 0
    t0 = time.perf_counter()
    while True:
        oracle.verify_chain(inp.logits, inp.draft_ids, inp.temperature, inp.seeds, draft_probs=inp.draft_probs,
                            onehot=inp.onehot, rule=rule, **filt)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": positions * calls / el, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} full calls of the same workload (input set 0), single-threaded C oracle, "
                      f"{el:.1f} s"}


def bench_compact(args, sv, torch, dev, workloads):
    """Accepted-path KV compaction on a Llama-3-8B-shaped pool: 32 layers,
    one 4 KB row per token and layer (8 KV heads x 128 x K and V, bf16), the
    nodes' slots a random permutation.  Two cases of 48 requests x 8 nodes:
    the accepted paths of the GPU tree verification of the tree workload's
    input sets (few rows move: most accepted nodes are already in place),
    and every request accepting 4 nodes off the first-child chain (path
    2, 4, 6, 7: 4 rows move).  Descriptors are built once, so the timed
    loop is launches only.  Algorithmic bytes: every moved row read once and
    written once; the roofline line is the second case."""
    import ctypes

    from lossless_draft_verification_amd import _lib

    rng = np.random.default_rng(23)
    layers, row = 32, 4096
    bs, N = 48, 8
    kv = torch.zeros((layers, bs * N, row), dtype=torch.uint8, device=dev)
    stream = _lib._stream(dev)

    def prepared(al, ap, sl):
        moved = torch.empty(bs, dtype=torch.int32, device=dev)
        keep = (al, ap, sl, moved)
        d = _lib.CompactDesc(bs, N, al.data_ptr(), ap.data_ptr(), sl.data_ptr(), kv.data_ptr(), layers, bs * N,
                             row, bs * N * row, row, moved.data_ptr())
        return d, keep

    cases = {}
    verified = []
    for s_i in range(args.sets):
        t = workloads.tree_fp32(s_i)
        out = sv.verify_tree(torch.from_numpy(t.logits).to(dev), torch.from_numpy(t.node_tokens).to(dev),
                             torch.from_numpy(t.parent).to(dev), torch.from_numpy(t.temperature).to(dev),
                             torch.from_numpy(t.seeds.view(np.int64)).to(dev))
        sl = torch.from_numpy(rng.permutation(bs * N).reshape(bs, N).astype(np.int64)).to(dev)
        verified.append(prepared(out["accept_len"].contiguous(), out["accept_path"].contiguous(), sl))
    cases["verified"] = verified
    moved_all = []
    for s_i in range(args.sets):
        al = torch.full((bs,), 4, dtype=torch.int32, device=dev)
        ap = torch.tensor([[2, 4, 6, 7, -1, -1, -1, -1]] * bs, dtype=torch.int32, device=dev)
        sl = torch.from_numpy(rng.permutation(bs * N).reshape(bs, N).astype(np.int64)).to(dev)
        moved_all.append(prepared(al, ap, sl))
    cases["all_moved"] = moved_all
    L = _lib.lib()
    res = {}
    for name, preps in cases.items():
        rows = []
        for d, keep in preps:
            assert L.sv_compact_kv(ctypes.byref(d), stream) == 0
            torch.cuda.synchronize()
            rows.append(int(keep[3].clamp(min=0).sum().item()))
        for i in range(args.warmup):
            L.sv_compact_kv(ctypes.byref(preps[i % len(preps)][0]), stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = torch.cuda.current_stream(dev)
        e0.record(ts)
        for i in range(args.steps):
            L.sv_compact_kv(ctypes.byref(preps[i % len(preps)][0]), stream)
        e1.record(ts)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        alg = float(np.mean([rows[i % len(preps)] for i in range(args.steps)]) * layers * row * 2)
        res[name] = {"us_per_call": us, "moved_rows_per_layer": rows, "algorithmic_bytes": alg,
                     "gb_per_s": alg / (us * 1e-6) / 1e9}
    r = res["all_moved"]
    print(json.dumps({"metric": "accepted-path KV compaction, 1 MI355X", "value": r["us_per_call"], "unit": "us/call",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False,
                      "data": "synthetic",
                      "config": {"workload": "KV compaction, 48 requests x 8 nodes, 32 layers x 4 KB rows",
                                 "cases": res},
                      "roofline": {"bound": "hbm", "achieved": r["gb_per_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": r["gb_per_s"] / HBM_PEAK_GBS, "traffic": None, "kernel": "compact_kernel",
                                   "algorithmic_bytes_per_launch": r["algorithmic_bytes"],
                                   "launch_us_mean": r["us_per_call"]}}), flush=True)


def bench_plan(args, sv, torch, dev):
    """Latency of one survival top-k plan (a single-workgroup kernel): the
    page's adaptive-verification shape (512 requests x 7 positions, half
    with accurate drafts) and the largest supported one (1024 x 8)."""
    rng = np.random.default_rng(11)
    lines = []
    for bs, K in ((512, 7), (1024, 8)):
        level = np.where(np.arange(bs)[:, None] < bs // 2, 0.9, 0.55)
        conf = np.minimum(level * (0.9 + 0.2 * rng.random((bs, K))), 0.99).astype(np.float32)
        n = bs * K
        # the pages' step-cost model: weights read once, compute-bound beyond
        step = np.maximum(16e9 / (3.35e12 * 0.8), (bs + np.arange(n + 1)) * 16e9 / (989e12 * 0.5))
        cost = torch.from_numpy(0.25e-3 + step).to(dev)
        c = torch.from_numpy(conf).to(dev)
        for _ in range(args.warmup):
            sv.plan_budget(c, cost, float(bs))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        stream = torch.cuda.current_stream(dev)
        e0.record(stream)
        for _ in range(args.steps):
            out = sv.plan_budget(c, cost, float(bs))
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        lines.append({"batch": bs, "K": K, "slots": n, "us_per_plan": us, "budget": int(out["budget"].item())})
    print(json.dumps({"metric": "survival top-k draft budget latency, 1 MI355X", "value": lines[0]["us_per_plan"],
                      "unit": "us/plan", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "higher_is_better": False, "data": "synthetic",
                      "config": {"workload": "plan 512 requests x 7 positions (and 1024 x 8)", "cases": lines},
                      "roofline": {"bound": "latency", "note": "one workgroup; a few thousand slots"}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="chain_bf16_mixed", choices=sorted(WORKLOADS))
    ap.add_argument("--sets", type=int, default=4, help="input sets rotated over the timed steps")
    ap.add_argument("--rule", choices=["standard", "block"], default="standard",
                    help="acceptance rule of the stochastic requests (block: block verification)")
    ap.add_argument("--top-k", type=int, default=0,
                    help="top-k filtering of every stochastic request's target (0: off)")
    ap.add_argument("--top-p", type=float, default=1.0,
                    help="top-p filtering of every stochastic request's target (1: off)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--schedule", choices=["auto", "phased", "fused"], default="auto",
                    help="library schedule (auto: the library's default for the shape)")
    ap.add_argument("--compact", action="store_true",
                    help="time accepted-path KV compaction (sv_compact_kv) after tree verification instead")
    ap.add_argument("--plan", action="store_true",
                    help="time the survival top-k draft budget (sv_plan_budget) instead and print its line")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB a few times (the "
                         "reference kernel for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the verification hot path runs on a single MI355X here; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration_mib:
        dev = torch.device("cuda", 0)
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.zeros_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)
        return

    import lossless_draft_verification_amd as sv
    import workloads

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.plan:
        bench_plan(args, sv, torch, dev)
        return
    if args.compact:
        bench_compact(args, sv, torch, dev, workloads)
        return
    gen = getattr(workloads, args.workload)
    print(f"[bench] generating {args.sets} input sets of {args.workload}", file=sys.stderr, flush=True)
    inputs = [gen(s) for s in range(args.sets)]

    def to_dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        if a.dtype == np.uint64:
            return torch.from_numpy(a.view(np.int64)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    flags = {"auto": 0, "phased": sv.FLAG_PHASED, "fused": sv.FLAG_FUSED}[args.schedule]
    block = args.rule == "block"
    if block:
        flags |= sv.FLAG_BLOCK
    V0 = inputs[0].vocab
    filtered = (0 < args.top_k < V0) or (0.0 < args.top_p < 1.0)
    if filtered and args.schedule == "fused":
        raise SystemExit("top-k / top-p filtering needs the phased schedule")
    calls, plain_calls = [], []
    for inp in inputs:
        dl, di, dt, ds = to_dev(inp.logits), to_dev(inp.draft_ids), to_dev(inp.temperature), to_dev(inp.seeds)
        dq = to_dev(inp.draft_probs)
        fk = fp = None
        if filtered:
            fk = torch.full((inp.batch,), args.top_k, dtype=torch.int32, device=dev)
            fp = torch.full((inp.batch,), args.top_p, dtype=torch.float32, device=dev)
            # the same call without the filter: its statistics pass alone, for timing
            plain_calls.append(sv.PreparedChain(dl, di, dt, ds, draft_probs=dq, onehot=inp.onehot, flags=flags,
                                                workspace=sv.Workspace(1 << 20, dev)))
        calls.append(sv.PreparedChain(dl, di, dt, ds, draft_probs=dq, onehot=inp.onehot, flags=flags,
                                      workspace=sv.Workspace(1 << 20, dev), top_k=fk, top_p=fp))
    resident = sum(c.logits.numel() * c.logits.element_size() + (c.q.numel() * 4 if c.q is not None else 0)
                   for c in calls)
    stream = torch.cuda.current_stream(dev)
    # algorithmic bytes of each set, from its outcome
    alg = []
    for c, inp in zip(calls, inputs):
        c.launch()
        torch.cuda.synchronize()
        if (c.out["status"] != 0).any():
            raise RuntimeError("a request reported a non-OK status on the benchmark inputs")
        alg.append(algorithmic_bytes(inp, c.out["accept_len"].cpu().numpy(), block)
                   + (filter_bytes(inp, args.top_k, args.top_p),))
        if args.schedule != "fused":
            # the split phases must reproduce the plain call
            ref = {n: t.clone() for n, t in c.out.items()}
            for t in c.out.values():
                t.fill_(-7)
            c.launch(phase_flag=sv.FLAG_STATS_ONLY)
            c.launch(phase_flag=sv.FLAG_DECIDE_ONLY)
            torch.cuda.synchronize()
            if any(not torch.equal(ref[n], c.out[n]) for n in ref):
                raise RuntimeError("split-phase call differs from the plain call")
    positions = [int((inp.draft_ids >= 0).cumprod(axis=1).sum()) for inp in inputs]

    for i in range(args.warmup):
        calls[i % len(calls)].launch()
    torch.cuda.synchronize()

    K = args.steps
    # pass 1: throughput of plain calls
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        calls[i % len(calls)].launch()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    pos_total = sum(positions[i % len(calls)] for i in range(K))
    value = pos_total / (total_ms * 1e-3)

    # pass 2: per-kernel durations; events on the launch stream around each
    # group of one phase's launches over all input sets
    split = args.schedule != "fused"
    S = len(calls)
    groups = max(1, K // S)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(groups)]
    torch.cuda.synchronize()
    for g in range(groups):
        if filtered:
            # the statistics pass alone (the unfiltered call's first phase)
            ev[g][3].record(stream)
            for c in plain_calls:
                c.launch(phase_flag=sv.FLAG_STATS_ONLY)
        ev[g][0].record(stream)
        if split:
            for c in calls:
                c.launch(phase_flag=sv.FLAG_STATS_ONLY)
            ev[g][1].record(stream)
            for c in calls:
                c.launch(phase_flag=sv.FLAG_DECIDE_ONLY)
        else:
            for c in calls:
                c.launch()
            ev[g][1].record(stream)
        ev[g][2].record(stream)
    torch.cuda.synchronize()
    first_ms = np.array([e[0].elapsed_time(e[1]) for e in ev]) / S
    k1_ms = np.array([e[3].elapsed_time(e[0]) for e in ev]) / S if filtered else None
    filt_bytes = np.array([a[2] for a in alg] * groups, dtype=np.float64)
    second_ms = np.array([e[1].elapsed_time(e[2]) for e in ev]) / S if split else None
    stats_bytes = np.array([a[0] for a in alg] * groups, dtype=np.float64)
    decide_bytes = np.array([a[1] for a in alg] * groups, dtype=np.float64)
    if split and filtered:
        # the first phase is the statistics pass then the thresholds pass;
        # the roofline covers the statistics pass timed alone
        kf_ms = first_ms - k1_ms
        first_ms = k1_ms
        kernel = "row statistics (k1_kernel)"
        kbytes = stats_bytes
    elif split:
        kernel = "row statistics (k1_kernel)"
        kbytes = stats_bytes
    else:
        kernel = "fused verify (fused_kernel)"
        kbytes = stats_bytes + decide_bytes
    achieved = kbytes.sum() / (first_ms.sum() * S * 1e-3) / 1e9
    traffic = None if (block or filtered) else load_traffic(args.workload, "k1_kernel" if split else "fused_kernel")
    line = {
        "metric": "verified draft positions/sec and achieved HBM GB/s (% of peak), 1 MI355X",
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": total_ms / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": WORKLOADS[args.workload] + (", block verification" if block else "")
                        + (f", target filtered top-k {args.top_k} top-p {args.top_p}" if filtered else ""),
            "rule": args.rule,
            "batch": int(inputs[0].batch),
            "k": int(inputs[0].max_draft),
            "vocab": int(inputs[0].vocab),
            "logits_dtype": "bf16" if inputs[0].logits.dtype == np.uint16 else "f32",
            "positions_per_step": positions[0],
            "input_sets": len(calls),
            "resident_input_bytes": int(resident),
            "schedule": args.schedule,
            "top_k": args.top_k,
            "top_p": args.top_p,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "kernel": kernel,
            "algorithmic_bytes_per_launch": float(kbytes.mean()),
            "launch_us_mean": float(first_ms.mean() * 1e3),
            "launch_us_p50": float(np.median(first_ms) * 1e3),
        },
    }
    if split:
        line["roofline"]["other_kernel"] = {
            "kernel": ("residual masses, decisions and sampling (kr_kernel + k23_kernel)" if block
                       else "decisions and sampling (k23_kernel)"),
            "algorithmic_bytes_per_launch": float(decide_bytes.mean()),
            "launch_us_mean": float(second_ms.mean() * 1e3),
            "achieved": float(decide_bytes.sum() / (second_ms.sum() * S * 1e-3) / 1e9),
        }
    if split and filtered:
        line["roofline"]["filter_kernel"] = {
            "kernel": "top-k / top-p thresholds (kf_kernel)",
            "algorithmic_bytes_per_launch": float(filt_bytes.mean()),
            "launch_us_mean": float(kf_ms.mean() * 1e3),
            "achieved": float(filt_bytes.sum() / (kf_ms.sum() * S * 1e-3) / 1e9),
            "timing": "first phase minus the statistics pass timed alone",
        }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(inputs, args.cpu_seconds, args.rule,
                                            args.top_k if filtered else 0, args.top_p if filtered else 1.0)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
