"""Benchmark: batched lossless draft verification on one MI355X.

One step = one verification call (the whole hot path: streaming row
statistics, per-request decisions, residual/bonus sampling) over one batch.
The default workload is the chain workload bs=64, k=7, V=128256, bf16 target
logits, half the requests greedy and half at T=0.8 with fp32 draft
probabilities; --workload picks the others (chain_small, chain_fp32,
onehot_bf16, tree_fp32).  Inputs are resident in HBM before the timed
region; the timed steps rotate over several input sets whose total size
exceeds the 256 MB Infinity Cache, so the stream really comes from HBM.

The call is two stream-ordered kernels: the row-statistics pass (streams
every logit row once; the dominant kernel) and the decision/sampling pass;
--top-k / --top-p add the thresholds pass between them (and, for top-k, the
statistics pass also keeps the candidate groups), --rule block the residual
pass.  The first phase is always the statistics pass alone; the second
phase holds the rest.  Three timed passes:
  1. throughput: K plain calls between two events -> value, ms_per_step;
  2. kernels: the same K calls, split into their two phases
     (FLAG_STATS_ONLY, FLAG_DECIDE_ONLY) and grouped by input set: the
     row-statistics launches of all sets between one event pair, then their
     decision launches between the next (each set has its own workspace)
     -> each kernel's mean launch duration;
  3. read ceiling: sv_stream_read over the same sets' logit buffers (the
     row-statistics pass's bytes, access pattern and rotation) at a few grid
     sizes -> the attainable read bandwidth of the chip for this stream.
`roofline` is the row-statistics kernel (its algorithmic bytes / its launch
time, against the 8 TB/s HBM peak), with `roofline.call` for the whole call
(all its algorithmic bytes over the call time, and over the sum of its
kernels' times; HBM bytes by counters over the kernels' times when a counter
record of this kernel source is committed) and `pct_of_ceiling`.

Prints one JSON line, with the acceptance statistics of the timed inputs and
the oracle timed on the host (one core, and sharded by request over the
host's cores) as a CPU baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
WORKLOADS = {
    "chain_small": "chain verify bs=1 k=3 V=1000, fp32 target logits, T=1, fp32 draft probs (launch-bound)",
    "chain_fp32": "chain verify bs=8 k=3 V=128256, fp32 target logits, T=1, fp32 draft probs",
    "chain_bf16_mixed": "chain verify bs=64 k=7 V=128256, bf16 target logits, half greedy, half T=0.8 with fp32 draft probs",
    "onehot_bf16": "one-hot (target-only) chain verify bs=256 k=3 V=151936, bf16 target logits, T=1",
    "tree_fp32": "target-only tree verify bs=48 N=8 (5 steps x top-4 topology) V=128256, fp32 target logits, T=1",
}
# grid sizes of the read-ceiling stream (workgroups of 256 threads)
CEILING_GRIDS = (1024, 1536, 2048, 4096, 8192)
KERNEL_SOURCE = os.path.join(ROOT, "lossless_draft_verification_amd", "csrc", "specverify.hip")


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def filter_bytes(inp, top_k, top_p):
    """Bytes the top-k / top-p thresholds must move beyond the statistics
    pass: the logits of a filtered row are already counted there (one pass
    can keep what the thresholds need), so only each filtered row's 16-byte
    record (rows 0..k_b of each stochastic request, when a filter is on)."""
    bs, R, V = inp.logits.shape
    k = R - 1
    if not ((0 < top_k < V) or (0.0 < top_p < 1.0)):
        return 0
    ids = inp.draft_ids
    kb = np.where((ids == -1).any(axis=1), np.argmax(ids == -1, axis=1), k) if k else np.zeros(bs, np.int64)
    stoch = (inp.temperature > 0) & np.isfinite(inp.temperature)
    return int(((kb + 1) * stoch).sum() * 16)


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


def tree_algorithmic_bytes(inp, accept_len):
    """Bytes a tree call must move, from the actual outcomes, split by
    phase.  Row statistics: every node's logit row once (all N rows are
    read), the gather of each node's token logit in its parent's row, the
    temperature.  Decision/sampling: per-request scalars (temperature, seed,
    parents, node tokens), the re-read of the one sampled row per stochastic
    request (p with the tried children removed, or the bonus p: no q), and
    the outputs (accept_len, accept_path, tokens, status)."""
    bs, N, V = inp.logits.shape
    bl = inp.logits.dtype.itemsize
    stoch = (inp.temperature > 0) & np.isfinite(inp.temperature)
    stats = decide = 0
    for b in range(bs):
        stats += N * V * bl + (N - 1) * (bl + 4 + 4) + 4
        decide += 4 + 8 + 8 * N
        if stoch[b]:
            decide += V * bl
        decide += 4 + 8 * N + 4
    return int(stats), int(decide)


def load_traffic(workload: str, kernels, top_k=0, top_p=1.0):
    """HBM bytes per launch of `kernels` (one name, or several whose bytes
    add) measured with rocprofv3 counters for this kernel source (committed
    under profiles/), or None if there is no record or the kernels changed
    since the counters were taken."""
    path = traffic_name(workload, top_k, top_p)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    total = 0
    for k in ([kernels] if isinstance(kernels, str) else kernels):
        b = rec.get("kernels", {}).get(k, {}).get("bytes_per_launch")
        if b is None:
            return None
        total += b
    return total


def _pmc_per_dispatch(db_path, counter):
    """Mean value of `counter` per dispatch of each kernel in a rocprofv3
    results database."""
    import sqlite3
    import collections

    con = sqlite3.connect(db_path)
    q = """select ks.kernel_name, ip.name, pe.value, kd.id from rocpd_pmc_event pe
           join rocpd_info_pmc ip on pe.pmc_id = ip.id
           join rocpd_event ev on pe.event_id = ev.id
           join rocpd_kernel_dispatch kd on kd.event_id = ev.id
           join rocpd_info_kernel_symbol ks on kd.kernel_id = ks.id"""
    tot = collections.defaultdict(float)
    disp = collections.defaultdict(set)
    for kname, cname, value, did in con.execute(q):
        if cname == counter:
            tot[kname] += value
            disp[kname].add(did)
    return {k: tot[k] / len(disp[k]) for k in tot}


def _library_kernel(name):
    """Short name of a library kernel from a profiler's kernel name, mangled
    (_ZN2sv9kf_kernel...) or not (void sv::kf_kernel<true>(sv::Params)); None
    for other kernels."""
    m = re.match(r"_ZN(?:2sv|3svp)(\d+)", name)
    if m:
        n = int(m.group(1))
        return name[m.end():m.end() + n]
    if name.startswith("_ZN12_GLOBAL__N_118stream_read_kernel"):
        return "stream_read_kernel"
    m = re.match(r"(?:void )?(?:sv|svp)::(\w+)", name)
    if m:
        return m.group(1)
    return "stream_read_kernel" if name.startswith("(anonymous namespace)::stream_read_kernel") else None


def traffic_name(workload, top_k=0, top_p=1.0):
    """profiles/ file of a workload's counter record (filtered calls apart)."""
    tag = "" if not ((top_k and top_k > 0) or top_p < 1.0) else f"_topk{top_k}_topp{top_p:g}"
    return os.path.join(ROOT, "profiles", f"traffic_{workload}{tag}.json")


def write_traffic(workload, fetch_db, write_db, copy_fetch_db, copy_write_db, top_k=0, top_p=1.0):
    """Write profiles/traffic_<workload>[_topk.._topp..].json from four
    rocprofv3 --pmc runs: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the
    benchmark, and of a plain device copy of known size (bench.py
    --copy-calibration-mib 1024), whose counts scale the kernels' to bytes.
    Every kernel of the library in the run is recorded."""
    copy_bytes = 1024 << 20

    def pick(d, name):
        vals = [v for k, v in d.items() if name in k]
        if not vals:
            raise SystemExit(f"no dispatch of {name} in the database")
        return vals[0]

    cf = pick(_pmc_per_dispatch(copy_fetch_db, "FETCH_SIZE"), "copyBuffer")
    cw = pick(_pmc_per_dispatch(copy_write_db, "WRITE_SIZE"), "copyBuffer")
    ff, wf = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    fetch = _pmc_per_dispatch(fetch_db, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_db, "WRITE_SIZE")
    rec = {"workload": WORKLOADS[workload], "top_k": top_k, "top_p": top_p,
           "kernel_source_sha256_16": kernel_source_hash(),
           "calibration": {"copy_bytes": copy_bytes, "fetch_size_kib": cf, "write_size_kib": cw,
                           "fetch_factor": ff, "write_factor": wf},
           "kernels": {}}
    for full in sorted(fetch):
        k = _library_kernel(full)
        if k is None or k in rec["kernels"]:
            continue
        fk, wk = pick(fetch, full), pick(write, full)
        rec["kernels"][k] = {"fetch_size_kib_per_dispatch": round(fk, 1), "write_size_kib_per_dispatch": round(wk, 1),
                             "fetch_bytes_per_launch": int(round(fk * 1024 * ff)),
                             "bytes_per_launch": int(round(fk * 1024 * ff + wk * 1024 * wf))}
    path = traffic_name(workload, top_k, top_p)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def positions_of(inp):
    """Verified draft positions of one call: sum of k_b (chain) or N - 1 per
    request (tree)."""
    if hasattr(inp, "parent"):
        return int(inp.batch * (inp.num_nodes - 1))
    return int((inp.draft_ids >= 0).cumprod(axis=1).sum()) if inp.max_draft else 0


def _oracle_call(inp, lo, hi, rule, filt):
    """The oracle on requests [lo, hi) of one input set (slices along the
    batch axis are contiguous views; the oracle's C loop runs without the
    interpreter lock)."""
    import oracle

    f = {k: v[lo:hi] for k, v in filt.items()}
    if hasattr(inp, "parent"):
        return oracle.verify_tree(inp.logits[lo:hi], inp.node_tokens[lo:hi], inp.parent[lo:hi],
                                  inp.temperature[lo:hi], inp.seeds[lo:hi], **f)
    return oracle.verify_chain(inp.logits[lo:hi], inp.draft_ids[lo:hi], inp.temperature[lo:hi], inp.seeds[lo:hi],
                               draft_probs=None if inp.draft_probs is None else inp.draft_probs[lo:hi],
                               onehot=inp.onehot, rule=rule, **f)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inputs, seconds: float, threads: int, rule: str = "standard", top_k: int = 0, top_p: float = 1.0):
    """The oracle timed on the host on full calls of input set 0: on one
    core, then sharded by request over `threads` threads (each thread runs
    the unchanged oracle on a contiguous slice of the batch).  Also returns
    the oracle's decision count and near-tie (margin < 1e-6) requests of
    that set."""
    from concurrent.futures import ThreadPoolExecutor

    inp = inputs[0]
    bs = inp.batch
    filt = {}
    if top_k or top_p != 1.0:
        filt = dict(top_k=np.full(bs, top_k, np.int32), top_p=np.full(bs, top_p, np.float32))
    positions = positions_of(inp)
    ref = _oracle_call(inp, 0, bs, rule, filt)
    margins = {"decisions": int(ref["n_decisions"].sum()),
               "near_tie_requests": int(((ref["min_margin"] < 1e-6) & (ref["status"] == 0)).sum())}
    calls = 0
    t0 = time.perf_counter()
    while True:
        _oracle_call(inp, 0, bs, rule, filt)
        calls += 1
        el1 = time.perf_counter() - t0
        if el1 >= seconds:
            break
    one = positions * calls / el1
    nt = max(1, min(threads, bs))
    bounds = [(i * bs // nt, (i + 1) * bs // nt) for i in range(nt)]
    calls_n = 0
    with ThreadPoolExecutor(max_workers=nt) as ex:
        t0 = time.perf_counter()
        while True:
            list(ex.map(lambda lh: _oracle_call(inp, lh[0], lh[1], rule, filt), bounds))
            calls_n += 1
            eln = time.perf_counter() - t0
            if eln >= seconds:
                break
    many = positions * calls_n / eln
    return ({"value": many, "unit": "positions/s", "cores": nt, "kind": "oracle", "cpu_model": cpu_model(),
             "host_cpu_count": os.cpu_count(),
             "sample": f"{calls_n} full calls of the same workload (input set 0), the C oracle sharded by request "
                       f"over {nt} threads, {eln:.1f} s",
             "single_core": {"value": one, "unit": "positions/s", "cores": 1,
                             "sample": f"{calls} full calls, single-threaded, {el1:.1f} s"}},
            margins)


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
    """Latency of one survival top-k plan (two launches: slot ranks over
    many workgroups, then the prefix sums, ratios and admitted counts in
    one): the page's adaptive-verification shape (512 requests x 7
    positions, half with accurate drafts) and the largest supported one
    (1024 x 8)."""
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
        # descriptor built once: the loop below enqueues launches only, so the
        # events see back-to-back kernels, not Python's per-call set-up
        plan = sv.PreparedPlan(c, cost, float(bs))
        for _ in range(args.warmup):
            plan.launch()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        stream = torch.cuda.current_stream(dev)
        e0.record(stream)
        for _ in range(args.steps):
            plan.launch()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        lines.append({"batch": bs, "K": K, "slots": n, "us_per_plan": us,
                      "budget": int(plan.out["budget"].item())})
    print(json.dumps({"metric": "survival top-k draft budget latency, 1 MI355X", "value": lines[0]["us_per_plan"],
                      "unit": "us/plan", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "higher_is_better": False, "data": "synthetic",
                      "config": {"workload": "plan 512 requests x 7 positions (and 1024 x 8)", "cases": lines},
                      "roofline": {"bound": "latency", "note": "a few thousand slots ranked over many workgroups, then one workgroup"}}), flush=True)


def read_ceiling(sv, torch, dev, buffers, steps):
    """Attainable read bandwidth for the row-statistics pass's stream: the
    same buffers (one per input set, rotated), each launch reading one whole
    buffer with sv_stream_read, at each grid size of CEILING_GRIDS.
    Returns (best GB/s, its grid, {grid: GB/s}, bytes per launch)."""
    sink = torch.zeros(max(CEILING_GRIDS), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    nbytes = [b.numel() * b.element_size() for b in buffers]
    per = {}
    for g in CEILING_GRIDS:
        for i in range(len(buffers)):
            sv.stream_read(buffers[i], sink, g)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            sv.stream_read(buffers[i % len(buffers)], sink, g)
        e1.record(stream)
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3
        per[g] = sum(nbytes[i % len(buffers)] for i in range(steps)) / sec / 1e9
    best = max(per, key=per.get)
    return per[best], best, per, float(np.mean(nbytes))


def acceptance_stats(outs, inputs, tree):
    """Acceptance of the timed inputs, from the GPU's outputs: drafts
    accepted at each position (the per-position counter the zoo page names
    for vLLM), the mean accepted length, and tokens per round (accepted + the
    emitted one)."""
    acc = np.concatenate([o["accept_len"] for o in outs])
    ok = np.concatenate([o["status"] for o in outs]) == 0
    stoch = np.concatenate([(i.temperature > 0) & np.isfinite(i.temperature) for i in inputs])
    R = inputs[0].logits.shape[1]
    depth = R - 1
    hist = [int(((acc > i) & ok).sum()) for i in range(depth)]

    def summary(sel):
        if not sel.any():
            return None
        return {"requests": int(sel.sum()), "mean_accepted": float(acc[sel].mean()),
                "mean_tokens_per_round": float(acc[sel].mean() + 1.0),
                "accepted_per_position": [int(((acc > i) & sel).sum()) for i in range(depth)]}

    return {"calls": len(outs), "accepted_per_position": hist, "mean_accepted": float(acc[ok].mean()),
            "mean_tokens_per_round": float(acc[ok].mean() + 1.0),
            "stochastic": summary(ok & stoch), "greedy": summary(ok & ~stoch),
            "note": "positions are tree depths" if tree else "positions are draft indices"}


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
    ap.add_argument("--kf-rows", action="store_true",
                    help="top-k thresholds from passes over the rows instead of the statistics pass's candidates")
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="seconds of each oracle timing (one core, all)")
    ap.add_argument("--cpu-threads", type=int, default=16,
                    help="threads of the sharded oracle timing (capped by the host's cores and the batch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--schedule", choices=["auto", "phased", "fused"], default="auto",
                    help="library schedule (auto: the library's default for the shape)")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="only measure the attainable read bandwidth (sv_stream_read) over the workload's "
                         "logit buffers and print its line")
    ap.add_argument("--compact", action="store_true",
                    help="time accepted-path KV compaction (sv_compact_kv) after tree verification instead")
    ap.add_argument("--plan", action="store_true",
                    help="time the survival top-k draft budget (sv_plan_budget) instead and print its line")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB a few times (the "
                         "reference kernel for scaling HBM byte counters) and exit")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB", "COPY_WRITE_DB"),
                    help="write profiles/traffic_<workload>.json from four rocprofv3 --pmc result databases "
                         "(no GPU needed) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the verification hot path runs on a single MI355X here; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.traffic_from:
        write_traffic(args.workload, *args.traffic_from, top_k=args.top_k, top_p=args.top_p)
        return

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
    tree = args.workload.startswith("tree")
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

    if args.read_ceiling:
        bufs = [to_dev(inp.logits) for inp in inputs]
        gbs, grid, per, nb = read_ceiling(sv, torch, dev, bufs, args.steps)
        print(json.dumps({"metric": "attainable HBM read bandwidth (sv_stream_read), 1 MI355X", "value": gbs,
                          "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "higher_is_better": True,
                          "data": "synthetic",
                          "config": {"workload": WORKLOADS[args.workload] + ": its logit buffers, one per launch",
                                     "bytes_per_launch": nb, "buffers": len(bufs), "best_grid": grid,
                                     "gbs_by_grid": {str(k): v for k, v in per.items()}},
                          "frac_of_peak": gbs / HBM_PEAK_GBS, "us_per_launch": nb / (gbs * 1e3)}), flush=True)
        return

    flags = {"auto": 0, "phased": sv.FLAG_PHASED, "fused": sv.FLAG_FUSED}[args.schedule]
    block = args.rule == "block"
    if block:
        if tree:
            raise SystemExit("the block rule is defined for chains only")
        flags |= sv.FLAG_BLOCK
    if args.kf_rows:
        flags |= sv.FLAG_KF_ROWS
    V0 = inputs[0].vocab
    filtered = (0 < args.top_k < V0) or (0.0 < args.top_p < 1.0)
    if filtered and args.schedule == "fused":
        raise SystemExit("top-k / top-p filtering needs the phased schedule")
    calls = []
    for inp in inputs:
        fk = fp = None
        if filtered:
            # a filter that is off for every request is not passed at all
            if 0 < args.top_k < inp.vocab:
                fk = torch.full((inp.batch,), args.top_k, dtype=torch.int32, device=dev)
            if 0.0 < args.top_p < 1.0:
                fp = torch.full((inp.batch,), args.top_p, dtype=torch.float32, device=dev)
        dl, dt, ds = to_dev(inp.logits), to_dev(inp.temperature), to_dev(inp.seeds)
        if tree:
            dn, dp = to_dev(inp.node_tokens), to_dev(inp.parent)
            mk = lambda f, w, k=None, p=None: sv.PreparedTree(dl, dn, dp, dt, ds, flags=f, workspace=w, top_k=k,
                                                              top_p=p)
        else:
            di, dq = to_dev(inp.draft_ids), to_dev(inp.draft_probs)
            mk = lambda f, w, k=None, p=None: sv.PreparedChain(dl, di, dt, ds, draft_probs=dq, onehot=inp.onehot,
                                                               flags=f, workspace=w, top_k=k, top_p=p)
        calls.append(mk(flags, sv.Workspace(1 << 20, dev), fk, fp))
    resident = sum(c.logits.numel() * c.logits.element_size()
                   + (c.q.numel() * 4 if getattr(c, "q", None) is not None else 0) for c in calls)
    stream = torch.cuda.current_stream(dev)
    # algorithmic bytes of each set, from its outcome; the outcomes' acceptance
    alg, outs = [], []
    for c, inp in zip(calls, inputs):
        c.launch()
        torch.cuda.synchronize()
        if (c.out["status"] != 0).any():
            raise RuntimeError("a request reported a non-OK status on the benchmark inputs")
        out = {n: t.cpu().numpy() for n, t in c.out.items()}
        outs.append(out)
        if tree:
            alg.append(tree_algorithmic_bytes(inp, out["accept_len"]) + (0,))
        else:
            alg.append(algorithmic_bytes(inp, out["accept_len"], block)
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
    positions = [positions_of(inp) for inp in inputs]

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
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(groups)]
    torch.cuda.synchronize()
    for g in range(groups):
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
    filt_bytes = np.array([a[2] for a in alg] * groups, dtype=np.float64)
    second_ms = np.array([e[1].elapsed_time(e[2]) for e in ev]) / S if split else None
    stats_bytes = np.array([a[0] for a in alg] * groups, dtype=np.float64)
    decide_bytes = np.array([a[1] for a in alg] * groups, dtype=np.float64)
    # top-k calls' statistics pass also keeps the candidate groups; bf16
    # calls with top-p and no top-k take the thresholds from value counts
    cand = filtered and 0 < args.top_k <= 128 and args.top_k < V0 and not args.kf_rows
    bf16_logits = inputs[0].logits.dtype == np.uint16
    thr_name = "kft_kernel" if (filtered and bf16_logits and not 0 < args.top_k < V0) else "kf_kernel"
    if split:
        kernel = "row statistics with top-k candidates (k1f_kernel)" if cand else "row statistics (k1_kernel)"
        kbytes = stats_bytes
    else:
        kernel = "fused verify (fused_kernel)"
        kbytes = stats_bytes + decide_bytes
    achieved = kbytes.sum() / (first_ms.sum() * S * 1e-3) / 1e9

    # pass 3: the attainable read bandwidth of the same stream
    gbs_ceiling, grid_ceiling, ceiling_by_grid, _ = read_ceiling(sv, torch, dev, [c.logits for c in calls], K)

    # the whole call
    call_bytes = (stats_bytes + decide_bytes + filt_bytes).mean()
    call_us = total_ms * 1e3 / K
    kernel_us = float(first_ms.mean() * 1e3 + (second_ms.mean() * 1e3 if split else 0.0))
    k1_name = ("k1f_kernel" if cand else "k1_kernel") if split else "fused_kernel"
    tk, tp = (args.top_k, args.top_p) if filtered else (0, 1.0)
    traffic = None if block else load_traffic(args.workload, k1_name, tk, tp)
    rest = ([thr_name] if filtered else []) + ["k23_kernel"]
    traffic23 = None if (block or not split) else load_traffic(args.workload, rest, tk, tp)
    call = {
        "kernels": (f"{k1_name} + k23_kernel" if split else "fused_kernel")
                   + (f" + {thr_name}" if filtered else "") + (" + kr_kernel" if block else ""),
        "algorithmic_bytes": float(call_bytes),
        "us_per_call": call_us,
        "achieved_gbs_by_call_time": call_bytes / (call_us * 1e3),
        "frac_by_call_time": call_bytes / (call_us * 1e3) / HBM_PEAK_GBS,
        "kernel_us_sum": kernel_us,
        "achieved_gbs_by_kernel_time": call_bytes / (kernel_us * 1e3),
        "frac_by_kernel_time": call_bytes / (kernel_us * 1e3) / HBM_PEAK_GBS,
    }
    if traffic is not None and (traffic23 is not None or not split):
        hbm = traffic + (traffic23 or 0)
        call["hbm_bytes_by_counters"] = hbm
        call["hbm_gbs_by_kernel_time"] = hbm / (kernel_us * 1e3)
        call["hbm_frac_by_kernel_time"] = hbm / (kernel_us * 1e3) / HBM_PEAK_GBS
    line = {
        "metric": "verified draft positions/sec and achieved HBM GB/s (% of peak), 1 MI355X",
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": total_ms / K,
        "us_per_call": call_us,
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
            ("nodes" if tree else "k"): int(inputs[0].num_nodes if tree else inputs[0].max_draft),
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
            "ceiling_gbs": gbs_ceiling,
            "ceiling_grid": grid_ceiling,
            "ceiling_gbs_by_grid": {str(k): v for k, v in ceiling_by_grid.items()},
            "pct_of_ceiling": 100.0 * achieved / gbs_ceiling,
            "call": call,
        },
        "acceptance": acceptance_stats(outs, inputs, tree),
    }
    line["roofline"]["call"]["pct_of_ceiling_by_kernel_time"] = 100.0 * call["achieved_gbs_by_kernel_time"] / gbs_ceiling
    if split:
        line["roofline"]["other_kernel"] = {
            "kernel": ("residual masses, decisions and sampling (kr_kernel + k23_kernel)" if block
                       else f"filter thresholds, decisions and sampling ({thr_name} + k23_kernel)" if filtered
                       else "decisions and sampling (k23_kernel)"),
            "algorithmic_bytes_per_launch": float((decide_bytes + filt_bytes).mean()),
            "launch_us_mean": float(second_ms.mean() * 1e3),
            "achieved": float((decide_bytes + filt_bytes).sum() / (second_ms.sum() * S * 1e-3) / 1e9),
            "traffic": traffic23,
        }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        base, margins = cpu_baseline(inputs, args.cpu_seconds, args.cpu_threads, args.rule,
                                     args.top_k if filtered else 0, args.top_p if filtered else 1.0)
        line["cpu_baseline"] = base
        line["acceptance"]["oracle_set0"] = margins
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
