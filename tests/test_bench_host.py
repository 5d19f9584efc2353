"""Host checks of the benchmark's byte accounting (no GPU): the algorithmic
bytes that the roofline divides by a kernel's time, on tiny hand-counted
inputs."""
import numpy as np

import bench
import workloads


def _inputs(bf16, onehot):
    bs, k, V = 3, 2, 10
    l = np.zeros((bs, k + 1, V), np.float32)
    logits = workloads.f32_to_bf16_bits(l) if bf16 else l
    ids = np.array([[1, 2], [3, -1], [4, 5]], np.int32)        # k_b = 2, 1, 2
    q = None if onehot else np.full((bs, k, V), 0.1, np.float32)
    temp = np.array([0.0, 1.0, 0.7], np.float32)              # request 0 greedy
    return workloads.ChainInputs(logits, ids, q, temp, np.arange(bs, dtype=np.uint64), onehot, "tiny")


def test_algorithmic_bytes_by_hand():
    inp = _inputs(bf16=True, onehot=False)
    accept = np.array([2, 0, 1], np.int32)                    # request 1 rejects, request 2 rejects at 1
    stats, decide = bench.algorithmic_bytes(inp, accept)
    V, bl, R, k = 10, 2, 3, 2
    kb = [2, 1, 2]
    want_stats = sum((kb[b] + 1) * V * bl + kb[b] * (bl + 4 + 4) + 4 for b in range(3))
    want_decide = 3 * (4 + 8 + 4 * k) + 3 * (4 + 4 * R + 4)
    want_decide += 2 * (V * bl + V * 4)                       # two stochastic requests, both rejected
    assert stats == want_stats and decide == want_decide
    # block rule: residual masses of rows 1..k_b-1 of the stochastic requests with k_b >= 2
    _, decide_blk = bench.algorithmic_bytes(inp, accept, block=True)
    assert decide_blk == want_decide + (2 - 1) * V * (bl + 4)


def test_algorithmic_bytes_onehot_reads_no_q():
    inp = _inputs(bf16=False, onehot=True)
    accept = np.array([2, 0, 2], np.int32)
    stats, decide = bench.algorithmic_bytes(inp, accept)
    V, bl = 10, 4
    kb = [2, 1, 2]
    assert stats == sum((kb[b] + 1) * V * bl + kb[b] * (bl + 4) + 4 for b in range(3))
    assert decide == 3 * (4 + 8 + 8) + 3 * (4 + 12 + 4) + 2 * V * bl


def test_filter_bytes_counts_the_filtered_rows_records():
    inp = _inputs(bf16=True, onehot=False)
    assert bench.filter_bytes(inp, 0, 1.0) == 0               # no filter
    assert bench.filter_bytes(inp, 10, 1.0) == 0              # k >= V is off
    # stochastic requests 1 and 2 read rows 0..1 and 0..2: 5 rows
    # the rows' logits belong to the statistics pass; only the records remain
    assert bench.filter_bytes(inp, 3, 1.0) == 5 * 16
    assert bench.filter_bytes(inp, 0, 0.9) == 5 * 16


def test_tree_algorithmic_bytes_by_hand():
    bs, N, V = 2, 4, 10
    logits = np.zeros((bs, N, V), np.float32)
    tok = np.array([[0, 1, 2, 3], [0, 4, 5, 6]], np.int32)
    par = np.array([[-1, 0, 0, 1], [-1, 0, 1, 2]], np.int32)
    temp = np.array([1.0, 0.0], np.float32)                   # request 1 greedy
    inp = workloads.TreeInputs(logits, tok, par, temp, np.arange(bs, dtype=np.uint64), "tiny tree")
    stats, decide = bench.tree_algorithmic_bytes(inp, np.array([1, 3], np.int32))
    bl = 4
    assert stats == bs * (N * V * bl + (N - 1) * (bl + 8) + 4)
    assert decide == bs * (4 + 8 + 8 * N) + V * bl + bs * (4 + 8 * N + 4)


def test_positions_of_chains_and_trees():
    inp = _inputs(bf16=False, onehot=True)
    assert bench.positions_of(inp) == 2 + 1 + 2
    t = workloads.tree_fp32(0, bs=3, N=5, V=64)
    assert bench.positions_of(t) == 3 * 4
