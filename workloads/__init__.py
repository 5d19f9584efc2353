"""Seeded synthetic inputs for batched draft verification.

These generators serve both the GPU tests/benchmark and the oracle tests.
They synthesise *inputs* only (target logits, draft distributions, draft ids,
tree topologies, temperatures, seeds); none of the verification arithmetic
lives here.  Every draw comes from ``numpy.random.Generator(PCG64(seed))`` in
a fixed order, so a (config, set) pair always yields the same arrays.

Workload shapes stand in for real target logits of 128256-entry (Llama-3
family) and 151936-entry (Qwen family) vocabularies; the pages measure on no
public dataset and none is needed.

Logit arrays are float32, or uint16 holding bf16 bits (fp32 rounded to
nearest even).
"""
from __future__ import annotations

import dataclasses
import json
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

# Draft-noise scales chosen so that the mean per-position acceptance
# sum_y min(p, q) of the stochastic rows is about 0.70; written by
# calibrate_sigma.py (bisection on a fixed sample).
_SIGMA_PATH = os.path.join(_HERE, "sigma.json")


def _sigmas():
    with open(_SIGMA_PATH) as f:
        return json.load(f)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    """Draft distribution synthesis: softmax over the last axis in float64,
    returned as float32 (the draft model's probabilities are an input)."""
    z = z.astype(np.float64)
    z -= z.max(axis=-1, keepdims=True)
    np.exp(z, out=z)
    z /= z.sum(axis=-1, keepdims=True)
    return z.astype(np.float32)


def _sample_rows(rng: np.random.Generator, probs: np.ndarray) -> np.ndarray:
    """One categorical draw per row of a [rows, V] probability array."""
    rows, V = probs.shape
    cdf = np.cumsum(probs.astype(np.float64), axis=1)
    u = rng.random(rows) * cdf[:, -1]
    ids = np.array([np.searchsorted(cdf[i], u[i], side="right") for i in range(rows)], dtype=np.int64)
    return np.minimum(ids, V - 1).astype(np.int32)


@dataclasses.dataclass
class ChainInputs:
    logits: np.ndarray            # [bs, k+1, V] float32 or uint16 (bf16 bits)
    draft_ids: np.ndarray         # [bs, k] int32
    draft_probs: np.ndarray | None  # [bs, k, V] float32, None for one-hot drafts
    temperature: np.ndarray       # [bs] float32
    seeds: np.ndarray             # [bs] uint64
    onehot: bool
    name: str

    @property
    def batch(self):
        return self.logits.shape[0]

    @property
    def max_draft(self):
        return self.logits.shape[1] - 1

    @property
    def vocab(self):
        return self.logits.shape[2]


@dataclasses.dataclass
class TreeInputs:
    logits: np.ndarray            # [bs, N, V]
    node_tokens: np.ndarray       # [bs, N] int32 (entry 0 unused, set to -1)
    parent: np.ndarray            # [bs, N] int32 (parent[0] = -1)
    temperature: np.ndarray
    seeds: np.ndarray
    name: str

    @property
    def batch(self):
        return self.logits.shape[0]

    @property
    def num_nodes(self):
        return self.logits.shape[1]

    @property
    def vocab(self):
        return self.logits.shape[2]


def _boosted_normal_logits(rng, rows, V, sigma=3.0, boost=8.0):
    """N(0, sigma^2) logits with +boost on one uniformly chosen token per row."""
    l = rng.standard_normal((rows, V), dtype=np.float32) * np.float32(sigma)
    hot = rng.integers(0, V, size=rows)
    l[np.arange(rows), hot] += np.float32(boost)
    return l


def _philox_seeds(tag: int, bs: int, set_index: int) -> np.ndarray:
    return ((np.uint64(tag) << np.uint64(32)) | (np.arange(bs, dtype=np.uint64)
                                                 + np.uint64(set_index) * np.uint64(1 << 20)))


def chain_small(set_index: int = 0, greedy: bool = False) -> ChainInputs:
    """bs=1, k=3, V=1000: fp32 logits ~ N(0, 2^2); q = softmax(l + N(0, 0.5^2));
    x_i ~ q_i; T = 1 (or 0 for the greedy run); seed 0."""
    rng = np.random.default_rng([1, set_index])
    bs, k, V = 1, 3, 1000
    l = rng.standard_normal((bs, k + 1, V), dtype=np.float32) * np.float32(2.0)
    noise = rng.standard_normal((bs, k, V), dtype=np.float32) * np.float32(0.5)
    q = _softmax_rows((l[:, :k] + noise).reshape(bs * k, V)).reshape(bs, k, V)
    ids = _sample_rows(rng, q.reshape(bs * k, V)).reshape(bs, k)
    temp = np.full(bs, 0.0 if greedy else 1.0, np.float32)
    seeds = np.zeros(bs, np.uint64) + np.uint64(set_index)
    return ChainInputs(l, ids, q, temp, seeds, False, "chain bs=1 k=3 V=1000 fp32" + (" greedy" if greedy else ""))


def chain_fp32(set_index: int = 0, bs: int = 8, k: int = 3, V: int = 128256) -> ChainInputs:
    """bs=8, k=3, V=128256: fp32 logits ~ N(0, 3^2) with one +8 token per row;
    q = softmax(l + N(0, sigma^2)) with sigma tuned for acceptance ~0.7;
    x ~ q; T = 1; Philox seed (2<<32)|b."""
    sigma = _sigmas()["chain_fp32"]
    rng = np.random.default_rng([2, set_index])
    l = _boosted_normal_logits(rng, bs * (k + 1), V).reshape(bs, k + 1, V)
    noise = rng.standard_normal((bs, k, V), dtype=np.float32) * np.float32(sigma)
    q = _softmax_rows((l[:, :k] + noise).reshape(bs * k, V)).reshape(bs, k, V)
    ids = _sample_rows(rng, q.reshape(bs * k, V)).reshape(bs, k)
    temp = np.ones(bs, np.float32)
    return ChainInputs(l, ids, q, temp, _philox_seeds(2, bs, set_index), False,
                       f"chain bs={bs} k={k} V={V} fp32 T=1")


def chain_bf16_mixed(set_index: int = 0, bs: int = 64, k: int = 7, V: int = 128256) -> ChainInputs:
    """bs=64, k=7, V=128256: the boosted-normal generator stored as bf16;
    requests b < bs/2 greedy (T = 0), the rest at T = 0.8 with
    q = softmax((l + N(0, sigma^2)) / 0.8) in fp32; x ~ q; seed (3<<32)|b."""
    sigma = _sigmas()["chain_bf16_mixed"]
    rng = np.random.default_rng([3, set_index])
    T = 0.8
    l = _boosted_normal_logits(rng, bs * (k + 1), V).reshape(bs, k + 1, V)
    lb = f32_to_bf16_bits(l)
    lw = bf16_bits_to_f32(lb)
    noise = rng.standard_normal((bs, k, V), dtype=np.float32) * np.float32(sigma)
    q = _softmax_rows(((lw[:, :k] + noise) / np.float32(T)).reshape(bs * k, V)).reshape(bs, k, V)
    ids = _sample_rows(rng, q.reshape(bs * k, V)).reshape(bs, k)
    temp = np.where(np.arange(bs) < bs // 2, 0.0, T).astype(np.float32)
    return ChainInputs(lb, ids, q, temp, _philox_seeds(3, bs, set_index), False,
                       f"chain bs={bs} k={k} V={V} bf16 half greedy, T=0.8")


def onehot_bf16(set_index: int = 0, bs: int = 256, k: int = 3, V: int = 151936) -> ChainInputs:
    """bs=256, k=3, V=151936, one-hot drafts: bf16 logits ~ N(0, 3^2) plus
    Zipf(1.1)-ranked boosts 8 * rank^-1.1 over a per-row random permutation;
    x_i = argmax(l_i + 0.5 * Gumbel); T = 1; seed (4<<32)|b."""
    rng = np.random.default_rng([4, set_index])
    rows = bs * (k + 1)
    l = rng.standard_normal((rows, V), dtype=np.float32) * np.float32(3.0)
    ranks = np.arange(1, V + 1, dtype=np.float64)
    boost = (8.0 * ranks ** -1.1).astype(np.float32)
    for i in range(rows):
        l[i, rng.permutation(V)] += boost
    lb = f32_to_bf16_bits(l).reshape(bs, k + 1, V)
    lw = bf16_bits_to_f32(lb)
    g = rng.gumbel(size=(bs, k, V)).astype(np.float32)
    ids = np.argmax(lw[:, :k] + np.float32(0.5) * g, axis=-1).astype(np.int32)
    temp = np.ones(bs, np.float32)
    return ChainInputs(lb, ids, None, temp, _philox_seeds(4, bs, set_index), True,
                       f"one-hot chain bs={bs} k={k} V={V} bf16 T=1")


def random_tree(rng, N: int, max_depth: int = 5, max_children: int = 4):
    """Parent array of a random valid draft tree: node i attaches to a node
    j < i, chosen uniformly among those at depth < max_depth with fewer than
    max_children children."""
    parent = np.full(N, -1, np.int32)
    depth = np.zeros(N, np.int32)
    nchild = np.zeros(N, np.int32)
    for i in range(1, N):
        cand = [j for j in range(i) if depth[j] < max_depth and nchild[j] < max_children]
        j = cand[int(rng.integers(0, len(cand)))]
        parent[i] = j
        depth[i] = depth[j] + 1
        nchild[j] += 1
    return parent


def tree_fp32(set_index: int = 0, bs: int = 48, N: int = 8, V: int = 128256, greedy: bool = False) -> TreeInputs:
    """bs=48, N=8 (root + 7 drafted nodes from 5 steps x topk 4), V=128256:
    fp32 logits from the boosted-normal generator per node; random valid
    topology; the children of node n carry the top-1, top-2, ... tokens of
    q_n = softmax(l_n + N(0, sigma^2)) in increasing node index; T = 1
    (T = 0 for the greedy variant); seed (5<<32)|b."""
    sigma = _sigmas()["chain_fp32"]
    rng = np.random.default_rng([5, set_index])
    l = _boosted_normal_logits(rng, bs * N, V).reshape(bs, N, V)
    parent = np.stack([random_tree(rng, N) for _ in range(bs)])
    node_tokens = np.full((bs, N), -1, np.int32)
    for b in range(bs):
        for n in range(N):
            kids = [c for c in range(n + 1, N) if parent[b, c] == n]
            if not kids:
                continue
            z = l[b, n] + rng.standard_normal(V, dtype=np.float32) * np.float32(sigma)
            top = np.argpartition(-z, len(kids))[: len(kids)]
            top = top[np.argsort(-z[top], kind="stable")]
            for c, t in zip(kids, top):
                node_tokens[b, c] = int(t)
    temp = np.full(bs, 0.0 if greedy else 1.0, np.float32)
    return TreeInputs(l, node_tokens, parent, temp, _philox_seeds(5, bs, set_index),
                      f"tree bs={bs} N={N} V={V} fp32" + (" greedy" if greedy else " T=1"))


# Named workloads, smallest first.
CONFIGS = {
    "chain_small": chain_small,
    "chain_fp32": chain_fp32,
    "chain_bf16_mixed": chain_bf16_mixed,
    "onehot_bf16": onehot_bf16,
    "tree_fp32": tree_fp32,
}
