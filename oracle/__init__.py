"""Reference oracle for batched lossless draft verification (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  The oracle is a plain, slow, single-threaded C
implementation (``svo.c``) of what the GPU library computes, in double
precision.  Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package; the product path never does.

Logit arrays are numpy ``float32`` (fp32 logits) or ``uint16`` (raw bf16 bits).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "svo.c")
_LIB_PATH = os.path.join(_HERE, "libsvo.so")

REQ_OK, REQ_BAD_DRAFT_ID, REQ_BAD_TREE, REQ_NONFINITE, REQ_BAD_TEMPERATURE = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
DRAFT_PROBS, DRAFT_ONEHOT = 0, 1
RULE_STANDARD, RULE_BLOCK = 0, 1


def build(force: bool = True) -> str:
    """Compile svo.c into libsvo.so with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-Wall", "-Wextra",
                               "-Wno-unused-parameter", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_D = ctypes.c_double


class _ChainArgs(ctypes.Structure):
    _fields_ = [("batch", _I32), ("max_draft", _I32), ("vocab", _I32),
                ("logits_dtype", _I32), ("logits", _P), ("logits_row_stride", _I64),
                ("draft_kind", _I32), ("draft_probs", _P), ("q_row_stride", _I64),
                ("draft_ids", _P), ("temperature", _P), ("seed", _P),
                ("accept_len", _P), ("tokens", _P), ("req_status", _P),
                ("p_draft", _P), ("min_margin", _P), ("n_decisions", _P), ("rule", _I32),
                ("top_k", _P), ("top_p", _P), ("cut_margin", _P)]


class _PlanArgs(ctypes.Structure):
    _fields_ = [("batch", _I32), ("max_steps", _I32), ("confidence", _P), ("num_steps", _P),
                ("max_budget", _I32), ("cost", _P), ("base_tokens", _D),
                ("budget", _P), ("draft_len", _P), ("rate", _P), ("margin", _P)]


class _CompactArgs(ctypes.Structure):
    _fields_ = [("batch", _I32), ("num_nodes", _I32), ("accept_len", _P), ("accept_path", _P), ("node_slot", _P),
                ("kv", _P), ("num_layers", _I32), ("num_slots", _I64), ("slot_stride", _I64),
                ("layer_stride", _I64), ("row_bytes", _I64), ("moved", _P)]


class _TreeArgs(ctypes.Structure):
    _fields_ = [("batch", _I32), ("num_nodes", _I32), ("vocab", _I32),
                ("logits_dtype", _I32), ("logits", _P), ("logits_row_stride", _I64),
                ("node_tokens", _P), ("parent", _P), ("temperature", _P), ("seed", _P),
                ("accept_len", _P), ("accept_path", _P), ("tokens", _P), ("req_status", _P),
                ("min_margin", _P), ("n_decisions", _P),
                ("threshold_acc", _D), ("threshold_single", _D), ("top_k", _P), ("top_p", _P),
                ("cut_margin", _P)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        L.svo_philox4x32_10.argtypes = [_P, _P, _P]
        L.svo_philox4x32_10.restype = None
        L.svo_uniform.argtypes = [ctypes.c_uint32]
        L.svo_uniform.restype = _D
        L.svo_coin.argtypes = [ctypes.c_uint64, _I32, _I32]
        L.svo_coin.restype = _D
        L.svo_noise_uniform.argtypes = [ctypes.c_uint64, _I32, _I32, _I32]
        L.svo_noise_uniform.restype = _D
        L.svo_chunk_uniform.argtypes = [ctypes.c_uint64, _I32, _I32, _I32]
        L.svo_chunk_uniform.restype = _D
        L.svo_race.argtypes = [_P, _I32, _I32, ctypes.c_uint64, _I32, _I32, _P]
        L.svo_race.restype = _I32
        L.svo_row_stats.argtypes = [_I32, _I32, _I32, _P, _I64, _P, _P, _P, _P, _P]
        L.svo_row_stats.restype = None
        L.svo_verify_chain.argtypes = [ctypes.POINTER(_ChainArgs)]
        L.svo_verify_chain.restype = None
        L.svo_verify_tree.argtypes = [ctypes.POINTER(_TreeArgs)]
        L.svo_verify_tree.restype = None
        L.svo_plan_budget.argtypes = [ctypes.POINTER(_PlanArgs)]
        L.svo_plan_budget.restype = None
        L.svo_compact_kv.argtypes = [ctypes.POINTER(_CompactArgs)]
        L.svo_compact_kv.restype = None
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _logits_view(logits):
    """Return (contiguous 2-D-or-more array, dtype code, V)."""
    if logits.dtype == np.float32:
        code = F32
    elif logits.dtype == np.uint16:
        code = BF16
    else:
        raise TypeError("logits must be float32 or uint16 (bf16 bits)")
    return np.ascontiguousarray(logits), code, logits.shape[-1]


def philox4x32_10(ctr, key):
    """One Philox4x32-10 block: ctr is 4 uint32 words, key 2 uint32 words."""
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32).reshape(4))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32).reshape(2))
    out = np.zeros(4, dtype=np.uint32)
    lib().svo_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(w: int) -> float:
    return lib().svo_uniform(int(w) & 0xFFFFFFFF)


def coin(seed: int, b: int, r: int) -> float:
    return lib().svo_coin(int(seed), int(b), int(r))


def noise_uniform(seed: int, b: int, r: int, y: int) -> float:
    return lib().svo_noise_uniform(int(seed), int(b), int(r), int(y))


def chunk_uniform(seed: int, b: int, r: int, c: int) -> float:
    return lib().svo_chunk_uniform(int(seed), int(b), int(r), int(c))


RACE_CHUNK = 2048


def race(w, seed: int, b: int, r: int, chunk: int = RACE_CHUNK):
    """The two-level exponential race over the weights w (fp64): (id, margin)."""
    w = np.ascontiguousarray(np.asarray(w, dtype=np.float64))
    m = np.zeros(1, np.float64)
    y = lib().svo_race(_ptr(w), int(w.size), int(chunk), int(seed), int(b), int(r), _ptr(m))
    return int(y), float(m[0])


def row_stats(logits, temperature):
    """Row statistics of a [rows, V] array: (max, argmax, sumexp, status)."""
    x, code, V = _logits_view(logits)
    x = x.reshape(-1, V)
    rows = x.shape[0]
    t = np.ascontiguousarray(np.broadcast_to(np.asarray(temperature, dtype=np.float32), (rows,)))
    m = np.empty(rows, np.float64)
    am = np.empty(rows, np.int32)
    s = np.empty(rows, np.float64)
    st = np.empty(rows, np.int32)
    lib().svo_row_stats(rows, V, code, _ptr(x), V, _ptr(t), _ptr(m), _ptr(am), _ptr(s), _ptr(st))
    return m, am, s, st


def verify_chain(logits, draft_ids, temperature, seeds, draft_probs=None, onehot=False, rule="standard",
                 top_k=None, top_p=None):
    """Chain verification.

    rule: "standard" (left-to-right rejection sampling) or "block" (block
    verification); greedy requests ignore it.  top_k [bs] int32 / top_p [bs]
    float32 (or None): the stochastic requests' target is top-k / top-p
    filtered before verification.

    logits: [bs, k+1, V] float32 or uint16 (bf16 bits); draft_ids: [bs, k] int32;
    draft_probs: [bs, k, V] float32 (standard rule) or None with onehot=True.
    Returns a dict with accept_len, tokens, status, p_draft, min_margin, n_decisions and
    cut_margin (the smallest relative gap of a top-p cut; +inf without one).
    """
    x, code, V = _logits_view(logits)
    bs, R = x.shape[0], x.shape[1]
    k = R - 1
    ids = np.ascontiguousarray(np.asarray(draft_ids, dtype=np.int32).reshape(bs, k))
    temp = np.ascontiguousarray(np.asarray(temperature, dtype=np.float32).reshape(bs))
    sd = np.ascontiguousarray(np.asarray(seeds, dtype=np.uint64).reshape(bs))
    if onehot:
        q = None
        kind = DRAFT_ONEHOT
    else:
        if draft_probs is None:
            raise ValueError("draft_probs required unless onehot=True")
        q = np.ascontiguousarray(np.asarray(draft_probs, dtype=np.float32).reshape(bs, k, V))
        kind = DRAFT_PROBS
    out = dict(accept_len=np.empty(bs, np.int32), tokens=np.empty((bs, R), np.int32),
               status=np.empty(bs, np.int32), p_draft=np.empty((bs, max(k, 1)), np.float64),
               min_margin=np.empty(bs, np.float64), n_decisions=np.empty(bs, np.int32),
               cut_margin=np.empty(bs, np.float64))
    if rule not in ("standard", "block"):
        raise ValueError(f"unknown rule {rule!r}")
    tk = None if top_k is None else np.ascontiguousarray(np.asarray(top_k, np.int32).reshape(bs))
    tp = None if top_p is None else np.ascontiguousarray(np.asarray(top_p, np.float32).reshape(bs))
    a = _ChainArgs(bs, k, V, code, _ptr(x), V, kind, _ptr(q), V, _ptr(ids), _ptr(temp), _ptr(sd),
                   _ptr(out["accept_len"]), _ptr(out["tokens"]), _ptr(out["status"]),
                   _ptr(out["p_draft"]), _ptr(out["min_margin"]), _ptr(out["n_decisions"]),
                   RULE_BLOCK if rule == "block" else RULE_STANDARD,
                   _ptr(tk), _ptr(tp), _ptr(out["cut_margin"]))
    lib().svo_verify_chain(ctypes.byref(a))
    out["p_draft"] = out["p_draft"][:, :k]
    return out


def verify_tree(logits, node_tokens, parent, temperature, seeds, threshold_acc=1.0, threshold_single=1.0,
                top_k=None, top_p=None):
    """Target-only tree verification.

    logits: [bs, N, V]; node_tokens, parent: [bs, N] int32; top_k [bs] int32 /
    top_p [bs] float32 (or None) filter the stochastic requests' target rows.
    threshold_acc / threshold_single other than 1.0 give the lossy relaxed
    rule and exist only for the statistical tests' negative controls.
    """
    x, code, V = _logits_view(logits)
    bs, N = x.shape[0], x.shape[1]
    nt = np.ascontiguousarray(np.asarray(node_tokens, dtype=np.int32).reshape(bs, N))
    par = np.ascontiguousarray(np.asarray(parent, dtype=np.int32).reshape(bs, N))
    temp = np.ascontiguousarray(np.asarray(temperature, dtype=np.float32).reshape(bs))
    sd = np.ascontiguousarray(np.asarray(seeds, dtype=np.uint64).reshape(bs))
    out = dict(accept_len=np.empty(bs, np.int32), accept_path=np.empty((bs, N), np.int32),
               tokens=np.empty((bs, N), np.int32), status=np.empty(bs, np.int32),
               min_margin=np.empty(bs, np.float64), n_decisions=np.empty(bs, np.int32),
               cut_margin=np.empty(bs, np.float64))
    tk = None if top_k is None else np.ascontiguousarray(np.asarray(top_k, np.int32).reshape(bs))
    tp = None if top_p is None else np.ascontiguousarray(np.asarray(top_p, np.float32).reshape(bs))
    a = _TreeArgs(bs, N, V, code, _ptr(x), V, _ptr(nt), _ptr(par), _ptr(temp), _ptr(sd),
                  _ptr(out["accept_len"]), _ptr(out["accept_path"]), _ptr(out["tokens"]),
                  _ptr(out["status"]), _ptr(out["min_margin"]), _ptr(out["n_decisions"]),
                  float(threshold_acc), float(threshold_single), _ptr(tk), _ptr(tp),
                  _ptr(out["cut_margin"]))
    lib().svo_verify_tree(ctypes.byref(a))
    return out


def plan_budget(confidence, cost, base_tokens, num_steps=None):
    """Survival top-k draft budget.

    confidence: [bs, K] float32; cost: [max_budget + 1] float64 (the step cost
    when B draft positions are verified); base_tokens: tokens a step yields
    with none; num_steps: [bs] int32 drafted positions per request or None.
    Returns a dict with budget, draft_len [bs], rate, margin.
    """
    c = np.ascontiguousarray(np.asarray(confidence, dtype=np.float32))
    bs, K = c.shape
    cost = np.ascontiguousarray(np.asarray(cost, dtype=np.float64).reshape(-1))
    ns = None if num_steps is None else np.ascontiguousarray(np.asarray(num_steps, dtype=np.int32).reshape(bs))
    out = dict(budget=np.zeros(1, np.int32), draft_len=np.zeros(bs, np.int32), rate=np.zeros(1, np.float64),
               margin=np.zeros(1, np.float64))
    a = _PlanArgs(bs, K, _ptr(c), _ptr(ns), len(cost) - 1, _ptr(cost), float(base_tokens),
                  _ptr(out["budget"]), _ptr(out["draft_len"]), _ptr(out["rate"]), _ptr(out["margin"]))
    lib().svo_plan_budget(ctypes.byref(a))
    return dict(budget=int(out["budget"][0]), draft_len=out["draft_len"], rate=float(out["rate"][0]),
                margin=float(out["margin"][0]))


def compact_kv(kv, accept_len, accept_path, node_slot):
    """Accepted-path KV compaction in place on a host pool.

    kv: uint8/any array [layers, slots, row] (contiguous, modified in place);
    accept_len [bs] int32; accept_path [bs, N] int32; node_slot [bs, N] int64.
    Returns moved [bs] int32 (rows moved per layer, -1: request skipped).
    """
    assert kv.flags.c_contiguous and kv.ndim == 3
    L, S = kv.shape[0], kv.shape[1]
    row = kv.shape[2] * kv.itemsize
    al = np.ascontiguousarray(np.asarray(accept_len, np.int32))
    ap = np.ascontiguousarray(np.asarray(accept_path, np.int32))
    ns = np.ascontiguousarray(np.asarray(node_slot, np.int64))
    bs, N = ap.shape
    moved = np.zeros(bs, np.int32)
    a = _CompactArgs(bs, N, _ptr(al), _ptr(ap), _ptr(ns), kv.ctypes.data, L, S, row, S * row, row, _ptr(moved))
    lib().svo_compact_kv(ctypes.byref(a))
    return moved
