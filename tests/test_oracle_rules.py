"""Deterministic pins of the oracle: closed forms, special cases that reduce
to library routines, the greedy prefix-match formula quoted on the pages, the
edge-case rules and the structural invariants of the chain and tree walks."""
import json
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- row stats
def test_row_stats_match_closed_form_softmax():
    rng = np.random.default_rng(0)
    for T in (1.0, 0.8, 2.5, 0.05):
        l = (rng.standard_normal((6, 3000)) * 3).astype(np.float32)
        m, am, S, st = oracle.row_stats(l, T)
        assert (st == 0).all()
        np.testing.assert_array_equal(m, l.max(axis=1).astype(np.float64))
        np.testing.assert_array_equal(am, l.argmax(axis=1))
        # S = sum exp((l - m)/T) = exp(logsumexp(l/T) - m/T); T is an fp32 input
        T32 = float(np.float32(T))
        ref = np.exp(logsumexp(l.astype(np.float64) / T32, axis=1) - m / T32)
        np.testing.assert_allclose(S, ref, rtol=1e-12)


def test_row_stats_bf16_widening_and_first_argmax():
    rng = np.random.default_rng(1)
    l = (rng.standard_normal((4, 500)) * 3).astype(np.float32)
    h = workloads.f32_to_bf16_bits(l)
    lw = workloads.bf16_bits_to_f32(h)
    # plant exact ties: the first occurrence must win
    lw_max = lw.max(axis=1)
    h[:, 7] = workloads.f32_to_bf16_bits(lw_max)
    h[:, 400] = workloads.f32_to_bf16_bits(lw_max)
    lw = workloads.bf16_bits_to_f32(h)
    m, am, S, st = oracle.row_stats(h, 1.0)
    np.testing.assert_array_equal(am, np.argmax(lw, axis=1))
    assert (am <= 7).all()
    np.testing.assert_allclose(S, np.exp(logsumexp(lw.astype(np.float64), axis=1) - m), rtol=1e-12)


def test_row_stats_nonfinite_rules():
    l = np.zeros((5, 8), np.float32)
    l[0, 3] = np.nan
    l[1, 2] = np.inf
    l[2, :] = -np.inf
    l[3, 5] = -np.inf          # a masked token is fine
    l[4, 0] = -np.inf
    l[4, 1] = 5.0
    m, am, S, st = oracle.row_stats(l, 1.0)
    assert list(st) == [oracle.REQ_NONFINITE, oracle.REQ_NONFINITE, oracle.REQ_NONFINITE, 0, 0]
    assert S[3] == pytest.approx(7.0)  # the -inf token contributes exp(-inf) = 0
    assert am[4] == 1 and m[4] == 5.0


# -------------------------------------------------------------- greedy mode
def test_greedy_equals_prefix_match_formula():
    """T = 0: accept while draft == target argmax; correct_len = cumprod(matches).sum(),
    the emitted token is argmax[correct_len] (the DFlash prefix match on the page
    "The speculative decoding zoo", section "DFlash - the draft that borrows everything")."""
    rng = np.random.default_rng(2)
    bs, k, V = 300, 5, 50
    l = (rng.standard_normal((bs, k + 1, V)) * 2).astype(np.float32)
    amax = l.argmax(axis=-1)
    # drafts: argmax with prob 0.7 per slot, otherwise a random token
    ids = np.where(rng.random((bs, k)) < 0.7, amax[:, :k], rng.integers(0, V, (bs, k))).astype(np.int32)
    o = oracle.verify_chain(l, ids, np.zeros(bs, np.float32), np.arange(bs, dtype=np.uint64), onehot=True)
    matches = (ids == amax[:, :k]).astype(np.int32)
    correct_len = np.cumprod(matches, axis=1).sum(axis=1)
    np.testing.assert_array_equal(o["accept_len"], correct_len)
    bonus = amax[np.arange(bs), correct_len]
    for b in range(bs):
        a = correct_len[b]
        np.testing.assert_array_equal(o["tokens"][b, :a], ids[b, :a])
        assert o["tokens"][b, a] == bonus[b]
        assert (o["tokens"][b, a + 1:] == -1).all()
    # greedy results do not depend on the draft kind, the draft probs or the seed
    q = np.full((bs, k, V), 1.0 / V, np.float32)
    o2 = oracle.verify_chain(l, ids, np.zeros(bs, np.float32), np.arange(bs, dtype=np.uint64) + 99, draft_probs=q)
    np.testing.assert_array_equal(o2["tokens"], o["tokens"])
    assert (o["min_margin"] == np.inf).all()


# ------------------------------------------------------- edge-case rules
def test_minus_one_ends_chain_and_bonus_comes_from_row_kb():
    rng = np.random.default_rng(3)
    bs, k, V = 4, 4, 30
    l = (rng.standard_normal((bs, k + 1, V)) * 2).astype(np.float32)
    amax = l.argmax(axis=-1)
    ids = amax[:, :k].astype(np.int32).copy()
    ids[0, 2] = -1          # k_b = 2; slot 3 ignored even though it is garbage
    ids[0, 3] = 12345
    ids[1, 0] = -1          # k_b = 0: only a bonus
    o = oracle.verify_chain(l, ids, np.zeros(bs, np.float32), np.zeros(bs, np.uint64), onehot=True)
    assert list(o["status"]) == [0, 0, 0, 0]
    assert o["accept_len"][0] == 2 and o["tokens"][0, 2] == amax[0, 2]
    assert o["accept_len"][1] == 0 and o["tokens"][1, 0] == amax[1, 0]
    assert o["accept_len"][2] == k and o["tokens"][2, k] == amax[2, k]


def test_bad_inputs_set_request_status_only():
    rng = np.random.default_rng(4)
    bs, k, V = 5, 3, 20
    l = rng.standard_normal((bs, k + 1, V)).astype(np.float32)
    ids = rng.integers(0, V, (bs, k)).astype(np.int32)
    temp = np.ones(bs, np.float32)
    ids[0, 1] = V           # out of range
    ids[1, 0] = -2          # below -1
    temp[2] = np.nan
    l[3, 1, 4] = np.nan     # row 1 is read
    o = oracle.verify_chain(l, ids, temp, np.zeros(bs, np.uint64), onehot=True)
    assert list(o["status"]) == [oracle.REQ_BAD_DRAFT_ID, oracle.REQ_BAD_DRAFT_ID,
                                 oracle.REQ_BAD_TEMPERATURE, oracle.REQ_NONFINITE, 0]
    for b in range(4):
        assert o["accept_len"][b] == 0 and (o["tokens"][b] == -1).all()
    assert o["tokens"][4, o["accept_len"][4]] >= 0
    # a NaN in a row after the first -1 is not read
    ids2 = ids.copy()
    ids2[3] = [-1, 0, 0]
    l2 = l.copy()
    l2[3, 1, 4] = np.nan
    o2 = oracle.verify_chain(l2, ids2, np.ones(bs, np.float32), np.zeros(bs, np.uint64), onehot=True)
    assert o2["status"][3] == 0


def test_q_nonpositive_rule():
    """q(x) <= 0: accept iff p(x) > 0 (the mistral.rs verifier on page "投机解码",
    section "对照：mistral.rs")."""
    V = 8
    l = np.zeros((2, 2, V), np.float32)
    l[1, 0, 5] = -np.inf           # p(5) = 0 in request 1
    q = np.full((2, 1, V), 1.0 / V, np.float32)
    q[:, 0, 5] = 0.0
    ids = np.array([[5], [5]], np.int32)
    o = oracle.verify_chain(l, ids, np.ones(2, np.float32), np.array([1, 2], np.uint64), draft_probs=q)
    assert o["accept_len"][0] == 1     # p > 0, q = 0: accepted regardless of the coin
    assert o["accept_len"][1] == 0     # p = 0, q = 0: rejected


def test_decision_matches_coin_and_p():
    """Each stochastic decision is the strict test u*q(x) < p(x) with the row's coin."""
    rng = np.random.default_rng(6)
    bs, k, V = 400, 3, 40
    l = (rng.standard_normal((bs, k + 1, V)) * 1.5).astype(np.float32)
    q = workloads._softmax_rows(l[:, :k].reshape(-1, V) + rng.standard_normal((bs * k, V)).astype(np.float32)
                                ).reshape(bs, k, V)
    ids = rng.integers(0, V, (bs, k)).astype(np.int32)
    seeds = rng.integers(0, 2**63, bs).astype(np.uint64)
    o = oracle.verify_chain(l, ids, np.ones(bs, np.float32), seeds, draft_probs=q)
    m, am, S, st = oracle.row_stats(l.reshape(-1, V), 1.0)
    for b in range(bs):
        a = o["accept_len"][b]
        for i in range(min(a + 1, k)):
            r = b * (k + 1) + i
            p = np.exp(np.float64(l[b, i, ids[b, i]]) - m[r]) / S[r]
            assert o["p_draft"][b, i] == pytest.approx(p, rel=1e-13)
            u = oracle.coin(int(seeds[b]), b, i)
            accepted = u * float(q[b, i, ids[b, i]]) < p
            assert accepted == (i < a)


# -------------------------------------------------------------- trees
def _chain_tree(bs, k):
    parent = np.tile(np.arange(-1, k, dtype=np.int32), (bs, 1))
    return parent


def test_chain_shaped_tree_equals_onehot_chain_bit_for_bit():
    rng = np.random.default_rng(7)
    for T in (1.0, 0.7, 0.0):
        bs, k, V = 200, 4, 300
        l = (rng.standard_normal((bs, k + 1, V)) * 2).astype(np.float32)
        # drafts likely to be accepted sometimes: sample from the tempered target
        ids = np.argmax(l[:, :k] + rng.gumbel(size=(bs, k, V)).astype(np.float32), axis=-1).astype(np.int32)
        seeds = rng.integers(0, 2**63, bs).astype(np.uint64)
        temp = np.full(bs, T, np.float32)
        oc = oracle.verify_chain(l, ids, temp, seeds, onehot=True)
        node_tokens = np.concatenate([np.full((bs, 1), -1, np.int32), ids], axis=1)
        ot = oracle.verify_tree(l, node_tokens, _chain_tree(bs, k), temp, seeds)
        np.testing.assert_array_equal(ot["accept_len"], oc["accept_len"])
        np.testing.assert_array_equal(ot["tokens"][:, : k + 1], oc["tokens"])
        for b in range(bs):
            a = oc["accept_len"][b]
            np.testing.assert_array_equal(ot["accept_path"][b, :a], np.arange(1, a + 1))


def test_tree_validation():
    V, N = 10, 4
    l = np.zeros((4, N, V), np.float32)
    par = np.array([[-1, 0, 0, 1]] * 4, np.int32)
    tok = np.array([[-1, 1, 2, 3]] * 4, np.int32)
    par[0, 2] = 2            # parent not earlier
    tok[1, 2] = 1            # duplicate sibling token
    par[2, 0] = 0            # root must have parent -1
    tok[3, 3] = V            # token out of range
    o = oracle.verify_tree(l, tok, par, np.ones(4, np.float32), np.zeros(4, np.uint64))
    assert (o["status"] == oracle.REQ_BAD_TREE).all()


def test_tree_greedy_follows_argmax():
    rng = np.random.default_rng(8)
    bs, N, V = 100, 8, 20
    l = (rng.standard_normal((bs, N, V)) * 2).astype(np.float32)
    par = np.stack([workloads.random_tree(rng, N) for _ in range(bs)])
    amax = l.argmax(-1)
    tok = np.full((bs, N), -1, np.int32)
    for b in range(bs):
        for n in range(N):
            kids = [c for c in range(1, N) if par[b, c] == n]
            choices = rng.choice(V, size=len(kids), replace=False)
            if kids and rng.random() < 0.6 and amax[b, n] not in choices:
                choices[int(rng.integers(0, len(kids)))] = amax[b, n]
            for c, t in zip(kids, choices):
                tok[b, c] = t
    o = oracle.verify_tree(l, tok, par, np.zeros(bs, np.float32), np.zeros(bs, np.uint64))
    for b in range(bs):
        cur, path = 0, []
        while True:
            nxt = [c for c in range(1, N) if par[b, c] == cur and tok[b, c] == amax[b, cur]]
            if not nxt:
                break
            cur = nxt[0]
            path.append(cur)
        assert o["accept_len"][b] == len(path)
        np.testing.assert_array_equal(o["accept_path"][b, : len(path)], path)
        assert o["tokens"][b, len(path)] == amax[b, cur]


# ------------------------------------------------- the pages' printed values
def test_toy_example_closed_form_rates():
    """The acceptance rates printed for the 6-token toy distribution follow
    from the rules in closed form."""
    g = json.load(open(os.path.join(GOLDEN, "toy_distribution.json")))
    P, Q = np.array(g["P"]), np.array(g["Q"])
    acc = g["acceptance"]
    assert np.minimum(P, Q).sum() == pytest.approx(acc["standard"], abs=5e-3)
    assert P[np.argmax(Q)] == pytest.approx(acc["onehot"], abs=5e-3)
    top3 = np.argsort(-Q, kind="stable")[:3]
    assert P[top3].sum() == pytest.approx(acc["tree_three_candidates"], abs=5e-3)


def test_expected_tokens_formula_value():
    g = json.load(open(os.path.join(GOLDEN, "expected_tokens.json")))
    a, k = g["alpha"], g["k"]
    assert (1 - a ** (k + 1)) / (1 - a) == pytest.approx(g["E"], abs=5e-4)
