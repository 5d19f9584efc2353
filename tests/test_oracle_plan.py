"""Pins of the oracle's survival top-k draft budget.

Page "New approaches to speculative decoding: block drafts, load-aware
verification and PD disaggregation", section "Deciding how much to verify by
load", defines adaptive verification: a (request, position) slot is worth
the chance that the request's drafts are all still accepted at that
position, the product of its confidences up to there; slots are admitted
best first, and the
number admitted maximises expected tokens over the step's cost; page "The
speculative decoding zoo", section "The finer loop: DSpark's confidence
budget", adds the earlier-position-first tie rule.

Pins: the page's worked example and printed output (tests/golden/
adaptive_verification.json); brute force over every prefix-closed admission
on small batches; the tie rule and the first-maximum rule on hand-made
cases; clamping and ragged lengths.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _page_example():
    """The page's inputs, regenerated: the CPU generator seeded with 0 and one
    uniform draw of [batch, K] per batch in the page's order."""
    import torch

    g = json.load(open(os.path.join(GOLDEN, "adaptive_verification.json")))
    K = g["K"]
    bw = g["bandwidth_peak_and_efficiency"][0] * g["bandwidth_peak_and_efficiency"][1]
    fl = g["flops_peak_and_efficiency"][0] * g["flops_peak_and_efficiency"][1]

    def step_time(tokens):
        return max(g["w_bytes"] / bw, tokens * g["flop_per_token"] / fl)

    torch.manual_seed(0)
    out = []
    for case in g["cases"]:
        batch = case["batch"]
        half = batch // 2
        # one [batch, K] uniform draw per batch, in the page's order; each
        # confidence is a base level (0.9 for the first half of the batch,
        # 0.55 for the rest) scaled by a jitter in [0.9, 1.1), in fp32,
        # capped at 0.99
        u = torch.rand(batch, K).numpy()
        jitter = u * np.float32(0.2) + np.float32(0.9)
        accurate = np.float32(0.9) * jitter[:half]
        other = np.float32(0.55) * jitter[half:]
        conf = np.minimum(np.concatenate([accurate, other]), np.float32(0.99)).astype(np.float32)
        cost = np.empty(batch * K + 1)
        for b in range(batch * K + 1):
            cost[b] = g["t_draft"] + step_time(batch + b)
        out.append((case, conf, cost, step_time, g["t_draft"], K))
    return out


def test_page_worked_example():
    for case, conf, cost, step_time, t_draft, K in _page_example():
        batch = case["batch"]
        r = oracle.plan_budget(conf, cost, float(batch))
        assert r["budget"] == case["admitted"], (batch, r["budget"])
        assert round(r["rate"]) == case["adaptive"], (batch, r["rate"])
        assert sum(r["draft_len"]) == r["budget"]
        half = batch // 2
        assert f"{r['draft_len'][:half].mean():.1f}" == f"{case['mean_accurate']:.1f}"
        assert f"{r['draft_len'][half:].mean():.1f}" == f"{case['mean_other']:.1f}"
        # the two reference points the page prints beside it
        surv = np.cumprod(conf.astype(np.float32), axis=1, dtype=np.float32)
        assert round(batch / step_time(batch)) == case["none"]
        assert round((batch + float(surv.sum(dtype=np.float64))) / (t_draft + step_time(batch * (1 + K)))) == case["all"]


def _brute_force(conf, cost, base, num_steps=None):
    """Best ratio over every admission that is a prefix of each request
    (any size), by enumeration, without sorting."""
    bs, K = conf.shape
    c = np.nan_to_num(conf.astype(np.float32), nan=0.0).clip(0, 1)
    surv = np.cumprod(c, axis=1, dtype=np.float32).astype(np.float64)
    lens = [K if num_steps is None else int(np.clip(num_steps[b], 0, K)) for b in range(bs)]
    best, best_set = -np.inf, None
    for pre in itertools.product(*[range(L + 1) for L in lens]):
        B = sum(pre)
        if B >= len(cost):
            continue
        val = (base + sum(surv[b, :pre[b]].sum() for b in range(bs))) / cost[B]
        if val > best + 1e-12 * abs(best) or best_set is None:
            best, best_set = val, pre
    return best, best_set


@pytest.mark.parametrize("seed", range(12))
def test_matches_brute_force_over_prefix_admissions(seed):
    rng = np.random.default_rng(seed)
    bs, K = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    conf = rng.random((bs, K)).astype(np.float32)
    if seed % 3 == 0:
        conf[:, 0] = 1.0
    num_steps = rng.integers(0, K + 1, size=bs) if seed % 2 else None
    n = bs * K
    cost = 1.0 + rng.random(n + 1) * 0.3 + np.arange(n + 1) * rng.random() * 0.4
    if seed % 4 == 1:
        cost = cost[: max(1, n // 2)]        # a cost table shorter than the slots
    base = float(rng.integers(1, 5))
    r = oracle.plan_budget(conf, cost, base, num_steps=num_steps)
    best, best_set = _brute_force(conf, cost, base, num_steps)
    assert r["rate"] == pytest.approx(best, rel=1e-12)
    # the oracle's admission is one of the maximisers and has the smallest size among them
    assert sum(r["draft_len"]) == r["budget"]
    assert r["budget"] <= sum(best_set)


def test_admission_is_a_prefix_and_scores_separate():
    rng = np.random.default_rng(3)
    bs, K = 40, 9
    conf = rng.beta(5, 1.5, size=(bs, K)).astype(np.float32)
    num_steps = rng.integers(0, K + 1, size=bs)
    cost = 1.0 + np.arange(bs * K + 1) * 0.004
    r = oracle.plan_budget(conf, cost, float(bs), num_steps=num_steps)
    surv = np.cumprod(conf, axis=1, dtype=np.float32)
    assert (r["draft_len"] <= num_steps).all()
    admitted = [surv[b, j] for b in range(bs) for j in range(r["draft_len"][b])]
    rejected = [surv[b, j] for b in range(bs) for j in range(r["draft_len"][b], num_steps[b])]
    if admitted and rejected:
        assert min(admitted) >= max(rejected)
    assert sum(r["draft_len"]) == r["budget"]


def test_tie_rule_earlier_position_then_smaller_request():
    # survival [1.0, 0.5] and [0.5, 0.25]: slot (0,1) and slot (1,0) tie at 0.5;
    # the earlier position (request 1, position 0) goes first
    conf = np.array([[1.0, 0.5], [0.5, 0.5]], np.float32)
    cost = np.array([10.0, 1.0, 1.0, 1e9, 1e9])   # best with exactly two slots
    r = oracle.plan_budget(conf, cost, 0.0)
    assert r["budget"] == 2
    np.testing.assert_array_equal(r["draft_len"], [1, 1])
    # equal scores at the same position: the smaller request index goes first
    conf = np.array([[0.7, 0.1], [0.7, 0.1], [0.7, 0.1]], np.float32)
    cost = np.array([10.0, 1.0, 1e9, 1e9, 1e9, 1e9, 1e9])
    r = oracle.plan_budget(conf, cost, 0.0)
    np.testing.assert_array_equal(r["draft_len"], [1, 0, 0])


def test_first_maximum_on_flat_costs_and_zero_scores():
    # confidences 0 add nothing; with equal costs the smaller budget wins
    conf = np.array([[0.9, 0.0, 0.0], [0.8, 0.0, 0.0]], np.float32)
    cost = np.array([1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0])
    r = oracle.plan_budget(conf, cost, 2.0)
    assert r["budget"] == 2
    np.testing.assert_array_equal(r["draft_len"], [1, 1])
    assert r["rate"] == pytest.approx(2.0 + 0.9 + 0.8)


def test_clamping_nan_and_lengths():
    conf = np.array([[np.nan, 0.9], [1.5, -0.2], [0.5, 0.5]], np.float32)
    cost = np.ones(7)
    r = oracle.plan_budget(conf, cost, 1.0, num_steps=np.array([2, 5, -3]))
    # request 0: NaN counts as 0, so both scores are 0; request 1: 1.5 -> 1, -0.2 -> 0;
    # request 2 has no drafted position; flat costs admit the one positive slot
    np.testing.assert_array_equal(r["draft_len"], [0, 1, 0])
    assert r["budget"] == 1 and r["rate"] == pytest.approx(2.0)
    # a NaN after a positive confidence: the first slot is still admitted
    r = oracle.plan_budget(np.array([[0.9, np.nan, 0.9]], np.float32), np.ones(4), 1.0)
    np.testing.assert_array_equal(r["draft_len"], [1])
    assert r["budget"] == 1 and r["rate"] == pytest.approx(1.9)
    # a zero-length table admits nothing
    r = oracle.plan_budget(np.full((2, 2), 0.9, np.float32), np.ones(1), 1.0)
    assert r["budget"] == 0 and (r["draft_len"] == 0).all()
