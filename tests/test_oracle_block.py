"""Pins of the oracle's block-verification rule.

Page "The speculative decoding zoo", in its passage on vLLM's rejection
methods, gives the "block" rule's acceptance function: a prefix of the
drafts is accepted as a whole, with probability h = r / (r + 1 - w) built
from the prefix's clipped joint ratio w and the residual mass r at the next
position (h = w for the full chain), the accepted length being the longest
prefix whose coin passes.  The page also states the comparison theorem: the
expected accepted length is at least that of the standard rule, not always
more (identical draft and target accept everything under both).

What pins the oracle here, independently of how it computes h:
  * losslessness over rounds: sequences built round by round from a draft
    Markov chain, verified against a target Markov chain, must follow the
    target's exact joint (the property the method exists for);
  * one draft: the rule must reduce to the standard rule, which is pinned
    on its own, bit for bit;
  * identical, exactly representable draft and target: every draft accepted;
  * the comparison theorem, on the same drafts and coins;
  * one round's exact outcome distribution, enumerated over every draft
    sequence from the acceptance function above.

Seeds are fixed, so each test is deterministic; chi-square tests pass at a
p-value above 1e-6.
"""
import itertools

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from _stats import chi2_pvalue

P_PASS = 1e-6


def _seeds(n, base):
    return (np.arange(n, dtype=np.uint64) * np.uint64(2654435761) + np.uint64(base)).astype(np.uint64)


def _chains(rng, V):
    Pm = rng.dirichlet(np.ones(V) * 0.8, size=V)
    Qm = rng.dirichlet(np.ones(V) * 0.8, size=V)
    lP = np.log(Pm).astype(np.float32)
    Pw = softmax(lP.astype(np.float64), axis=1)  # the target as the verifier sees it
    return lP, Pw, Qm


def _draft(rng, Qm, last, k):
    """k draft tokens per sequence from the draft chain, by inverse CDF."""
    V = Qm.shape[0]
    cq = np.cumsum(Qm, axis=1)
    ids = np.zeros((len(last), k), np.int32)
    cur = last
    for j in range(k):
        u = rng.random(len(last))
        cur = np.minimum((u[:, None] > cq[cur]).sum(axis=1), V - 1)
        ids[:, j] = cur
    return ids


def _round_inputs(lP, Qm, last, ids, onehot):
    ctx = np.concatenate([last[:, None], ids], axis=1)       # token before each row
    logits = lP[ctx]                                          # [n, k+1, V]
    q = None if onehot else Qm[ctx[:, :-1]].astype(np.float32)
    return logits, q


def _markov_sequences(rule, V, k, onehot, n, seed, length=3, s0=0, chains=None):
    rng = np.random.default_rng(seed)
    if chains is None:
        lP, Pw, Qm = _chains(rng, V)
    else:
        Pm, Qm = (np.asarray(c, np.float64) / np.sum(c, axis=1, keepdims=True) for c in chains)
        lP = np.log(Pm).astype(np.float32)
        Pw = softmax(lP.astype(np.float64), axis=1)
    seqs = [[] for _ in range(n)]
    last = np.full(n, s0, np.int64)
    active = np.arange(n)
    rnd = 0
    while len(active):
        m = len(active)
        ids = _draft(rng, Qm, last[active], k)
        logits, q = _round_inputs(lP, Qm, last[active], ids, onehot)
        o = oracle.verify_chain(logits, ids, np.ones(m, np.float32),
                                _seeds(m, 11 + rnd * 104729) + np.uint64(rnd << 40),
                                draft_probs=q, onehot=onehot, rule=rule)
        assert (o["status"] == 0).all()
        still = []
        for j, b in enumerate(active):
            a = o["accept_len"][j]
            seqs[b].extend(int(t) for t in o["tokens"][j, : a + 1])
            if len(seqs[b]) < length:
                still.append(b)
                last[b] = seqs[b][-1]
        active = np.array(still, dtype=np.int64)
        rnd += 1
    idx = np.zeros(n, np.int64)
    for i in range(length):
        idx = idx * V + np.array([s[i] for s in seqs])
    exact = Pw[s0]  # exact[i * V + t] = exact_prev[i] P(t | last token of i)
    for _ in range(length - 1):
        exact = (exact[:, None] * Pw[np.arange(exact.size) % V]).reshape(-1)
    return np.bincount(idx, minlength=V ** length), exact


@pytest.mark.parametrize("V,k,onehot", [(4, 2, False), (3, 3, False), (4, 3, True)])
def test_block_rule_is_lossless_over_rounds(V, k, onehot):
    counts, exact = _markov_sequences("block", V, k, onehot, 200_000, seed=20261201 + 31 * V + k)
    chi2, pv, dof = chi2_pvalue(counts, exact)
    assert pv > P_PASS, (chi2, dof, pv)


# A 3-token pair of chains picked (by a search over random ones) so that the
# prefix weight changes the shape of the residual a lot: drafting 1 then 0
# from token 0 has weight about 0.6 at the second row, where p and q differ
# in opposite directions on tokens 0 and 2.
SHARP_P = [[0.1048, 0.6139, 0.2813], [0.0250, 0.2879, 0.6871], [0.3580, 0.1180, 0.5240]]
SHARP_Q = [[0.0021, 0.9594, 0.0386], [0.4930, 0.0019, 0.5051], [0.0027, 0.5525, 0.4447]]


def test_block_rule_is_lossless_on_a_sharp_chain_pair():
    counts, exact = _markov_sequences("block", 3, 2, False, 200_000, seed=41, chains=(SHARP_P, SHARP_Q))
    chi2, pv, dof = chi2_pvalue(counts, exact)
    assert pv > P_PASS, (chi2, dof, pv)


def test_losslessness_check_detects_a_draft_that_is_not_q():
    """Negative control: drafts drawn from one chain but verified against
    another chain's q make the rule lossy, and the first emitted token's
    frequencies must then reject the target."""
    rng = np.random.default_rng(5)
    V, k, n = 4, 2, 200_000
    lP, Pw, Qm = _chains(rng, V)
    Qwrong = rng.dirichlet(np.ones(V), size=V)
    last = np.zeros(n, np.int64)
    ids = _draft(rng, Qm, last, k)
    logits, _ = _round_inputs(lP, Qm, last, ids, False)
    q = Qwrong[np.concatenate([last[:, None], ids], axis=1)[:, :-1]].astype(np.float32)
    o = oracle.verify_chain(logits, ids, np.ones(n, np.float32), _seeds(n, 3), draft_probs=q, rule="block")
    first = np.bincount(o["tokens"][:, 0], minlength=V)
    _, pv, _ = chi2_pvalue(first, Pw[0])
    assert pv < 1e-12


def test_block_rule_with_one_draft_is_the_standard_rule():
    rng = np.random.default_rng(7)
    n, V = 6000, 64
    l = (rng.standard_normal((n, 2, V)) * 2).astype(np.float32)
    T = np.where(np.arange(n) % 3 == 0, 0.7, 1.0).astype(np.float32)
    T[5::50] = 0.0                                            # some greedy requests
    q = softmax((l[:, 0].astype(np.float64) + rng.standard_normal((n, V))) / T.clip(0.1)[:, None], axis=1)
    q = q.astype(np.float32)
    ids = np.array([rng.choice(V, p=qq / qq.sum()) for qq in q.astype(np.float64)], np.int32)[:, None]
    q[::97, :] = 0.0                                          # q(x) = 0 cases
    q[::97, 0] = 1.0
    std = oracle.verify_chain(l, ids, T, _seeds(n, 99), draft_probs=q[:, None, :])
    blk = oracle.verify_chain(l, ids, T, _seeds(n, 99), draft_probs=q[:, None, :], rule="block")
    np.testing.assert_array_equal(std["accept_len"], blk["accept_len"])
    np.testing.assert_array_equal(std["tokens"], blk["tokens"])
    oh_std = oracle.verify_chain(l, ids, T, _seeds(n, 5), onehot=True)
    oh_blk = oracle.verify_chain(l, ids, T, _seeds(n, 5), onehot=True, rule="block")
    np.testing.assert_array_equal(oh_std["accept_len"], oh_blk["accept_len"])
    np.testing.assert_array_equal(oh_std["tokens"], oh_blk["tokens"])


def test_identical_draft_and_target_accept_everything():
    """p uniform on a support of 4 (equal logits, the rest masked) is exact
    in fp64, and so is q = 1/4 in fp32: every prefix weight is exactly 1,
    every residual mass 0, and the rule must accept all k drafts."""
    rng = np.random.default_rng(3)
    n, V, k = 2000, 16, 6
    support = np.array([1, 5, 6, 12])
    l = np.full((n, k + 1, V), -np.inf, np.float32)
    l[:, :, support] = 2.5
    q = np.zeros((n, k, V), np.float32)
    q[:, :, support] = 0.25
    ids = support[rng.integers(0, 4, size=(n, k))].astype(np.int32)
    o = oracle.verify_chain(l, ids, np.ones(n, np.float32), _seeds(n, 17), draft_probs=q, rule="block")
    assert (o["accept_len"] == k).all()
    assert np.isin(o["tokens"][:, k], support).all()
    np.testing.assert_array_equal(o["tokens"][:, :k], ids)


def test_block_rule_accepts_at_least_as_many_drafts_on_average():
    """The comparison theorem on one round from a fixed context, with the
    same drafts and the same coins for both rules."""
    rng = np.random.default_rng(2024)
    V, k, n = 4, 4, 200_000
    lP, Pw, Qm = _chains(rng, V)
    last = np.zeros(n, np.int64)
    ids = _draft(rng, Qm, last, k)
    logits, q = _round_inputs(lP, Qm, last, ids, False)
    T = np.ones(n, np.float32)
    std = oracle.verify_chain(logits, ids, T, _seeds(n, 1), draft_probs=q)["accept_len"].astype(np.float64)
    blk = oracle.verify_chain(logits, ids, T, _seeds(n, 1), draft_probs=q, rule="block")["accept_len"]
    d = blk.astype(np.float64) - std
    se = d.std() / np.sqrt(n)
    assert d.mean() > -4 * se, (d.mean(), se)
    # the standard rule's mean has a closed form: sum over i of
    # E[prod_{j <= i} min(1, P/Q)] with X ~ Q, enumerated here
    e_std = 0.0
    for xs in itertools.product(range(V), repeat=k):
        pq, ctx, run = 1.0, 0, 1.0
        for x in xs:
            pq *= Qm[ctx, x]
            ctx = x
        ctx = 0
        for x in xs:
            run *= min(1.0, Pw[ctx, x] / float(np.float32(Qm[ctx, x])))
            e_std += pq * run
            ctx = x
    assert abs(std.mean() - e_std) < 5 * std.std() / np.sqrt(n)


def _block_round_exact(Pw, Qm, s0, k):
    """Exact distribution of one round's outcome (accept length a, accepted
    drafts, emitted token), enumerated over every draft sequence, from the
    acceptance function: P(a = i) = h_i prod_{j > i} (1 - h_j)."""
    V = Pw.shape[0]
    Q32 = Qm.astype(np.float32).astype(np.float64)
    out = {}
    for xs in itertools.product(range(V), repeat=k):
        ctx = [s0] + list(xs)
        pq = np.prod([Qm[ctx[i], xs[i]] for i in range(k)])
        w = [1.0]
        for i in range(k):
            w.append(min(w[-1] * Pw[ctx[i], xs[i]] / Q32[ctx[i], xs[i]], 1.0))
        h = [1.0]
        for i in range(1, k + 1):
            if i < k:
                r = np.maximum(w[i] * Pw[ctx[i]] - Q32[ctx[i]], 0.0).sum()
                h.append(r / (r + 1 - w[i]) if r + 1 - w[i] > 0 else 1.0)
            else:
                h.append(w[k])
        for a in range(k + 1):
            pa = h[a] * np.prod([1 - h[j] for j in range(a + 1, k + 1)])
            res = np.maximum(w[a] * Pw[ctx[a]] - Q32[ctx[a]], 0.0) if a < k else Pw[ctx[k]].copy()
            if res.sum() <= 0:
                res = Pw[ctx[a]].copy()
            res /= res.sum()
            for y in range(V):
                key = (a,) + tuple(xs[:a]) + (y,)
                out[key] = out.get(key, 0.0) + pq * pa * res[y]
    return out


def test_one_round_outcomes_match_the_enumerated_distribution():
    rng = np.random.default_rng(77)
    V, k, n = 3, 3, 300_000
    lP, Pw, Qm = _chains(rng, V)
    last = np.zeros(n, np.int64)
    ids = _draft(rng, Qm, last, k)
    logits, q = _round_inputs(lP, Qm, last, ids, False)
    o = oracle.verify_chain(logits, ids, np.ones(n, np.float32), _seeds(n, 8), draft_probs=q, rule="block")
    exact = _block_round_exact(Pw, Qm, 0, k)
    keys = sorted(exact)
    pos = {key: i for i, key in enumerate(keys)}
    cnt = np.zeros(len(keys))
    for a, row in zip(o["accept_len"], o["tokens"]):
        cnt[pos[(int(a),) + tuple(int(t) for t in row[: a + 1])]] += 1
    probs = np.array([exact[key] for key in keys])
    chi2, pv, dof = chi2_pvalue(cnt, probs / probs.sum())
    assert abs(probs.sum() - 1.0) < 1e-9
    assert pv > P_PASS, (chi2, dof, pv)
