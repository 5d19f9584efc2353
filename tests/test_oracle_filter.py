"""Pins of the oracle's top-k / top-p filtering of the target.

Page "投机解码", section "接受规则为什么不改变分布", takes the target p after
temperature and the top-k / top-p sampling parameters; the verification is
then lossless for that filtered p.  The filters have plain definitions that
reduce to library routines: top-k keeps the k largest logits (ties at the
k-th kept), top-p the fewest most probable tokens whose mass reaches p.

Pins: switched-off values give the unfiltered result bit for bit; the bonus
sample follows the filtered distribution built here with numpy's sort and
cumulative sum (chi-square), for top-k, top-p and both; top-k = 1 turns a
stochastic request into the greedy one; ties at the threshold are kept; the
multi-round Markov test against the filtered target's exact joint.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
from _stats import chi2_pvalue

P_PASS = 1e-6


def _seeds(n, base):
    return (np.arange(n, dtype=np.uint64) * np.uint64(2654435761) + np.uint64(base)).astype(np.uint64)


def _filtered(l, T, top_k, top_p):
    """The filtered target of one row, from numpy's sort and cumsum."""
    l = l.astype(np.float64)
    p = softmax(l / T)
    keep = np.ones(len(l), bool)
    if 0 < top_k < len(l):
        keep &= l >= np.sort(l)[::-1][top_k - 1]
    if 0 < top_p < 1:
        vals = np.unique(l[keep])[::-1]                       # distinct kept logits, descending
        mass = np.array([p[keep & (l == v)].sum() for v in vals])
        cum = np.cumsum(mass)
        cut = vals[np.searchsorted(cum, top_p * p[keep].sum())]
        keep &= l >= cut
    q = np.where(keep, p, 0.0)
    return q / q.sum()


def test_switched_off_filters_change_nothing():
    rng = np.random.default_rng(1)
    bs, k, V = 300, 3, 50
    l = (rng.standard_normal((bs, k + 1, V)) * 2).astype(np.float32)
    q = softmax(l[:, :k] + rng.standard_normal((bs, k, V)), axis=-1).astype(np.float32)
    ids = np.array([[rng.choice(V, p=qq / qq.sum()) for qq in row] for row in q.astype(np.float64)], np.int32)
    T = np.where(np.arange(bs) % 4 == 0, 0.0, 0.9).astype(np.float32)
    base = oracle.verify_chain(l, ids, T, _seeds(bs, 3), draft_probs=q)
    off_k = np.where(np.arange(bs) % 2 == 0, 0, V).astype(np.int32)
    off_p = np.where(np.arange(bs) % 3 == 0, np.float32(np.nan), np.float32(1.0)).astype(np.float32)
    for rule in ("standard", "block"):
        ref = oracle.verify_chain(l, ids, T, _seeds(bs, 3), draft_probs=q, rule=rule)
        got = oracle.verify_chain(l, ids, T, _seeds(bs, 3), draft_probs=q, rule=rule, top_k=off_k, top_p=off_p)
        for key in ("accept_len", "tokens", "status"):
            np.testing.assert_array_equal(got[key], ref[key])
    np.testing.assert_array_equal(base["tokens"], oracle.verify_chain(l, ids, T, _seeds(bs, 3), draft_probs=q,
                                                                       top_k=off_k)["tokens"])


@pytest.mark.parametrize("top_k,top_p", [(3, 1.0), (0, 0.6), (5, 0.8), (1, 0.3), (0, 0.97)])
def test_bonus_sample_follows_the_filtered_target(top_k, top_p):
    rng = np.random.default_rng(10 + top_k)
    V, n = 12, 200_000
    l = np.round(rng.standard_normal(V) * 1.5, 1).astype(np.float32)   # some equal logits
    T = np.float32(0.8)
    logits = np.tile(l, (n, 1))[:, None, :]
    o = oracle.verify_chain(logits, np.zeros((n, 0), np.int32), np.full(n, T), _seeds(n, 77), onehot=True,
                            top_k=np.full(n, top_k, np.int32), top_p=np.full(n, top_p, np.float32))
    target = _filtered(l, float(T), top_k, top_p)
    if (target > 0).sum() == 1:
        assert (o["tokens"][:, 0] == np.argmax(target)).all()
        return
    chi2, pv, dof = chi2_pvalue(np.bincount(o["tokens"][:, 0], minlength=V), target)
    assert pv > P_PASS, (chi2, dof, pv)


def test_top_k_one_is_greedy():
    rng = np.random.default_rng(4)
    bs, k, V = 400, 4, 30
    l = (rng.standard_normal((bs, k + 1, V)) * 2).astype(np.float32)
    q = softmax(l[:, :k] + rng.standard_normal((bs, k, V)), axis=-1).astype(np.float32)
    ids = np.where(rng.random((bs, k)) < 0.6, np.argmax(l[:, :k], axis=-1),
                   rng.integers(0, V, size=(bs, k))).astype(np.int32)
    greedy = oracle.verify_chain(l, ids, np.zeros(bs, np.float32), _seeds(bs, 1), draft_probs=q)
    for rule in ("standard", "block"):
        top1 = oracle.verify_chain(l, ids, np.full(bs, 0.7, np.float32), _seeds(bs, 1), draft_probs=q, rule=rule,
                                   top_k=np.ones(bs, np.int32))
        np.testing.assert_array_equal(top1["accept_len"], greedy["accept_len"])
        np.testing.assert_array_equal(top1["tokens"], greedy["tokens"])


def test_ties_at_the_threshold_are_kept():
    # logits 3, 2, 2, 1: top-2 keeps three tokens
    l = np.array([[[1.0, 2.0, 3.0, 2.0]]], np.float32).repeat(60000, axis=0)
    o = oracle.verify_chain(l, np.zeros((60000, 0), np.int32), np.ones(60000, np.float32), _seeds(60000, 5),
                            onehot=True, top_k=np.full(60000, 2, np.int32))
    counts = np.bincount(o["tokens"][:, 0], minlength=4)
    assert counts[0] == 0 and (counts[1:] > 0).all()
    chi2, pv, _ = chi2_pvalue(counts, _filtered(l[0, 0], 1.0, 2, 1.0))
    assert pv > P_PASS


@pytest.mark.parametrize("rule", ["standard", "block"])
def test_filtered_target_is_kept_over_rounds(rule):
    """Markov rounds as in the unfiltered pin, with top-k = 3 of 5 tokens and
    top-p = 0.9: sequences follow the filtered target chain's exact joint,
    under both acceptance rules."""
    rng = np.random.default_rng(20261202)
    V, n, s0 = 5, 200_000, 0
    Pm = rng.dirichlet(np.ones(V), size=V)
    Qm = rng.dirichlet(np.ones(V), size=V)
    lP = np.log(Pm).astype(np.float32)
    Pf = np.stack([_filtered(lP[a], 1.0, 3, 0.9) for a in range(V)])
    seqs = [[] for _ in range(n)]
    last = np.full(n, s0, np.int64)
    active = np.arange(n)
    rnd = 0
    while len(active):
        m = len(active)
        cq = np.cumsum(Qm, axis=1)
        d1 = np.minimum((rng.random((m, 1)) > cq[last[active]]).sum(axis=1), V - 1)
        d2 = np.minimum((rng.random((m, 1)) > cq[d1]).sum(axis=1), V - 1)
        ids = np.stack([d1, d2], axis=1).astype(np.int32)
        logits = np.stack([lP[last[active]], lP[d1], lP[d2]], axis=1)
        q = np.stack([Qm[last[active]], Qm[d1]], axis=1).astype(np.float32)
        o = oracle.verify_chain(logits, ids, np.ones(m, np.float32), _seeds(m, 1 + rnd * 7919) + np.uint64(rnd << 40),
                                draft_probs=q, top_k=np.full(m, 3, np.int32), top_p=np.full(m, 0.9, np.float32),
                                rule=rule)
        still = []
        for j, b in enumerate(active):
            a = o["accept_len"][j]
            seqs[b].extend(int(t) for t in o["tokens"][j, : a + 1])
            if len(seqs[b]) < 3:
                still.append(b)
                last[b] = seqs[b][-1]
        active = np.array(still, dtype=np.int64)
        rnd += 1
    idx = np.array([s[0] * V * V + s[1] * V + s[2] for s in seqs])
    exact = np.einsum("a,ab,bc->abc", Pf[s0], Pf, Pf).reshape(-1)
    chi2, pv, dof = chi2_pvalue(np.bincount(idx, minlength=V ** 3), exact)
    assert pv > P_PASS, (chi2, dof, pv)


def test_filtered_probability_of_each_token():
    """p_i(x) of a drafted token is the filtered p at x, for every token of
    rows with groups of equal logits, at top-p values just below and just
    above a group's cumulative mass (the fewest groups reaching the mass)."""
    rng = np.random.default_rng(8)
    V = 9
    cases = []
    for r in range(40):
        l = np.round(rng.standard_normal(V) * 1.2, 1).astype(np.float32)
        T = np.float32(rng.choice([0.5, 1.0, 1.7]))
        top_k = int(rng.choice([0, 2, 4, 7, V]))
        p = softmax(l.astype(np.float64) / float(T))
        keep = l >= np.sort(l)[::-1][top_k - 1] if 0 < top_k < V else np.ones(V, bool)
        vals = np.unique(l[keep])[::-1]
        cum = np.cumsum([p[keep & (l == v)].sum() for v in vals]) / p[keep].sum()
        m = int(rng.integers(0, len(vals)))
        for top_p in (cum[m] * (1 - 1e-5), cum[m] * (1 + 1e-5), float(rng.random())):
            cases.append((l, T, top_k, np.float32(min(top_p, 0.999999))))
    n = len(cases) * V
    logits = np.zeros((n, 2, V), np.float32)
    ids = np.zeros((n, 1), np.int32)
    T = np.zeros(n, np.float32)
    tk = np.zeros(n, np.int32)
    tp = np.zeros(n, np.float32)
    want = np.zeros(n)
    for c, (l, t, k, p) in enumerate(cases):
        f = _filtered(l, float(t), k, float(p))
        for x in range(V):
            j = c * V + x
            logits[j] = l
            ids[j, 0] = x
            T[j], tk[j], tp[j], want[j] = t, k, p, f[x]
    o = oracle.verify_chain(logits, ids, T, _seeds(n, 9), onehot=True, top_k=tk, top_p=tp)
    np.testing.assert_allclose(o["p_draft"][:, 0], want, rtol=1e-12, atol=0)


# ------------------------------------------------------------------ trees
@pytest.mark.parametrize("seed", [0, 1])
def test_filtered_tree_exact_joint(seed):
    """The tree rule under a filtered target: outcomes (accepted path,
    emitted token) against the exact joint built from the filtered rows."""
    import workloads
    from test_oracle_stats import _tree_joint
    rng = np.random.default_rng(700 + seed)
    N, V, n = 6, 6, 400_000
    parent = workloads.random_tree(rng, N, max_depth=3, max_children=3)
    tok = np.full(N, -1, np.int32)
    for node in range(N):
        kids = [c for c in range(1, N) if parent[c] == node]
        for c, t in zip(kids, rng.choice(V, size=len(kids), replace=False)):
            tok[c] = t
    l = np.round(rng.standard_normal((N, V)) * 1.3, 1).astype(np.float32)
    top_k, top_p = (3, 0.9) if seed == 0 else (0, 0.7)
    pf = np.stack([_filtered(l[r], 1.0, top_k, top_p) for r in range(N)])
    o = oracle.verify_tree(np.broadcast_to(l, (n, N, V)).copy(), np.broadcast_to(tok, (n, N)).copy(),
                           np.broadcast_to(parent, (n, N)).copy(), np.ones(n, np.float32), _seeds(n, 60 + seed),
                           top_k=np.full(n, top_k, np.int32), top_p=np.full(n, top_p, np.float32))
    joint = _tree_joint(pf, parent, tok)
    keys = [kk for kk in joint if joint[kk] > 0]
    index = {kk: i for i, kk in enumerate(keys)}
    counts = np.zeros(len(keys))
    for path_row, L, tk in zip(o["accept_path"], o["accept_len"], o["tokens"]):
        key = (tuple(int(v) for v in path_row[:L]), int(tk[L]))
        assert key in index, key        # nothing outside the filtered support
        counts[index[key]] += 1
    probs = np.array([joint[kk] for kk in keys])
    chi2, pv, dof = chi2_pvalue(counts, probs / probs.sum())
    assert pv > P_PASS, (chi2, dof, pv)


def test_filtered_chain_shaped_tree_equals_onehot_chain():
    rng = np.random.default_rng(31)
    bs, k, V = 300, 4, 40
    l = np.round(rng.standard_normal((bs, k + 1, V)) * 2, 1).astype(np.float32)
    ids = rng.integers(0, V, size=(bs, k)).astype(np.int32)
    ids[:, 0] = np.argmax(l[:, 0], axis=1)
    T = rng.choice([0.0, 0.6, 1.0], size=bs).astype(np.float32)
    tk = rng.choice([0, 1, 3, 10], size=bs).astype(np.int32)
    tp = rng.choice([1.0, 0.5, 0.9], size=bs).astype(np.float32)
    seeds = _seeds(bs, 5)
    chain = oracle.verify_chain(l, ids, T, seeds, onehot=True, top_k=tk, top_p=tp)
    node_tokens = np.concatenate([np.full((bs, 1), -1, np.int32), ids], axis=1)
    parent = np.tile(np.arange(-1, k, dtype=np.int32), (bs, 1))
    tree = oracle.verify_tree(l, node_tokens, parent, T, seeds, top_k=tk, top_p=tp)
    np.testing.assert_array_equal(tree["accept_len"], chain["accept_len"])
    np.testing.assert_array_equal(tree["tokens"], chain["tokens"])
    off = oracle.verify_tree(l, node_tokens, parent, T, seeds)
    assert (off["tokens"] != tree["tokens"]).any()
