"""Distributional pins of the oracle.

The verification rule is exact ("lossless"): its output follows the target
distribution whatever the draft.  Page "投机解码" (Speculative decoding),
section "采样：标准拒绝采样", proves it: a token y comes out either as an
accepted draft, with probability min(p(y), q(y)), or from the residual after
a rejection, with probability max(0, p(y) - q(y)); the sum is p(y), and the
argument repeats position by position.  The same section's one-hot and
target-only-tree cases follow by taking q one-hot, or by walking the tried
candidates in order.  These tests compare the oracle's outcome frequencies
with those closed forms, enumerated cell by cell, by Pearson chi-square.
The relaxed (lossy) tree thresholds are the negative control: the same test
must reject them.

Seeds are fixed, so each test is deterministic; the pass threshold is a
p-value of 1e-6.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from _stats import chi2_pvalue, total_variation

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
P_PASS = 1e-6


def _sample(rng, probs, n):
    """n categorical draws from one probability vector (inverse CDF)."""
    cdf = np.cumsum(probs / probs.sum())
    return np.minimum(np.searchsorted(cdf, rng.random(n), side="right"), len(probs) - 1).astype(np.int32)


def _seeds(n, base):
    return (np.arange(n, dtype=np.uint64) * np.uint64(2654435761) + np.uint64(base)).astype(np.uint64)


def _cells_chain(tokens, accept_len, V):
    """Index of outcome (a, s_0..s_{a-1}, y): offset[a] + sum_i tok_i V^i."""
    n, R = tokens.shape
    offsets = np.concatenate([[0], np.cumsum([V ** (a + 1) for a in range(R)])])
    idx = np.zeros(n, np.int64)
    for i in range(R):
        use = i <= accept_len
        idx += np.where(use, tokens[:, i].astype(np.int64) * V ** i, 0)
    return idx + offsets[accept_len], int(offsets[-1])


# ----------------------------------------------------- the page's toy example
def test_toy_example_rates_and_losslessness():
    g = json.load(open(os.path.join(GOLDEN, "toy_distribution.json")))
    P = np.array(g["P"])
    Q = np.array(g["Q"])
    n = g["draws"]
    base = g["seeds_on_page"][0]
    rng = np.random.default_rng(base)
    lp = np.log(P).astype(np.float32)
    T1 = np.ones(n, np.float32)
    acc = g["acceptance"]

    def check(first, accept, rate, lossless=True):
        se = np.sqrt(rate * (1 - rate) / n) if 0 < rate < 1 else 1e-9
        assert abs(accept.mean() - rate) < 5 * se + 5e-3, (accept.mean(), rate)
        counts = np.bincount(first, minlength=len(P))
        chi2, pv, dof = chi2_pvalue(counts, P)
        tv = total_variation(counts / n, P)
        if lossless:
            assert pv > P_PASS and tv < 0.01, (chi2, pv, tv)
        return chi2, pv, tv

    # standard rejection sampling, drafts drawn from Q
    logits = np.broadcast_to(lp, (n, 2, 6)).copy()
    x = _sample(rng, Q, n)[:, None]
    o = oracle.verify_chain(logits, x, T1, _seeds(n, base), draft_probs=np.broadcast_to(
        Q.astype(np.float32), (n, 1, 6)).copy())
    check(o["tokens"][:, 0], o["accept_len"] > 0, acc["standard"])

    # one-hot draft: the draft proposes argmax Q
    x = np.full((n, 1), int(np.argmax(Q)), np.int32)
    o = oracle.verify_chain(logits, x, T1, _seeds(n, base + 1), onehot=True)
    check(o["tokens"][:, 0], o["accept_len"] > 0, acc["onehot"])

    # target-only tree: three candidates (top three of Q, descending) under the root
    top3 = np.argsort(-Q, kind="stable")[:3]
    tl = np.broadcast_to(lp, (n, 4, 6)).copy()
    par = np.broadcast_to(np.array([-1, 0, 0, 0], np.int32), (n, 4)).copy()
    tok = np.broadcast_to(np.array([-1, *top3], np.int32), (n, 4)).copy()
    o = oracle.verify_tree(tl, tok, par, T1, _seeds(n, base + 2))
    check(o["tokens"][:, 0], o["accept_len"] > 0, acc["tree_three_candidates"])

    # negative control: the relaxed threshold makes the rule lossy
    o = oracle.verify_tree(tl, tok, par, T1, _seeds(n, base + 3), threshold_acc=0.5, threshold_single=0.5)
    chi2, pv, tv = check(o["tokens"][:, 0], o["accept_len"] > 0, acc["relaxed_threshold_0_5"], lossless=False)
    assert pv < 1e-100 and chi2 > 9e4
    assert abs(tv - g["relaxed_threshold_0_5_total_variation"]) < 0.01


# ------------------------------------------------ expected tokens per round
@pytest.mark.parametrize("onehot", [False, True])
def test_expected_tokens_per_round(onehot):
    """With every acceptance probability equal to alpha, tokens per round
    average E = (1 - alpha^(k+1)) / (1 - alpha) (2.533 at alpha 0.7, k 3)."""
    g = json.load(open(os.path.join(GOLDEN, "expected_tokens.json")))
    alpha, k = g["alpha"], g["k"]
    n = 1_000_000
    V = 4
    if onehot:
        # p(x) = alpha at the drafted token 0
        p = np.array([alpha, (1 - alpha) / 3, (1 - alpha) / 3, (1 - alpha) / 3])
        x = np.zeros((n, k), np.int32)
        q = None
    else:
        # q uniform on {0, 1}; p = alpha/2 there, so min(1, p/q) = alpha
        p = np.array([alpha / 2, alpha / 2, (1 - alpha) / 2, (1 - alpha) / 2])
        rng = np.random.default_rng(11)
        x = rng.integers(0, 2, (n, k)).astype(np.int32)
        q = np.broadcast_to(np.array([0.5, 0.5, 0, 0], np.float32), (n, k, V)).copy()
    logits = np.broadcast_to(np.log(p).astype(np.float32), (n, k + 1, V)).copy()
    o = oracle.verify_chain(logits, x, np.ones(n, np.float32), _seeds(n, 77 + onehot), draft_probs=q,
                            onehot=onehot)
    tokens_per_round = o["accept_len"] + 1
    # exact distribution of tokens per round: P(j) = alpha^(j-1)(1-alpha), j <= k; P(k+1) = alpha^k
    j = np.arange(1, k + 2)
    pj = np.where(j <= k, alpha ** (j - 1) * (1 - alpha), alpha ** k)
    E = float((j * pj).sum())
    sd = float(np.sqrt(((j - E) ** 2 * pj).sum()))
    assert E == pytest.approx(g["E"], abs=5e-4)
    assert abs(tokens_per_round.mean() - g["E"]) < 5 * sd / np.sqrt(n) + 5e-4
    chi2, pv, _ = chi2_pvalue(np.bincount(tokens_per_round, minlength=k + 2)[1:], pj)
    assert pv > P_PASS


# --------------------------------------------- exact per-round joint, chain
def _chain_joint_standard(p, q):
    """Closed form of one round: P(s_0..s_{a-1}, y) = prod_{j<a} min(p_j, q_j)(s_j) * w_a(y),
    w_a = max(0, p_a - q_a) for a < k (rejection at a), p_k for a = k."""
    k, V = q.shape
    cells = []
    for a in range(k + 1):
        if a < k:
            resid = np.maximum(p[a] - q[a], 0.0)
            last = resid / resid.sum() * np.maximum(q[a] - p[a], 0.0).sum()
        else:
            last = p[k]
        pref = np.ones(1)
        for j in range(a):
            pref = np.kron(np.minimum(p[j], q[j]), pref)  # index sum s_j V^j
        cells.append(np.kron(last, pref))
    return np.concatenate(cells)


@pytest.mark.parametrize("V,k,T", [(4, 3, 1.0), (6, 2, 0.7), (3, 3, 1.8)])
def test_standard_rule_exact_joint(V, k, T):
    rng = np.random.default_rng(100 + V)
    n = 1_000_000
    l = (rng.standard_normal((k + 1, V)) * 1.2).astype(np.float32)
    p = softmax(l.astype(np.float64) / np.float64(np.float32(T)), axis=1)
    q = rng.dirichlet(np.ones(V), size=k).astype(np.float32)
    x = np.stack([_sample(rng, q[j].astype(np.float64), n) for j in range(k)], axis=1)
    o = oracle.verify_chain(np.broadcast_to(l, (n, k + 1, V)).copy(), x, np.full(n, T, np.float32),
                            _seeds(n, 5 + V), draft_probs=np.broadcast_to(q, (n, k, V)).copy())
    idx, ncell = _cells_chain(o["tokens"], o["accept_len"], V)
    probs = _chain_joint_standard(p, q.astype(np.float64))
    assert len(probs) == ncell
    probs = probs / probs.sum()
    chi2, pv, dof = chi2_pvalue(np.bincount(idx, minlength=ncell), probs)
    assert pv > P_PASS, (chi2, dof, pv)
    # the first emitted token is distributed as p_0 whatever q is
    chi2, pv, _ = chi2_pvalue(np.bincount(o["tokens"][:, 0], minlength=V), p[0])
    assert pv > P_PASS


def test_standard_rule_detects_a_draft_that_is_not_q():
    """Negative control for the chain test: drafts drawn from r != q (the
    verifier is told q) break the guarantee, and the same test sees it."""
    V, k, n = 4, 2, 300_000
    rng = np.random.default_rng(9)
    l = (rng.standard_normal((k + 1, V)) * 1.2).astype(np.float32)
    p = softmax(l.astype(np.float64), axis=1)
    q = rng.dirichlet(np.ones(V), size=k).astype(np.float32)
    r = rng.dirichlet(np.ones(V), size=k)
    x = np.stack([_sample(rng, r[j], n) for j in range(k)], axis=1)
    o = oracle.verify_chain(np.broadcast_to(l, (n, k + 1, V)).copy(), x, np.ones(n, np.float32),
                            _seeds(n, 3), draft_probs=np.broadcast_to(q, (n, k, V)).copy())
    chi2, pv, _ = chi2_pvalue(np.bincount(o["tokens"][:, 0], minlength=V), p[0])
    assert pv < 1e-12


@pytest.mark.parametrize("V,k", [(4, 3), (5, 2)])
def test_onehot_rule_exact_joint(V, k):
    """One-hot draft x ~ r_j: accept with p_j(x); on rejection y ~ p with x removed.
    Closed form: prod_{j<a} r_j(s_j) p_j(s_j) * [a<k: p_a(y)(1 - r_a(y)); a=k: p_k(y)]."""
    rng = np.random.default_rng(200 + V)
    n = 1_000_000
    l = (rng.standard_normal((k + 1, V)) * 1.5).astype(np.float32)
    p = softmax(l.astype(np.float64), axis=1)
    r = rng.dirichlet(np.ones(V), size=k)
    x = np.stack([_sample(rng, r[j], n) for j in range(k)], axis=1)
    o = oracle.verify_chain(np.broadcast_to(l, (n, k + 1, V)).copy(), x, np.ones(n, np.float32),
                            _seeds(n, 40 + V), onehot=True)
    cells = []
    for a in range(k + 1):
        last = p[a] * (1 - r[a]) if a < k else p[k]
        pref = np.ones(1)
        for j in range(a):
            pref = np.kron(r[j] * p[j], pref)
        cells.append(np.kron(last, pref))
    probs = np.concatenate(cells)
    idx, ncell = _cells_chain(o["tokens"], o["accept_len"], V)
    chi2, pv, dof = chi2_pvalue(np.bincount(idx, minlength=ncell), probs / probs.sum())
    assert pv > P_PASS, (chi2, dof, pv)


def test_bonus_race_samples_p():
    """k = 0: the single emitted token is the race over p."""
    for V, T in ((8, 1.0), (8, 0.5), (5, 3.0)):
        n = 400_000
        rng = np.random.default_rng(V * 10 + int(T * 10))
        l = (rng.standard_normal((1, V)) * 2).astype(np.float32)
        p = softmax(l[0].astype(np.float64) / np.float64(np.float32(T)))
        o = oracle.verify_chain(np.broadcast_to(l, (n, 1, V)).copy(), np.zeros((n, 0), np.int32),
                                np.full(n, T, np.float32), _seeds(n, 1000 + V), onehot=True)
        chi2, pv, _ = chi2_pvalue(np.bincount(o["tokens"][:, 0], minlength=V), p)
        assert pv > P_PASS, (V, T, chi2, pv)


# ---------------------------------------------- exact per-round joint, tree
def _tree_joint(p, parent, tok):
    """Outcome (accepted path, emitted y) -> probability: the product of
    p_parent(tok_child) along the path, times p_last(y) with the last node's
    children's tokens removed (all of p at a leaf)."""
    N, V = p.shape
    out = {}

    def rec(node, path, prob):
        kids = [c for c in range(1, N) if parent[c] == node]
        for c in kids:
            rec(c, path + (c,), prob * p[node, tok[c]])
        excluded = {tok[c] for c in kids}
        for y in range(V):
            if y not in excluded:
                out[(path, y)] = out.get((path, y), 0.0) + prob * p[node, y]

    rec(0, (), 1.0)
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tree_rule_exact_joint(seed):
    import workloads
    rng = np.random.default_rng(300 + seed)
    N, V, n = 6, 5, 600_000
    parent = workloads.random_tree(rng, N, max_depth=3, max_children=3)
    tok = np.full(N, -1, np.int32)
    for node in range(N):
        kids = [c for c in range(1, N) if parent[c] == node]
        for c, t in zip(kids, rng.choice(V, size=len(kids), replace=False)):
            tok[c] = t
    l = (rng.standard_normal((N, V)) * 1.3).astype(np.float32)
    p = softmax(l.astype(np.float64), axis=1)
    o = oracle.verify_tree(np.broadcast_to(l, (n, N, V)).copy(), np.broadcast_to(tok, (n, N)).copy(),
                           np.broadcast_to(parent, (n, N)).copy(), np.ones(n, np.float32), _seeds(n, 50 + seed))
    joint = _tree_joint(p, parent, tok)
    keys = list(joint)
    index = {kk: i for i, kk in enumerate(keys)}
    counts = np.zeros(len(keys))
    for path_row, L, tk in zip(o["accept_path"], o["accept_len"], o["tokens"]):
        counts[index[(tuple(int(v) for v in path_row[:L]), int(tk[L]))]] += 1
    probs = np.array([joint[kk] for kk in keys])
    chi2, pv, dof = chi2_pvalue(counts, probs / probs.sum())
    assert pv > P_PASS, (chi2, dof, pv)
    # per-level acceptance at the root is the sum of the candidates' target probabilities
    root_kids = [c for c in range(1, N) if parent[c] == 0]
    rate = (o["accept_len"] > 0).mean()
    expect = p[0, tok[root_kids]].sum()
    assert abs(rate - expect) < 5 * np.sqrt(expect * (1 - expect) / n) + 1e-9


def test_tree_relaxed_threshold_is_detected():
    """Negative control: threshold_single < 1 lets a likely candidate through
    unconditionally, which the joint test rejects."""
    import workloads
    rng = np.random.default_rng(400)
    N, V, n = 4, 4, 200_000
    parent = np.array([-1, 0, 0, 1], np.int32)
    tok = np.array([-1, 0, 1, 2], np.int32)
    l = np.log(np.array([[0.5, 0.2, 0.2, 0.1]] * N)).astype(np.float32)
    p = softmax(l.astype(np.float64), axis=1)
    o = oracle.verify_tree(np.broadcast_to(l, (n, N, V)).copy(), np.broadcast_to(tok, (n, N)).copy(),
                           np.broadcast_to(parent, (n, N)).copy(), np.ones(n, np.float32), _seeds(n, 9),
                           threshold_single=0.3)
    first = np.bincount(o["tokens"][:, 0], minlength=V)
    chi2, pv, _ = chi2_pvalue(first, p[0])
    assert pv < 1e-12


# ------------------------------------------------ multi-round losslessness
def test_markov_chain_sequences_match_exact_joint():
    """A 4-token Markov chain: two drafts per round from a draft chain Q,
    verified against the target chain P with the standard rule, rounds
    repeated until 3 tokens exist.  The 64 length-3 sequences must follow the
    exact joint P[s0,a] P[a,b] P[b,c] (the construction the page "投机解码"
    describes in section "数学验证：拒绝采样不改分布"; its matrices are not given, so
    these are seeded random ones)."""
    rng = np.random.default_rng(20261031)
    V, n, s0 = 4, 300_000, 0
    Pm = rng.dirichlet(np.ones(V) * 0.8, size=V)
    Qm = rng.dirichlet(np.ones(V) * 0.8, size=V)
    lP = np.log(Pm).astype(np.float32)
    Pw = softmax(lP.astype(np.float64), axis=1)    # the target as the verifier sees it
    Q32 = Qm.astype(np.float32)
    seqs = [[] for _ in range(n)]
    last = np.full(n, s0, np.int64)
    rnd = 0
    active = np.arange(n)
    while len(active):
        m = len(active)
        # draft sampling by inverse CDF, one row per sequence
        u = rng.random((m, 2))
        cq = np.cumsum(Qm, axis=1)
        d1 = np.minimum((u[:, :1] > cq[last[active]]).sum(axis=1), V - 1)
        d2 = np.minimum((u[:, 1:] > cq[d1]).sum(axis=1), V - 1)
        ids = np.stack([d1, d2], axis=1).astype(np.int32)
        logits = np.stack([lP[last[active]], lP[d1], lP[d2]], axis=1)
        q = np.stack([Q32[last[active]], Q32[d1]], axis=1)
        o = oracle.verify_chain(logits, ids, np.ones(m, np.float32),
                                _seeds(m, 1 + rnd * 7919) + np.uint64(rnd << 40), draft_probs=q)
        still = []
        for j, b in enumerate(active):
            a = o["accept_len"][j]
            seqs[b].extend(int(t) for t in o["tokens"][j, : a + 1])
            if len(seqs[b]) < 3:
                still.append(b)
                last[b] = seqs[b][-1]
        active = np.array(still, dtype=np.int64)
        rnd += 1
    idx = np.array([s[0] * 16 + s[1] * 4 + s[2] for s in seqs])
    exact = np.einsum("a,ab,bc->abc", Pw[s0], Pw, Pw).reshape(-1)
    chi2, pv, dof = chi2_pvalue(np.bincount(idx, minlength=64), exact)
    assert pv > P_PASS, (chi2, dof, pv)


# ------------------------------------------------ the two-level sampling race
def test_single_chunk_race_is_the_one_level_race():
    """With one chunk the race is argmax_y w(y) / -ln U_y over the id noise
    alone (the textbook exponential race / Gumbel-max), ties to the
    smaller id."""
    rng = np.random.default_rng(77)
    for trial in range(20):
        V = int(rng.integers(1, 300))
        w = rng.random(V) * (rng.random(V) < 0.7)
        if not w.any():
            w[0] = 1.0
        seed, b, r = int(rng.integers(0, 2**63)), int(rng.integers(0, 64)), int(rng.integers(0, 8))
        E = -np.log([oracle.noise_uniform(seed, b, r, y) for y in range(V)])
        want = int(np.argmax(w / E))
        assert oracle.race(w, seed, b, r, chunk=V)[0] == want
        assert oracle.race(w, seed, b, r, chunk=V + 5)[0] == want


def test_two_level_race_samples_the_weights_small_chunks():
    """Chunks of 4 ids over V = 10 (the last chunk partial, one chunk all
    zero): the two-level race still samples w / sum w exactly."""
    w = np.array([0.5, 0.0, 1.5, 0.25, 0.0, 0.0, 0.0, 0.0, 2.0, 0.75])
    n = 300_000
    L = oracle.lib()
    wc = np.ascontiguousarray(w)
    ptr = wc.ctypes.data_as(__import__("ctypes").c_void_p)
    seed = 0x5EED5EED1234
    out = np.array([L.svo_race(ptr, 10, 4, seed, b % 4096, b // 4096, None) for b in range(n)])
    chi2, pv, dof = chi2_pvalue(np.bincount(out, minlength=10), w / w.sum())
    assert pv > P_PASS, (chi2, dof, pv)


def test_two_level_race_samples_the_weights_at_the_verifier_chunk():
    """The verifiers' chunk (2048 ids) over V = 2*2048 + 300: the chunk
    frequencies follow the chunk weight sums, and the ids inside a chunk
    follow their weights (coarse bins)."""
    rng = np.random.default_rng(5)
    V, C = 2 * 2048 + 300, oracle.RACE_CHUNK
    w = rng.random(V) ** 3
    w[100:2048] = 0.0            # chunk 0 is light: ids 0..99 only
    w[2048 + 7] = 40.0           # one heavy id in chunk 1
    n = 24_000
    L = oracle.lib()
    wc = np.ascontiguousarray(w)
    ptr = wc.ctypes.data_as(__import__("ctypes").c_void_p)
    out = np.array([L.svo_race(ptr, V, C, 99, b % 64, b // 64, None) for b in range(n)])
    assert (w[out] > 0).all()
    chunk = out // C
    sums = np.array([w[:C].sum(), w[C:2 * C].sum(), w[2 * C:].sum()])
    chi2, pv, dof = chi2_pvalue(np.bincount(chunk, minlength=3), sums / sums.sum())
    assert pv > P_PASS, (chi2, dof, pv)
    # inside chunk 1: the heavy id against 8 bins of the rest
    sel = out[chunk == 1] - C
    bins = np.where(sel == 7, 8, np.minimum(sel * 8 // C, 7))
    wb = np.array([w[C + i * C // 8: C + (i + 1) * C // 8].sum() for i in range(8)])
    wb[0] -= w[C + 7]
    probs = np.append(wb, w[C + 7]) / w[C:2 * C].sum()
    chi2, pv, dof = chi2_pvalue(np.bincount(bins, minlength=9), probs)
    assert pv > P_PASS, (chi2, dof, pv)


def test_chunk_noise_is_its_own_stream():
    """Chunk noise of chunk c is word 0 of Philox counter (c, r, b, 2)."""
    seed = 0x0123456789ABCDEF
    key = [seed & 0xFFFFFFFF, seed >> 32]
    for c in (0, 1, 62, 1000):
        out = oracle.philox4x32_10([c, 3, 11, 2], key)
        assert oracle.chunk_uniform(seed, 11, 3, c) == oracle.uniform(int(out[0]))
