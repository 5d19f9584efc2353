"""Distribution pins of the verifiers' sampling at vocabularies of several
race chunks.

The emitted token of a round follows a closed form (page "投机解码",
section "接受规则为什么不改变分布"): after a standard rejection it is
normalize(max(0, p - q)) (sub-section "采样：标准拒绝采样"); after a one-hot
rejection, p with the draft removed (sub-section "默认路径：草稿当 one-hot");
after a tree level rejects every child, p with the tried children removed
(sub-section "SGLang 默认：只看目标概率，可以验证一棵树"); with every draft
accepted, the next row's p.  The sampler draws from those weights by a
two-level race over chunks of 2048 ids, a constant of the sampler's
definition.  Here V = 3 * 2048 + 300, so every sample crosses both levels,
including the partial last chunk, and the frequencies of the tokens the
oracle's verifiers emit are compared with the closed form by Pearson
chi-square over binned ids and over the chunks.

Seeds are fixed (each test is deterministic); the pass threshold is a
p-value of 1e-6.
"""
import numpy as np
from scipy.special import softmax

import oracle
from _stats import chi2_pvalue

P_PASS = 1e-6
V = 3 * oracle.RACE_CHUNK + 300
CALLS, BS = 16, 1250          # 20 000 rounds per test


def _seeds(call, n):
    return (np.arange(n, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15 % 2**63)
            + np.uint64(call * 7_654_321 + 17)).astype(np.uint64)


def _target_row(rng):
    """fp32 logits with mass in every chunk: chunk 0 lighter, the partial
    last chunk heavier, a few heavy ids."""
    l = rng.normal(0.0, 1.5, V).astype(np.float32)
    l[: oracle.RACE_CHUNK] -= 1.0
    l[3 * oracle.RACE_CHUNK:] += 1.5
    l[rng.choice(V, 6, replace=False)] += 5.0
    return l


def _p(l):
    return softmax(l.astype(np.float64))


def _check(tokens, w):
    """Emitted ids against weights w (fp64, unnormalised): never an id of
    weight 0, and chi-square over bins of 64 ids and over the chunks."""
    tokens = np.asarray(tokens)
    assert tokens.size > 5000
    assert ((tokens >= 0) & (tokens < V)).all()
    assert (w[tokens] > 0).all(), "an id of zero weight was emitted"
    probs = w / w.sum()
    nb = (V + 63) // 64
    pb = np.bincount(np.arange(V) // 64, weights=probs, minlength=nb)
    chi2, pv, dof = chi2_pvalue(np.bincount(tokens // 64, minlength=nb), pb)
    assert pv > P_PASS, ("bins", chi2, dof, pv)
    pc = np.bincount(np.arange(V) // oracle.RACE_CHUNK, weights=probs, minlength=4)
    chi2, pv, dof = chi2_pvalue(np.bincount(tokens // oracle.RACE_CHUNK, minlength=4), pc)
    assert pv > P_PASS, ("chunks", chi2, dof, pv)


def test_standard_rejection_residual_over_chunks():
    """Draft x0 has p(x0) = 0 and q(x0) > 0, so row 0 always rejects and
    the token comes from normalize(max(0, p0 - q0))."""
    rng = np.random.default_rng(2048)
    l0 = _target_row(rng)
    q0 = softmax(0.7 * l0.astype(np.float64) + rng.normal(0.0, 1.0, V)).astype(np.float32)
    x0 = 5000
    l0[x0] = -np.inf
    logits = np.stack([l0, np.zeros(V, np.float32)])[None]
    w = np.maximum(_p(l0) - q0.astype(np.float64), 0.0)
    assert w[x0] == 0.0 and (w > 0).sum() > 1000
    out = []
    for c in range(CALLS):
        o = oracle.verify_chain(np.broadcast_to(logits, (BS, 2, V)), np.full((BS, 1), x0, np.int32),
                                np.ones(BS, np.float32), _seeds(c, BS),
                                draft_probs=np.broadcast_to(q0, (BS, 1, V)))
        assert (o["status"] == 0).all() and (o["accept_len"] == 0).all()
        out.append(o["tokens"][:, 0])
    _check(np.concatenate(out), w)


def test_onehot_rejection_removes_the_draft_over_chunks():
    """One-hot draft x0 with p(x0) about one half: the rounds that reject it
    emit from p with x0 removed."""
    rng = np.random.default_rng(4096)
    l0 = _target_row(rng)
    x0 = 2 * oracle.RACE_CHUNK + 11
    l0[x0] = np.float32(np.log(np.exp(l0.astype(np.float64)).sum()))  # p(x0) about 1/2
    logits = np.stack([l0, np.zeros(V, np.float32)])[None]
    p = _p(l0)
    assert 0.4 < p[x0] < 0.6
    out = []
    for c in range(CALLS):
        o = oracle.verify_chain(np.broadcast_to(logits, (BS, 2, V)), np.full((BS, 1), x0, np.int32),
                                np.ones(BS, np.float32), _seeds(c, BS) + np.uint64(3), onehot=True)
        assert (o["status"] == 0).all()
        rej = o["accept_len"] == 0
        out.append(o["tokens"][rej, 0])
    w = p.copy()
    w[x0] = 0.0
    _check(np.concatenate(out), w)


def test_bonus_token_follows_p_over_chunks():
    """k = 0: the token is the bonus, drawn from p of row 0 at T = 0.7."""
    rng = np.random.default_rng(8192)
    l0 = _target_row(rng)
    T = np.float32(0.7)
    out = []
    for c in range(CALLS):
        o = oracle.verify_chain(np.broadcast_to(l0[None, None], (BS, 1, V)), np.zeros((BS, 0), np.int32),
                                np.full(BS, T, np.float32), _seeds(c, BS) + np.uint64(5), onehot=True)
        assert (o["status"] == 0).all()
        out.append(o["tokens"][:, 0])
    _check(np.concatenate(out), softmax(l0.astype(np.float64) / np.float64(T)))


def test_tree_level_rejection_removes_the_children_over_chunks():
    """A root with three children whose tokens sit in different chunks; the
    rounds in which the root's level accepts none of them emit from p_root
    with the three tokens removed."""
    rng = np.random.default_rng(16384)
    l0 = _target_row(rng)
    kids = np.array([7, oracle.RACE_CHUNK + 5, 3 * oracle.RACE_CHUNK + 299])
    l0[kids] = np.float32(np.log(np.exp(l0.astype(np.float64)).sum() / 6.0))  # each about 1/9 of the mass
    N = 4
    logits = np.zeros((N, V), np.float32)
    logits[0] = l0
    node_tokens = np.array([0, *kids], np.int32)
    parent = np.array([-1, 0, 0, 0], np.int32)
    p = _p(l0)
    out = []
    for c in range(CALLS):
        o = oracle.verify_tree(np.broadcast_to(logits[None], (BS, N, V)), np.broadcast_to(node_tokens, (BS, N)),
                               np.broadcast_to(parent, (BS, N)), np.ones(BS, np.float32),
                               _seeds(c, BS) + np.uint64(7))
        assert (o["status"] == 0).all()
        rej = o["accept_len"] == 0
        out.append(o["tokens"][rej, 0])
    w = p.copy()
    w[kids] = 0.0
    _check(np.concatenate(out), w)
