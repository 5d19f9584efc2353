"""Pins of the oracle's accepted-path KV compaction.

Pages "投机解码", section "与调度、KV 的交互" (sub-section "SGLang：按最坏情况预留，
结束时归还"), and "Draft sources: draft models, n-gram, suffix decoding",
section "SGLang's suffix automaton, in tree": after tree verification the
accepted path is scattered in the tree's KV slots, and its rows are moved so
that the accepted tokens sit contiguously after the committed prefix.

The pins state the result as a gather from the pool before the call (the
row of the i-th accepted node lands in node i's slot, every other slot keeps
its row) and compare the oracle's in-place moves with it, on random trees
whose accepted paths come from the oracle's tree verification, on chain
paths (no move at all), on the overlap case where a destination is an
earlier source, and on malformed requests (left untouched).
"""
import numpy as np

import oracle


def _gather_reference(kv, accept_len, accept_path, node_slot):
    out = kv.copy()
    bs, N = accept_path.shape
    for b in range(bs):
        for i in range(accept_len[b]):
            out[:, node_slot[b, i + 1]] = kv[:, node_slot[b, accept_path[b, i]]]
    return out


def _random_case(rng, bs, N, layers=3, row=24, spare=7):
    """Random trees verified by the oracle, every node on its own slot."""
    l = (rng.standard_normal((bs, N, 50)) * 2).astype(np.float32)
    parent = np.full((bs, N), -1, np.int32)
    tok = np.zeros((bs, N), np.int32)
    for b in range(bs):
        for n in range(1, N):
            parent[b, n] = int(rng.integers(0, n))
        for n in range(1, N):
            sib = [m for m in range(1, n) if parent[b, m] == parent[b, n]]
            choices = [t for t in range(50) if t not in {tok[b, m] for m in sib}]
            tok[b, n] = int(rng.choice(choices))
        l[b, parent[b, 1:], tok[b, 1:]] += 4.0  # make acceptance likely
    temp = np.where(rng.random(bs) < 0.3, 0.0, 1.0).astype(np.float32)
    t = oracle.verify_tree(l, tok, parent, temp, np.arange(bs, dtype=np.uint64) + 5)
    slots = rng.permutation(bs * N + spare)[: bs * N].reshape(bs, N).astype(np.int64)
    kv = rng.integers(0, 256, size=(layers, bs * N + spare, row), dtype=np.uint8)
    return kv, t["accept_len"].astype(np.int32), t["accept_path"].astype(np.int32), slots


def test_compaction_is_the_gather_of_the_accepted_rows():
    rng = np.random.default_rng(0)
    for trial in range(20):
        bs, N = int(rng.integers(1, 12)), int(rng.integers(2, 12))
        kv, al, ap, slots = _random_case(rng, bs, N)
        ref = _gather_reference(kv, al, ap, slots)
        moved = oracle.compact_kv(kv, al, ap, slots)
        np.testing.assert_array_equal(kv, ref)
        assert (moved >= 0).all()
        assert (moved == [sum(ap[b, i] != i + 1 for i in range(al[b])) for b in range(bs)]).all()
    assert (al > 0).any()


def test_chain_path_moves_nothing_and_overlap_is_ordered():
    rng = np.random.default_rng(1)
    kv = rng.integers(0, 256, size=(2, 10, 8), dtype=np.uint8)
    slots = np.arange(10, dtype=np.int64).reshape(2, 5)
    # request 0: chain path 1, 2, 3 (in place); request 1: path 2, 3 -- node 2's
    # slot is the first copy's source and the second copy's destination
    al = np.array([3, 2], np.int32)
    ap = np.array([[1, 2, 3, -1, -1], [2, 3, -1, -1, -1]], np.int32)
    before = kv.copy()
    moved = oracle.compact_kv(kv, al, ap, slots)
    assert list(moved) == [0, 2]
    np.testing.assert_array_equal(kv[:, :5], before[:, :5])
    np.testing.assert_array_equal(kv[:, 6], before[:, 7])   # node 1 <- node 2
    np.testing.assert_array_equal(kv[:, 7], before[:, 8])   # node 2 <- node 3
    np.testing.assert_array_equal(kv[:, 8:], before[:, 8:])
    np.testing.assert_array_equal(kv[:, 5], before[:, 5])


def test_malformed_requests_are_left_untouched():
    rng = np.random.default_rng(2)
    kv = rng.integers(0, 256, size=(1, 20, 4), dtype=np.uint8)
    before = kv.copy()
    slots = np.arange(20, dtype=np.int64).reshape(4, 5)
    slots[3, 4] = 99                                       # outside the pool
    al = np.array([2, 5, 1, 1], np.int32)                  # 5 > N - 1
    ap = np.array([[3, 2, -1, -1, -1],                     # node ids must grow
                   [1, 2, 3, 4, -1],
                   [0, -1, -1, -1, -1],                    # node 0 is the root
                   [4, -1, -1, -1, -1]], np.int32)
    moved = oracle.compact_kv(kv, al, ap, slots)
    assert list(moved) == [-1, -1, -1, -1]
    np.testing.assert_array_equal(kv, before)
