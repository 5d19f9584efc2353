"""GPU parity: the HIP library against the oracle, through the C ABI.

Bar: per-request status, accepted counts and emitted token ids equal the
oracle's bit for bit, except for requests where some decision taken by the
oracle has a relative margin below 1e-6 (|u - p| / max(u, p), |u q - p| /
max(u q, p), the tree's cumulative sums, or the race's top-two key gap):
those are excluded from the comparison and counted, and they must stay a
tiny fraction of all decisions.  Probabilities at the draft ids agree to
1e-5 relative (fp32 input, fp64 decisions).  Argmax (greedy) work is exact.
"""
import numpy as np
import pytest
import torch

import lossless_draft_verification_amd as sv
import oracle
import workloads
from _parity import count

pytestmark = pytest.mark.gpu

MARGIN = 1e-6
# A top-p cut compares fp64 sums of up to V masses, which both sides hold to
# about 1e-11 relative; over a large vocabulary the cut group is one token of
# tiny mass, so its relative gap is often below MARGIN without being at risk.
# A request is exempt for its cut only below this gap.
CUT_MARGIN = 1e-9
P_RTOL = 1e-5
# p at the drafts of a filtered stochastic row uses the thresholds pass's
# kept sum S', which both sides hold to about 1e-13 (fixed-point sums of an
# fp64 exponential on the GPU, sequential fp64 sums in the oracle); the
# 1e-9 cut exemption above relies on that precision, so it is pinned here.
P_RTOL_FILTERED = 1e-10


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d = torch.device("cuda", 0)
    torch.cuda.set_device(d)
    return d


def _t(arr, dev):
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)
    if arr.dtype == np.uint64:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int64)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)


def _np(out):
    return {k: v.cpu().numpy() for k, v in out.items()}


def _compare(ref, got, name, tokens_key="tokens", extra=(), kind="chain"):
    np.testing.assert_array_equal(got["status"], ref["status"], err_msg=f"{name}: status")
    bad = ref["status"] != 0
    assert (got["accept_len"][bad] == 0).all() and (got[tokens_key][bad] == -1).all(), name
    near = (ref["min_margin"] < MARGIN) | (ref["cut_margin"] < CUT_MARGIN)
    ok = (ref["status"] == 0) & ~near
    exempt = (ref["status"] == 0) & near
    count(kind, int(ref["n_decisions"].sum()), int(exempt.sum()), int(ref["status"].size))
    np.testing.assert_array_equal(got["accept_len"][ok], ref["accept_len"][ok], err_msg=f"{name}: accept_len")
    np.testing.assert_array_equal(got[tokens_key][ok], ref[tokens_key][ok], err_msg=f"{name}: tokens")
    for k in extra:
        np.testing.assert_array_equal(got[k][ok], ref[k][ok], err_msg=f"{name}: {k}")
    # the exemption is rare: at most one request per call, or 1e-4 of the decisions
    assert exempt.sum() <= max(1, 1e-4 * ref["n_decisions"].sum()), (name, int(exempt.sum()))
    return int(ok.sum()), int(exempt.sum())


def _compare_p(ref_p, got_p, ref_status, name, cut_ok=None, filtered=None):
    m = (ref_status == 0)[:, None] & np.isfinite(ref_p)
    if cut_ok is not None:
        m &= cut_ok[:, None]
    r, g = ref_p[m], got_p[m]
    assert np.isfinite(g).all(), name
    big = r >= 1e-30
    rel = np.abs(g[big] - r[big]) / r[big]
    assert (rel <= P_RTOL).all(), (name, float(rel.max()))
    if filtered is not None and filtered.any():
        mf = m & filtered[:, None]
        rf, gf = ref_p[mf], got_p[mf]
        bf = rf >= 1e-30
        relf = np.abs(gf[bf] - rf[bf]) / rf[bf]
        assert (relf <= P_RTOL_FILTERED).all(), (name, "filtered rows", float(relf.max()))
        assert (gf[~bf] == rf[~bf]).all() or (np.abs(gf[~bf] - rf[~bf]) <= 1e-30).all(), name
    assert (np.abs(g[~big] - r[~big]) <= 1e-30).all(), name
    # unused slots are NaN on both sides
    np.testing.assert_array_equal(np.isnan(got_p[ref_status == 0]), np.isnan(ref_p[ref_status == 0]))
    return float(rel.max()) if rel.size else 0.0


def _filtered_requests(inp, top_k, top_p):
    """Requests whose target is filtered: stochastic, with top-k in (0, V)
    or top-p in (0, 1)."""
    bs, V = inp.temperature.shape[0], inp.logits.shape[-1]
    t = inp.temperature
    stoch = (t > 0) & np.isfinite(t)
    on = np.zeros(bs, bool)
    if top_k is not None:
        tk = np.asarray(top_k).reshape(bs)
        on |= (tk > 0) & (tk < V)
    if top_p is not None:
        tp = np.asarray(top_p, np.float32).reshape(bs)
        on |= (tp > 0) & (tp < 1)
    return stoch & on


def run_chain(inp, dev, flags=0, top_k=None, top_p=None):
    ref = oracle.verify_chain(inp.logits, inp.draft_ids, inp.temperature, inp.seeds,
                              draft_probs=inp.draft_probs, onehot=inp.onehot,
                              rule="block" if flags & sv.FLAG_BLOCK else "standard", top_k=top_k, top_p=top_p)
    out = sv.verify_chain(_t(inp.logits, dev), _t(inp.draft_ids, dev), _t(inp.temperature, dev),
                          _t(inp.seeds, dev), draft_probs=None if inp.onehot else _t(inp.draft_probs, dev),
                          onehot=inp.onehot, flags=flags, return_p_draft=True, top_k=_t(top_k, dev),
                          top_p=_t(top_p, dev))
    torch.cuda.synchronize()
    return ref, _np(out)


def check_chain(inp, dev, flags=0, top_k=None, top_p=None):
    print(f"[parity] chain {inp.name} flags={flags} filtered={top_k is not None or top_p is not None}", flush=True)
    ref, got = run_chain(inp, dev, flags, top_k, top_p)
    filtered = _filtered_requests(inp, top_k, top_p)
    kind = "filtered chain" if filtered.any() else ("block chain" if flags & sv.FLAG_BLOCK else "chain")
    n_ok, n_ex = _compare(ref, got, inp.name, kind=kind)
    prel = _compare_p(ref["p_draft"], got["p_draft"], ref["status"], inp.name, ref["cut_margin"] >= CUT_MARGIN,
                      filtered)
    print(f"[parity]   compared {n_ok} requests, exempt {n_ex}, max p rel err {prel:.2e}", flush=True)
    return ref, got


def run_tree(inp, dev, flags=0, top_k=None, top_p=None):
    ref = oracle.verify_tree(inp.logits, inp.node_tokens, inp.parent, inp.temperature, inp.seeds, top_k=top_k,
                             top_p=top_p)
    out = sv.verify_tree(_t(inp.logits, dev), _t(inp.node_tokens, dev), _t(inp.parent, dev),
                         _t(inp.temperature, dev), _t(inp.seeds, dev), flags=flags, top_k=_t(top_k, dev),
                         top_p=_t(top_p, dev))
    torch.cuda.synchronize()
    return ref, _np(out)


def check_tree(inp, dev, flags=0, top_k=None, top_p=None):
    print(f"[parity] tree {inp.name} flags={flags} filtered={top_k is not None or top_p is not None}", flush=True)
    ref, got = run_tree(inp, dev, flags, top_k, top_p)
    kind = "filtered tree" if _filtered_requests(inp, top_k, top_p).any() else "tree"
    n_ok, n_ex = _compare(ref, got, inp.name, extra=("accept_path",), kind=kind)
    print(f"[parity]   compared {n_ok} requests, exempt {n_ex}", flush=True)
    return ref, got


# --------------------------------------------------------- the five workloads
@pytest.mark.parametrize("greedy", [False, True])
def test_chain_small_workload(dev, greedy):
    check_chain(workloads.chain_small(0, greedy=greedy), dev)


def test_chain_fp32_workload(dev):
    for s in range(2):
        check_chain(workloads.chain_fp32(s), dev)


def test_chain_bf16_mixed_workload(dev):
    ref, got = check_chain(workloads.chain_bf16_mixed(0), dev)
    # both halves exercised: greedy requests and stochastic ones with rejections
    assert (ref["accept_len"][:32] >= 0).all() and (ref["accept_len"][32:] < 7).any()


def test_onehot_bf16_workload(dev):
    check_chain(workloads.onehot_bf16(0), dev)


@pytest.mark.parametrize("greedy", [False, True])
def test_tree_workload(dev, greedy):
    check_tree(workloads.tree_fp32(0, greedy=greedy), dev)


# ------------------------------------------------- schedules and determinism
def test_all_schedules_are_bit_identical(dev):
    inp = workloads.chain_bf16_mixed(1, bs=24)
    ref = None
    for flags in (sv.FLAG_PHASED, sv.FLAG_FUSED, 0):
        _, out = run_chain(inp, dev, flags=flags)
        if ref is None:
            ref = out
            continue
        for k in ("accept_len", "tokens", "status"):
            np.testing.assert_array_equal(out[k], ref[k])
        np.testing.assert_array_equal(out["p_draft"].view(np.int64), ref["p_draft"].view(np.int64))
    t = workloads.tree_fp32(1, bs=12)
    ref = None
    for flags in (sv.FLAG_PHASED, sv.FLAG_FUSED):
        _, out = run_tree(t, dev, flags=flags)
        if ref is None:
            ref = out
            continue
        for k in ("accept_len", "tokens", "status", "accept_path"):
            np.testing.assert_array_equal(out[k], ref[k])


@pytest.mark.parametrize("kind", ["onehot", "tree"])
def test_chunk_sum_path_equals_the_row_rereading_path(dev, kind):
    """One-hot chains and trees race from the race-chunk sums the statistics
    pass publishes (phased schedule); the fused schedule re-reads the sampled
    row instead.  Both fold the rows alike, so every output is equal bit for
    bit, p included; the fp64 race agrees too.  V = 70001 spans 35 chunks
    with a partial last one."""
    if kind == "onehot":
        rng = np.random.default_rng(31)
        bs, k, V = 40, 3, 70001
        l = (rng.standard_normal((bs, k + 1, V)) * 2.5).astype(np.float32)
        ids = rng.integers(0, V, (bs, k)).astype(np.int32)
        ids[::3, 0] = np.argmax(l[::3, 0], axis=-1)
        temp = np.where(np.arange(bs) % 5 == 0, 0.0, 0.9).astype(np.float32)
        inp = workloads.ChainInputs(workloads.f32_to_bf16_bits(l), ids, None, temp,
                                    np.arange(bs, dtype=np.uint64) * 7 + 1, True, "one-hot chunk sums")
        ref, a = run_chain(inp, dev, flags=sv.FLAG_PHASED)
        _compare(ref, a, inp.name, kind="chain")
        _, b = run_chain(inp, dev, flags=sv.FLAG_FUSED)
        _, c = run_chain(inp, dev, flags=sv.FLAG_PHASED | sv.FLAG_FP64_RACE)
        keys = ("accept_len", "tokens", "status")
        np.testing.assert_array_equal(a["p_draft"].view(np.int64), b["p_draft"].view(np.int64))
    else:
        inp = _random_tree_inputs(77, 24, 12, 70001, "f32")
        ref, a = run_tree(inp, dev, flags=sv.FLAG_PHASED)
        _compare(ref, a, inp.name, extra=("accept_path",), kind="tree")
        _, b = run_tree(inp, dev, flags=sv.FLAG_FUSED)
        _, c = run_tree(inp, dev, flags=sv.FLAG_PHASED | sv.FLAG_FP64_RACE)
        keys = ("accept_len", "tokens", "status", "accept_path")
    for key in keys:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
        np.testing.assert_array_equal(a[key], c[key], err_msg=key)


def test_large_batch_groups_race_chunks(dev):
    """96 requests x 49 race chunks exceed two rounds of one-chunk items, so
    each decision/sampling item takes 3 chunks (the last item one): parity
    with the oracle, and both schedules bit-identical."""
    inp = workloads.chain_bf16_mixed(5, bs=96, V=100000)
    ref, got = check_chain(inp, dev)
    assert (ref["accept_len"][48:] < 7).any()  # stochastic requests with rejections
    _, fused = run_chain(inp, dev, flags=sv.FLAG_FUSED)
    for k in ("accept_len", "tokens", "status"):
        np.testing.assert_array_equal(fused[k], got[k])


@pytest.mark.parametrize("name", ["chain_bf16_mixed", "onehot_bf16"])
def test_split_phases_equal_the_plain_call(dev, name):
    """STATS_ONLY leaves the outputs alone; STATS_ONLY then DECIDE_ONLY on
    one stream gives the plain call's outputs, also with other calls on the
    same workspace queued before."""
    inp = getattr(workloads, name)(4, bs=20, V=30000)
    other = workloads.chain_fp32(5, bs=6, V=20000)

    ws = sv.Workspace(1 << 20, dev)

    def prep(x):
        return sv.PreparedChain(_t(x.logits, dev), _t(x.draft_ids, dev), _t(x.temperature, dev),
                                _t(x.seeds, dev), draft_probs=_t(x.draft_probs, dev), onehot=x.onehot,
                                workspace=ws)

    c, o = prep(inp), prep(other)
    c.launch()
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in c.out.items()}
    for t in c.out.values():
        t.fill_(-5)
    c.launch(phase_flag=sv.FLAG_STATS_ONLY)
    torch.cuda.synchronize()
    for t in c.out.values():
        assert bool((t == -5).all())
    c.launch(phase_flag=sv.FLAG_DECIDE_ONLY)
    torch.cuda.synchronize()
    for n in ref:
        assert torch.equal(ref[n], c.out[n]), n
    # a second request set on the same workspace in between the phases of
    # its own call does not disturb the first call's plain rerun
    o.launch(phase_flag=sv.FLAG_STATS_ONLY)
    o.launch(phase_flag=sv.FLAG_DECIDE_ONLY)
    c.launch()
    torch.cuda.synchronize()
    for n in ref:
        assert torch.equal(ref[n], c.out[n]), n
    out_o = {n: t.cpu().numpy() for n, t in o.out.items()}
    _, plain_o = run_chain(other, dev)
    for n in ("accept_len", "tokens", "status"):
        np.testing.assert_array_equal(out_o[n], plain_o[n])


def test_fp64_race_flag_gives_the_same_tokens(dev):
    inp = workloads.chain_fp32(1, bs=6, V=50000)
    _, a = run_chain(inp, dev)
    _, b = run_chain(inp, dev, flags=sv.FLAG_FP64_RACE)
    np.testing.assert_array_equal(a["tokens"], b["tokens"])
    inp = workloads.chain_bf16_mixed(2, bs=8, V=20000)
    _, a = run_chain(inp, dev)
    _, b = run_chain(inp, dev, flags=sv.FLAG_FP64_RACE | sv.FLAG_PHASED)
    np.testing.assert_array_equal(a["tokens"], b["tokens"])


def test_runs_are_deterministic(dev):
    inp = workloads.chain_fp32(3, bs=8, V=40000)
    _, a = run_chain(inp, dev)
    for _ in range(3):
        _, b = run_chain(inp, dev)
        for k in ("accept_len", "tokens", "status"):
            np.testing.assert_array_equal(a[k], b[k])
        np.testing.assert_array_equal(a["p_draft"].view(np.int64), b["p_draft"].view(np.int64))


def test_workspace_reuse_across_shapes(dev):
    ws = sv.Workspace(1 << 20, dev)
    shapes = [(16, 7, 30000), (3, 2, 1000), (40, 3, 9000), (1, 0, 17), (16, 7, 30000)]
    for i, (bs, k, V) in enumerate(shapes):
        inp = workloads.chain_fp32(10 + i, bs=bs, k=k, V=V)
        ref = oracle.verify_chain(inp.logits, inp.draft_ids, inp.temperature, inp.seeds, draft_probs=inp.draft_probs)
        out = sv.verify_chain(_t(inp.logits, dev), _t(inp.draft_ids, dev), _t(inp.temperature, dev),
                              _t(inp.seeds, dev), draft_probs=_t(inp.draft_probs, dev) if k else None,
                              onehot=(k == 0), workspace=ws)
        torch.cuda.synchronize()
        _compare(ref, _np(out), f"reuse {bs}x{k}x{V}")


@pytest.mark.parametrize("flags", [sv.FLAG_PHASED, sv.FLAG_FUSED])
def test_workspace_reuse_chain_then_tree(dev, flags):
    """Calls of different kinds and shapes on one workspace: each call's
    sampling records sit where the previous call kept other data, so a call
    must not trust that region's contents (a tree call after a chain call
    once read stale completion markers)."""
    ws = sv.Workspace(1 << 20, dev)
    for i in range(2):
        inp = workloads.chain_bf16_mixed(20 + i, bs=24, V=50000)
        ref = oracle.verify_chain(inp.logits, inp.draft_ids, inp.temperature, inp.seeds, draft_probs=inp.draft_probs)
        out = sv.verify_chain(_t(inp.logits, dev), _t(inp.draft_ids, dev), _t(inp.temperature, dev),
                              _t(inp.seeds, dev), draft_probs=_t(inp.draft_probs, dev), flags=flags, workspace=ws)
        torch.cuda.synchronize()
        _compare(ref, _np(out), f"reuse chain {i}")
        t = workloads.tree_fp32(30 + i, bs=12, V=40000)
        ref = oracle.verify_tree(t.logits, t.node_tokens, t.parent, t.temperature, t.seeds)
        out = sv.verify_tree(_t(t.logits, dev), _t(t.node_tokens, dev), _t(t.parent, dev), _t(t.temperature, dev),
                             _t(t.seeds, dev), flags=flags, workspace=ws)
        torch.cuda.synchronize()
        _compare(ref, _np(out), f"reuse tree {i}", extra=("accept_path",), kind="tree")


# ---------------------------------------------------- random small shapes
def _random_chain(seed, bs, k, V, dtype, kind, greedy_frac=0.3, pad_frac=0.3, scale=3.0):
    rng = np.random.default_rng(seed)
    l = (rng.standard_normal((bs, k + 1, V)) * scale).astype(np.float32)
    hot = rng.integers(0, V, size=(bs, k + 1))
    l[np.arange(bs)[:, None], np.arange(k + 1)[None, :], hot] += 6.0
    q = None
    if kind == "probs":
        q = workloads._softmax_rows(l[:, :k].reshape(-1, V) + rng.standard_normal((bs * k, V)).astype(np.float32)
                                    ).reshape(bs, k, V) if k else np.zeros((bs, 0, V), np.float32)
        ids = workloads._sample_rows(rng, q.reshape(-1, V)).reshape(bs, k) if k else np.zeros((bs, 0), np.int32)
    else:
        g = rng.gumbel(size=(bs, k, V)).astype(np.float32)
        ids = np.argmax(l[:, :k] + g, axis=-1).astype(np.int32)
    ids = ids.astype(np.int32)
    for b in range(bs):
        if k and rng.random() < pad_frac:
            ids[b, int(rng.integers(0, k)):] = -1
    temp = rng.choice([0.05, 0.7, 1.0, 2.5], size=bs).astype(np.float32)
    temp[rng.random(bs) < greedy_frac] = 0.0
    seeds = rng.integers(0, 2**63, size=bs).astype(np.uint64)
    logits = workloads.f32_to_bf16_bits(l) if dtype == "bf16" else l
    return workloads.ChainInputs(logits, ids, q, temp, seeds, kind == "onehot",
                                 f"random seed={seed} bs={bs} k={k} V={V} {dtype} {kind}")


SMALL_SHAPES = [
    (1, 1, 0, 1), (2, 3, 1, 2), (3, 5, 3, 7), (4, 33, 7, 1000), (5, 17, 2, 4095), (6, 9, 4, 4096),
    (7, 9, 3, 4097), (8, 4, 7, 8191), (9, 4, 6, 8192), (10, 4, 5, 8193), (11, 6, 3, 12345),
    (12, 3, 63, 300), (13, 7, 2, 33001), (14, 2, 1, 65537), (15, 12, 3, 1001),
]


@pytest.mark.parametrize("seed,bs,k,V", SMALL_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["probs", "onehot"])
def test_random_chain_shapes(dev, seed, bs, k, V, dtype, kind):
    inp = _random_chain(seed * 7 + (dtype == "bf16") * 3 + (kind == "onehot"), bs, k, V, dtype, kind)
    check_chain(inp, dev)


def test_unaligned_row_strides(dev):
    """Rows that are not 16-byte aligned take the scalar-load path."""
    inp = _random_chain(101, 5, 3, 1003, "f32", "probs")
    check_chain(inp, dev)
    inp = _random_chain(102, 5, 3, 1003, "bf16", "onehot")
    check_chain(inp, dev)
    # a strided view: every row is padded to 1010 entries
    base = _random_chain(103, 4, 2, 1010, "f32", "probs")
    lg = torch.from_numpy(base.logits).to(dev)[:, :, :1001]
    q = workloads._softmax_rows(base.logits[:, :2, :1001].reshape(-1, 1001)).reshape(4, 2, 1001)
    ids = np.minimum(base.draft_ids, 1000).astype(np.int32)
    ref = oracle.verify_chain(np.ascontiguousarray(base.logits[:, :, :1001]), ids, base.temperature, base.seeds,
                              draft_probs=q)
    out = sv.verify_chain(lg, _t(ids, dev), _t(base.temperature, dev), _t(base.seeds, dev),
                          draft_probs=_t(q, dev))
    torch.cuda.synchronize()
    _compare(ref, _np(out), "strided view")


# ------------------------------------------------------------- edge cases
def test_edge_statuses(dev):
    rng = np.random.default_rng(5)
    bs, k, V = 10, 3, 5000
    l = (rng.standard_normal((bs, k + 1, V)) * 2).astype(np.float32)
    ids = rng.integers(0, V, (bs, k)).astype(np.int32)
    temp = np.ones(bs, np.float32)
    l[0, 1, 77] = np.nan                 # NaN in a read row
    l[1, 2, 4999] = np.inf               # +inf in a read row
    l[2, 0, :] = -np.inf                 # an all-masked row
    l[3, 0, ::2] = -np.inf               # masked tokens are fine
    ids[4, 1] = V                        # draft id out of range
    ids[5, 0] = -7                       # below -1
    temp[6] = np.nan
    temp[7] = np.inf
    ids[8] = [-1, 5, 5]                  # k_b = 0
    l[8, 2, 3] = np.nan                  # ... so this row is never read
    temp[9] = 0.0                        # greedy
    l[9, :, 100] = 50.0
    ids[9] = [100, 100, 5]
    for dt in ("f32", "bf16"):
        logits = workloads.f32_to_bf16_bits(l) if dt == "bf16" else l
        for kind in ("probs", "onehot"):
            q = workloads._softmax_rows(rng.standard_normal((bs * k, V)).astype(np.float32)).reshape(bs, k, V)
            inp = workloads.ChainInputs(logits, ids, q, temp, np.arange(bs, dtype=np.uint64), kind == "onehot",
                                        f"edge {dt} {kind}")
            ref, got = check_chain(inp, dev)
            assert list(ref["status"][:8]) == [3, 3, 3, 0, 1, 1, 4, 4]
            assert ref["status"][8] == 0 and ref["accept_len"][8] == 0
            assert ref["accept_len"][9] == 2


def test_q_zero_rule_and_masked_drafts(dev):
    bs, k, V = 6, 2, 3000
    rng = np.random.default_rng(9)
    l = rng.standard_normal((bs, k + 1, V)).astype(np.float32)
    q = workloads._softmax_rows(rng.standard_normal((bs * k, V)).astype(np.float32)).reshape(bs, k, V)
    ids = rng.integers(0, V, (bs, k)).astype(np.int32)
    q[np.arange(bs), 0, ids[:, 0]] = 0.0     # q(x) = 0: accept iff p(x) > 0
    l[::2, 0, :] = -np.inf                    # p = 0 except at a few tokens in even requests
    l[::2, 0, 1:20] = 1.0
    inp = workloads.ChainInputs(l, ids, q, np.ones(bs, np.float32), np.arange(bs, dtype=np.uint64) + 3, False,
                                "q zero")
    check_chain(inp, dev)


def test_degenerate_distributions(dev):
    """A single possible token, a tiny temperature, huge logit spreads."""
    bs, k, V = 4, 2, 2000
    l = np.full((bs, k + 1, V), -np.inf, np.float32)
    l[:, :, 42] = 0.0                         # p is a point mass
    l[1, :, 43] = -200.0                      # a second token with negligible mass
    l[2] = np.linspace(-300, 0, V, dtype=np.float32)
    l[3] = np.random.default_rng(3).standard_normal((k + 1, V)).astype(np.float32) * 50
    ids = np.array([[42, 42], [43, 42], [V - 1, 7], [0, 1]], np.int32)
    temp = np.array([1.0, 1.0, 0.01, 1e-3], np.float32)
    check_chain(workloads.ChainInputs(l, ids, None, temp, np.arange(bs, dtype=np.uint64), True, "degenerate"), dev)


# ------------------------------------------------------------------ trees
def _random_tree_inputs(seed, bs, N, V, dtype="f32", greedy_frac=0.3):
    rng = np.random.default_rng(seed)
    l = (rng.standard_normal((bs, N, V)) * 2.5).astype(np.float32)
    def topology():
        depth = int(rng.integers(1, 6))
        kids = 4
        while sum(kids ** d for d in range(1, depth + 1)) < N - 1:  # room for every node
            kids += 1
        return workloads.random_tree(rng, N, max_depth=depth, max_children=kids)
    parent = np.stack([topology() for _ in range(bs)])
    tok = np.full((bs, N), -1, np.int32)
    for b in range(bs):
        for n in range(N):
            kids = [c for c in range(1, N) if parent[b, c] == n]
            if kids:
                z = l[b, n] + rng.gumbel(size=V).astype(np.float32)
                top = np.argsort(-z)[: len(kids)]
                for c, t in zip(kids, top):
                    tok[b, c] = t
    temp = rng.choice([0.5, 1.0, 1.7], size=bs).astype(np.float32)
    temp[rng.random(bs) < greedy_frac] = 0.0
    seeds = rng.integers(0, 2**63, bs).astype(np.uint64)
    logits = workloads.f32_to_bf16_bits(l) if dtype == "bf16" else l
    return workloads.TreeInputs(logits, tok, parent.astype(np.int32), temp, seeds,
                                f"random tree seed={seed} bs={bs} N={N} V={V} {dtype}")


@pytest.mark.parametrize("seed,bs,N,V,dtype", [
    (1, 3, 1, 50, "f32"), (2, 5, 2, 300, "bf16"), (3, 9, 8, 5000, "f32"), (4, 7, 16, 9000, "bf16"),
    (5, 4, 64, 700, "f32"), (6, 11, 8, 33000, "bf16"), (7, 2, 5, 4097, "f32"),
])
def test_random_trees(dev, seed, bs, N, V, dtype):
    check_tree(_random_tree_inputs(seed, bs, N, V, dtype), dev)


def test_bad_trees(dev):
    inp = _random_tree_inputs(8, 6, 6, 500)
    inp.parent[0, 0] = 3
    inp.parent[1, 4] = 4
    inp.node_tokens[2, 3] = 500
    b = 3
    kids = [c for c in range(1, 6) if inp.parent[b, c] == 0]
    if len(kids) < 2:
        inp.parent[b, 2] = 0
        inp.parent[b, 1] = 0
        kids = [1, 2]
    inp.node_tokens[b, kids[1]] = inp.node_tokens[b, kids[0]]
    inp.temperature[4] = np.nan
    ref, got = check_tree(inp, dev)
    assert list(ref["status"][:5]) == [2, 2, 2, 2, 4]


def test_chain_shaped_tree_matches_onehot_chain_on_gpu(dev):
    inp = _random_chain(55, 20, 5, 6000, "bf16", "onehot", pad_frac=0.0)
    _, chain = run_chain(inp, dev)
    node_tokens = np.concatenate([np.full((20, 1), -1, np.int32), inp.draft_ids], axis=1)
    parent = np.tile(np.arange(-1, 5, dtype=np.int32), (20, 1))
    tree = sv.verify_tree(_t(inp.logits, dev), _t(node_tokens, dev), _t(parent, dev), _t(inp.temperature, dev),
                          _t(inp.seeds, dev))
    torch.cuda.synchronize()
    t = _np(tree)
    np.testing.assert_array_equal(t["accept_len"], chain["accept_len"])
    np.testing.assert_array_equal(t["tokens"], chain["tokens"])


# -------------------------------------------------------------- row stats
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_row_stats_parity(dev, dtype):
    rng = np.random.default_rng(11)
    for V in (1, 7, 4096, 8192, 10000, 128256):
        rows = 12
        l = (rng.standard_normal((rows, V)) * 3).astype(np.float32)
        temp = rng.choice([0.0, 0.3, 1.0, 4.0], size=rows).astype(np.float32)
        if V > 10:
            l[0, 5] = l[0].max() + 1
            l[0, V - 1] = l[0, 5]            # an exact tie: the first index wins
            l[1, ::3] = -np.inf
            # far-negative and far-positive rows at small temperatures: large
            # scaled offsets (2^(-l/T) overflows fp32) in both directions
            l[2] -= 60.0
            l[3] += 60.0
            temp[2], temp[3] = 0.05, 0.01
            # -inf everywhere but the last entry
            l[4, :] = -np.inf
            l[4, V - 1] = -3.0
            temp[4] = 0.05
        logits = workloads.f32_to_bf16_bits(l) if dtype == "bf16" else l
        m, am, S, st = oracle.row_stats(logits, temp)
        out = _np(sv.row_stats(_t(logits, dev), _t(temp, dev)))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out["row_status"], st)
        np.testing.assert_array_equal(out["row_max"].astype(np.float64), m)
        np.testing.assert_array_equal(out["row_argmax"], am)
        stoch = temp > 0
        rel = np.abs(out["row_sumexp"][stoch] - S[stoch]) / S[stoch]
        assert (rel < 2e-6).all(), (V, float(rel.max()))
        assert np.isnan(out["row_sumexp"][~stoch]).all()
        print(f"[parity] row stats V={V} {dtype}: max rel err of S {rel.max() if rel.size else 0:.2e}", flush=True)


# ---------------------------------------------------- block verification
BLOCK_SHAPES = [(2, 3, 1, 2), (3, 5, 3, 7), (4, 33, 7, 1000), (5, 17, 2, 4095), (7, 9, 3, 4097),
                (8, 4, 7, 8191), (11, 6, 3, 12345), (12, 3, 63, 300), (13, 7, 2, 33001), (15, 12, 3, 1001)]


@pytest.mark.parametrize("seed,bs,k,V", BLOCK_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["probs", "onehot"])
def test_block_rule_random_chain_shapes(dev, seed, bs, k, V, dtype, kind):
    inp = _random_chain(seed * 11 + (dtype == "bf16") * 5 + (kind == "onehot") + 500, bs, k, V, dtype, kind)
    check_chain(inp, dev, flags=sv.FLAG_BLOCK)


@pytest.mark.parametrize("name", ["chain_bf16_mixed", "chain_fp32", "onehot_bf16"])
def test_block_rule_workloads(dev, name):
    check_chain(getattr(workloads, name)(0), dev, flags=sv.FLAG_BLOCK)


def test_block_rule_with_one_draft_equals_the_standard_rule_on_gpu(dev):
    for kind in ("probs", "onehot"):
        inp = _random_chain(61 + (kind == "onehot"), 40, 1, 5000, "bf16", kind, pad_frac=0.0)
        _, std = run_chain(inp, dev)
        _, blk = run_chain(inp, dev, flags=sv.FLAG_BLOCK)
        for key in ("accept_len", "tokens", "status"):
            np.testing.assert_array_equal(std[key], blk[key], err_msg=f"{kind} {key}")


def test_block_rule_split_phases_and_identical_drafts(dev):
    inp = workloads.chain_bf16_mixed(1, bs=16, k=5, V=20000)
    _, plain = run_chain(inp, dev, flags=sv.FLAG_BLOCK)
    pc = sv.PreparedChain(_t(inp.logits, dev), _t(inp.draft_ids, dev), _t(inp.temperature, dev), _t(inp.seeds, dev),
                          draft_probs=_t(inp.draft_probs, dev), flags=sv.FLAG_BLOCK)
    pc.launch(phase_flag=sv.FLAG_STATS_ONLY)
    pc.launch(phase_flag=sv.FLAG_DECIDE_ONLY)
    torch.cuda.synchronize()
    for key in ("accept_len", "tokens", "status"):
        np.testing.assert_array_equal(pc.out[key].cpu().numpy(), plain[key], err_msg=key)
    # p = q uniform on a support of 4 is exact on both sides: all drafts pass
    n, V, k = 32, 3000, 6
    support = np.array([3, 700, 701, 2999])
    l = np.full((n, k + 1, V), -np.inf, np.float32)
    l[:, :, support] = 1.5
    q = np.zeros((n, k, V), np.float32)
    q[:, :, support] = 0.25
    ids = support[np.random.default_rng(4).integers(0, 4, size=(n, k))].astype(np.int32)
    same = workloads.ChainInputs(l, ids, q, np.ones(n, np.float32), np.arange(n, dtype=np.uint64), False,
                                 "block identical")
    ref, got = check_chain(same, dev, flags=sv.FLAG_BLOCK)
    assert (got["accept_len"] == k).all()


def test_block_rule_zero_draft_probabilities(dev):
    """q(x) = 0 (ratio +inf) and p(x) = 0 (the prefix weight drops to 0)."""
    bs, k, V = 8, 4, 3000
    rng = np.random.default_rng(19)
    l = rng.standard_normal((bs, k + 1, V)).astype(np.float32)
    q = workloads._softmax_rows(rng.standard_normal((bs * k, V)).astype(np.float32)).reshape(bs, k, V)
    ids = rng.integers(0, V, (bs, k)).astype(np.int32)
    q[np.arange(bs), 0, ids[:, 0]] = 0.0
    l[1::2, 1, ids[1::2, 1]] = -np.inf
    inp = workloads.ChainInputs(l, ids, q, np.ones(bs, np.float32), np.arange(bs, dtype=np.uint64) + 40, False,
                                "block zero probabilities")
    check_chain(inp, dev, flags=sv.FLAG_BLOCK)


# ---------------------------------------------- top-k / top-p filtered target
def _filters(rng, bs, V):
    """Per-request top-k / top-p: switched off in several ways, k = 1, small
    and large k, p from 0.3 to 0.99, and both together."""
    tk = rng.choice(np.array([0, 0, 1, 3, 20, 300, V, -5], np.int64), size=bs).astype(np.int32)
    tp = rng.choice(np.array([1.0, 1.0, 0.3, 0.8, 0.95, 0.99, 0.0, np.nan]), size=bs).astype(np.float32)
    return tk, tp


FILTER_SHAPES = [(7, 4, 1, 1), (8, 6, 2, 2), (1, 9, 3, 7), (2, 17, 2, 1000), (3, 12, 4, 4097), (4, 8, 7, 8191), (5, 6, 3, 12345),
                 (6, 5, 2, 33001)]


@pytest.mark.parametrize("seed,bs,k,V", FILTER_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["probs", "onehot"])
@pytest.mark.parametrize("rule", ["standard", "block"])
def test_filtered_random_chain_shapes(dev, seed, bs, k, V, dtype, kind, rule):
    s = seed * 13 + (dtype == "bf16") * 5 + (kind == "onehot") * 2 + (rule == "block") + 900
    inp = _random_chain(s, bs, k, V, dtype, kind)
    tk, tp = _filters(np.random.default_rng(s), bs, V)
    check_chain(inp, dev, flags=sv.FLAG_BLOCK if rule == "block" else 0, top_k=tk, top_p=tp)


@pytest.mark.parametrize("rule", ["standard", "block"])
def test_filtered_bf16_mixed_workload(dev, rule):
    """The bs 64, k 7, V 128256 bf16 workload, every stochastic request filtered."""
    inp = workloads.chain_bf16_mixed(0)
    bs = inp.batch
    tk = np.where(np.arange(bs) % 3 == 0, 0, 50).astype(np.int32)
    tp = np.where(np.arange(bs) % 3 == 1, 1.0, 0.9).astype(np.float32)
    ref, got = check_chain(inp, dev, flags=sv.FLAG_BLOCK if rule == "block" else 0, top_k=tk, top_p=tp)
    assert (ref["accept_len"][32:] < 7).any()


def test_filtered_onehot_workload(dev):
    inp = workloads.onehot_bf16(0, bs=64)
    tk = np.full(inp.batch, 40, np.int32)
    tp = np.full(inp.batch, 0.95, np.float32)
    check_chain(inp, dev, top_k=tk, top_p=tp)


def test_filtered_split_phases(dev):
    inp = workloads.chain_bf16_mixed(2, bs=16, k=5, V=20000)
    tk, tp = _filters(np.random.default_rng(3), inp.batch, inp.vocab)
    for flags in (0, sv.FLAG_BLOCK):
        _, plain = run_chain(inp, dev, flags=flags, top_k=tk, top_p=tp)
        pc = sv.PreparedChain(_t(inp.logits, dev), _t(inp.draft_ids, dev), _t(inp.temperature, dev),
                              _t(inp.seeds, dev), draft_probs=_t(inp.draft_probs, dev), flags=flags,
                              top_k=_t(tk, dev), top_p=_t(tp, dev))
        pc.launch(phase_flag=sv.FLAG_STATS_ONLY)
        pc.launch(phase_flag=sv.FLAG_DECIDE_ONLY)
        pc.launch()
        torch.cuda.synchronize()
        for key in ("accept_len", "tokens", "status"):
            np.testing.assert_array_equal(pc.out[key].cpu().numpy(), plain[key], err_msg=f"{flags} {key}")


def test_filtered_edge_rows(dev):
    """Ties at the cut (integer logits), -inf entries counted by top-k, a
    cut that keeps only the largest group, top-k = 1, and a non-finite row."""
    rng = np.random.default_rng(77)
    bs, k, V = 12, 3, 5000
    l = np.round(rng.standard_normal((bs, k + 1, V)) * 2).astype(np.float32)
    l[1, :, 100:] = -np.inf                      # 100 finite entries, top-k of 400 counts -inf ones
    l[5, 2, 7] = np.nan                          # reported non-finite
    q = workloads._softmax_rows(l[:, :k].reshape(-1, V) * 0.5).reshape(bs, k, V)
    q = np.nan_to_num(q, nan=0.0).astype(np.float32)
    ids = np.argmax(l[:, :k] - np.log(-np.log(rng.random((bs, k, V)))), axis=-1).astype(np.int32)
    ids[1] = rng.integers(0, 100, size=k)
    temp = np.full(bs, 0.9, np.float32)
    temp[[3, 9]] = 0.0
    tk = np.array([5, 400, 1, 7, 0, 3, 1, 0, 2, 5, 4999, 64], np.int32)
    tp = np.array([1.0, 1.0, 1.0, 0.6, 1e-6, 0.5, 0.9, 0.999, 1.0, 0.7, 0.5, 0.25], np.float32)
    for kind in ("probs", "onehot"):
        inp = workloads.ChainInputs(l, ids, q if kind == "probs" else None, temp,
                                    rng.integers(0, 2**63, size=bs).astype(np.uint64), kind == "onehot",
                                    f"filter edges {kind}")
        for flags in (0, sv.FLAG_BLOCK):
            ref, got = check_chain(inp, dev, flags=flags, top_k=tk, top_p=tp)
            assert ref["status"][5] == 3


def test_filtered_crowded_bins(dev):
    """Rows whose logits take a handful of values, so one first-level bin
    holds more keys than the thresholds pass keeps in LDS (it then reads the
    row once per level), beside rows where the list suffices."""
    rng = np.random.default_rng(91)
    bs, k, V = 8, 2, 40000
    vals = np.array([-1.0, 0.0, 0.5, 0.75, 1.0, 2.0], np.float32)
    l = vals[rng.integers(0, len(vals), size=(bs, k + 1, V))]
    l[::2] += (rng.standard_normal((bs // 2, k + 1, V)) * 3).astype(np.float32)  # spread rows
    q = workloads._softmax_rows(l[:, :k].reshape(-1, V) + rng.standard_normal((bs * k, V)).astype(np.float32)
                                ).reshape(bs, k, V)
    ids = workloads._sample_rows(rng, q.reshape(-1, V)).reshape(bs, k).astype(np.int32)
    temp = np.full(bs, 1.0, np.float32)
    tk = np.array([5, 5, 20000, 20000, 0, 0, 9000, 30], np.int32)
    tp = np.array([1.0, 0.5, 1.0, 0.97, 0.5, 0.97, 0.8, 0.9], np.float32)
    inp = workloads.ChainInputs(l, ids, q, temp, rng.integers(0, 2**63, size=bs).astype(np.uint64), False,
                                "filter crowded bins")
    for flags in (0, sv.FLAG_BLOCK):
        check_chain(inp, dev, flags=flags, top_k=tk, top_p=tp)


@pytest.mark.parametrize("seed,bs,N,V,dtype", [
    (21, 5, 2, 300, "bf16"), (22, 9, 8, 5000, "f32"), (23, 7, 16, 9000, "bf16"), (24, 4, 64, 700, "f32"),
    (25, 11, 8, 33000, "bf16"), (26, 6, 5, 4097, "f32"),
])
def test_filtered_random_trees(dev, seed, bs, N, V, dtype):
    inp = _random_tree_inputs(seed + 100, bs, N, V, dtype)
    tk, tp = _filters(np.random.default_rng(seed), bs, V)
    check_tree(inp, dev, top_k=tk, top_p=tp)


def test_filtered_tree_workload(dev):
    inp = workloads.tree_fp32(0)
    bs = inp.node_tokens.shape[0]
    tk = np.where(np.arange(bs) % 3 == 0, 0, 40).astype(np.int32)
    tp = np.where(np.arange(bs) % 3 == 1, 1.0, 0.9).astype(np.float32)
    check_tree(inp, dev, top_k=tk, top_p=tp)


def test_filtered_chain_shaped_tree_matches_onehot_chain_on_gpu(dev):
    inp = _random_chain(56, 20, 5, 6000, "bf16", "onehot", pad_frac=0.0)
    tk, tp = _filters(np.random.default_rng(56), 20, 6000)
    _, chain = run_chain(inp, dev, top_k=tk, top_p=tp)
    node_tokens = np.concatenate([np.full((20, 1), -1, np.int32), inp.draft_ids], axis=1)
    parent = np.tile(np.arange(-1, 5, dtype=np.int32), (20, 1))
    tree = sv.verify_tree(_t(inp.logits, dev), _t(node_tokens, dev), _t(parent, dev), _t(inp.temperature, dev),
                          _t(inp.seeds, dev), top_k=_t(tk, dev), top_p=_t(tp, dev))
    torch.cuda.synchronize()
    t = _np(tree)
    np.testing.assert_array_equal(t["accept_len"], chain["accept_len"])
    np.testing.assert_array_equal(t["tokens"], chain["tokens"])


def test_filtered_calls_are_deterministic(dev):
    """The thresholds pass sums masses in integer fixed point and its LDS list
    order does not reach the results: repeated filtered calls agree bit for
    bit, p at the drafts included."""
    inp = workloads.chain_bf16_mixed(3, bs=32, k=5, V=50000)
    tk, tp = _filters(np.random.default_rng(8), inp.batch, inp.vocab)
    tp[::2] = 0.9  # top-p over the whole row on half the requests
    outs = []
    for _ in range(3):
        out = sv.verify_chain(_t(inp.logits, dev), _t(inp.draft_ids, dev), _t(inp.temperature, dev),
                              _t(inp.seeds, dev), draft_probs=_t(inp.draft_probs, dev), return_p_draft=True,
                              top_k=_t(tk, dev), top_p=_t(tp, dev))
        torch.cuda.synchronize()
        outs.append(_np(out))
    for o in outs[1:]:
        for key in ("accept_len", "tokens", "status"):
            np.testing.assert_array_equal(o[key], outs[0][key])
        np.testing.assert_array_equal(o["p_draft"].view(np.uint64), outs[0]["p_draft"].view(np.uint64))


def test_top_p_alone_trees(dev):
    """Top-p without top-k on bf16 trees: value counts (no top-k array)
    against the passes over the row (an all-zero top-k array), bit for bit,
    and both against the oracle."""
    inp = _random_tree_inputs(344, 9, 8, 20000, "bf16")
    tp = np.random.default_rng(344).choice(np.array([0.5, 0.9, 0.99], np.float32), size=9).astype(np.float32)
    check_tree(inp, dev, top_p=tp)
    outs = []
    for tk in (None, np.zeros(9, np.int32)):
        out = sv.verify_tree(_t(inp.logits, dev), _t(inp.node_tokens, dev), _t(inp.parent, dev),
                             _t(inp.temperature, dev), _t(inp.seeds, dev), top_k=_t(tk, dev), top_p=_t(tp, dev))
        torch.cuda.synchronize()
        outs.append(_np(out))
    _same(outs[0], outs[1], "top-p alone trees: value counts vs passes over the row")


@pytest.mark.parametrize("case", ["bf16_headline", "bf16_flat", "f32", "bf16_wide_temps", "bf16_overflow"])
def test_top_p_alone_paths(dev, case):
    """Top-p without top-k, every request.  bf16 calls without a top-k array
    take the thresholds from value counts; with an all-zero top-k array the
    same rows take the passes over the row (with the cut's lower bound and a
    table of up to 2048 values, or the histogram), and both must agree bit
    for bit.  Cases: the headline shape, flat bf16 rows whose range spans
    zero, fp32 rows, bf16 rows at several temperatures and top-p values, and
    bf16 rows where one value repeats more than 65535 times (a counter
    overflows and the row falls back)."""
    rng = np.random.default_rng(340)
    if case == "bf16_headline":
        inp = workloads.chain_bf16_mixed(5)
        tp = np.full(inp.batch, 0.9, np.float32)
    elif case == "bf16_flat":
        inp = _random_chain(341, 16, 4, 40000, "bf16", "probs", greedy_frac=0.0, scale=0.5)
        tp = np.full(inp.batch, 0.8, np.float32)
    elif case == "f32":
        inp = _random_chain(342, 16, 4, 40000, "f32", "probs", greedy_frac=0.0)
        tp = np.full(inp.batch, 0.9, np.float32)
    elif case == "bf16_wide_temps":
        inp = _random_chain(343, 24, 3, 70000, "bf16", "probs", greedy_frac=0.1)
        tp = rng.choice(np.array([0.3, 0.6, 0.9, 0.99, 0.999], np.float32), size=24)
    else:
        bs, k, V = 4, 2, 70000
        l = np.full((bs, k + 1, V), 0.25, np.float32)
        l[:, :, : V // 8] = (rng.standard_normal((bs, k + 1, V // 8)) * 2).astype(np.float32)
        l[1] = 0.25                                   # every logit equal
        q = workloads._softmax_rows(l[:, :k].reshape(-1, V) * 0.9).reshape(bs, k, V).astype(np.float32)
        ids = workloads._sample_rows(rng, q.reshape(-1, V)).reshape(bs, k).astype(np.int32)
        inp = workloads.ChainInputs(workloads.f32_to_bf16_bits(l), ids, q, np.full(bs, 0.9, np.float32),
                                    rng.integers(0, 2**63, size=bs).astype(np.uint64), False, "top-p overflow")
        tp = np.array([0.5, 0.7, 0.95, 0.2], np.float32)
    tp = tp.astype(np.float32)
    check_chain(inp, dev, top_p=tp)
    if inp.logits.dtype == np.uint16:
        outs = []
        for tk in (None, np.zeros(inp.batch, np.int32)):
            out = sv.verify_chain(_t(inp.logits, dev), _t(inp.draft_ids, dev), _t(inp.temperature, dev),
                                  _t(inp.seeds, dev), draft_probs=_t(inp.draft_probs, dev), return_p_draft=True,
                                  top_k=_t(tk, dev), top_p=_t(tp, dev))
            torch.cuda.synchronize()
            outs.append(_np(out))
        _same(outs[0], outs[1], f"top-p alone {case}: value counts vs passes over the row")


def test_filtered_with_one_array_only(dev):
    """top_k alone and top_p alone (the other pointer NULL), chain and tree."""
    inp = _random_chain(71, 10, 4, 7000, "bf16", "probs")
    tk, tp = _filters(np.random.default_rng(71), 10, 7000)
    check_chain(inp, dev, top_k=tk)
    check_chain(inp, dev, top_p=tp)
    check_chain(inp, dev, flags=sv.FLAG_BLOCK, top_p=tp)
    tree = _random_tree_inputs(72, 6, 8, 5000, "f32")
    tk6, tp6 = _filters(np.random.default_rng(72), 6, 5000)
    check_tree(tree, dev, top_k=tk6)
    check_tree(tree, dev, top_p=tp6)


# ------------------------------- top-k thresholds from candidate groups
# For top-k up to 128 the statistics pass keeps the groups the kept set can
# come from and the thresholds pass reads only those; FLAG_KF_ROWS makes it
# read the rows instead.  The two give bit-identical results, and the
# candidate path is compared with the oracle as well.
def _same(a, b, name):
    for key in ("accept_len", "tokens", "status", "accept_path"):
        if key in a:
            np.testing.assert_array_equal(a[key], b[key], err_msg=f"{name}: {key}")
    if "p_draft" in a:
        np.testing.assert_array_equal(a["p_draft"].view(np.uint64), b["p_draft"].view(np.uint64),
                                      err_msg=f"{name}: p_draft bits")


def _chain_both_paths(inp, dev, tk, tp, flags=0, logits=None):
    outs = []
    for f in (flags, flags | sv.FLAG_KF_ROWS):
        print(f"[parity] top-k candidates {inp.name} flags={f}", flush=True)
        out = sv.verify_chain(_t(inp.logits, dev) if logits is None else logits, _t(inp.draft_ids, dev),
                              _t(inp.temperature, dev), _t(inp.seeds, dev),
                              draft_probs=None if inp.onehot else _t(inp.draft_probs, dev), onehot=inp.onehot,
                              flags=f, return_p_draft=True, top_k=_t(tk, dev), top_p=_t(tp, dev))
        torch.cuda.synchronize()
        outs.append(_np(out))
    _same(outs[0], outs[1], inp.name)
    return outs[0]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_topk_candidates_equal_row_passes(dev, dtype):
    """k from 1 to 129 (the candidate path serves k <= 128), alone and with
    top-p, over rows of three and more statistics segments."""
    s = 310 + (dtype == "f32")
    inp = _random_chain(s, 24, 5, 50000, dtype, "probs")
    rng = np.random.default_rng(s)
    tk = rng.choice(np.array([1, 2, 7, 50, 64, 100, 127, 128, 129, 0], np.int32), size=24).astype(np.int32)
    tp = rng.choice(np.array([1.0, 1.0, 0.9, 0.5, 0.99], np.float32), size=24).astype(np.float32)
    _chain_both_paths(inp, dev, tk, tp)
    check_chain(inp, dev, top_k=tk, top_p=tp)


def test_topk_candidates_headline_shape(dev):
    """bs 64, k 7, V 128256 bf16 with top-k 50 and top-p 0.9 on every request."""
    inp = workloads.chain_bf16_mixed(4)
    tk = np.full(inp.batch, 50, np.int32)
    tp = np.full(inp.batch, 0.9, np.float32)
    _chain_both_paths(inp, dev, tk, tp)
    check_chain(inp, dev, top_k=tk, top_p=tp)


def test_topk_candidates_ties_and_short_rows(dev):
    """Ties at the k-th logit (few distinct values, some rows all equal, so
    lists overflow and rows are read instead), mostly -inf rows, rows shorter
    than one sub-chunk, and rows that end inside a group."""
    rng = np.random.default_rng(333)
    for V, name in ((5000, "ties"), (300, "short"), (4099, "ragged")):
        bs, k = 10, 3
        l = (rng.standard_normal((bs, k + 1, V)) * 2).astype(np.float32)
        l[0] = np.round(l[0])                       # a handful of values
        l[1] = 0.25                                 # every logit equal
        l[2, :, 40:] = -np.inf                      # 40 finite entries
        l[3, :, : V // 2] = np.round(l[3, :, : V // 2] * 4) / 4
        q = workloads._softmax_rows(l[:, :k].reshape(-1, V) * 0.7).reshape(bs, k, V).astype(np.float32)
        ids = workloads._sample_rows(rng, q.reshape(-1, V)).reshape(bs, k).astype(np.int32)
        temp = np.full(bs, 0.8, np.float32)
        temp[7] = 0.0
        tk = np.array([5, 50, 60, 128, 1, 3, 20, 9, 100, 64], np.int32)
        tp = np.array([1.0, 0.9, 1.0, 0.7, 1.0, 0.95, 1.0, 0.5, 0.8, 1.0], np.float32)
        for dtype in ("f32", "bf16"):
            lg = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(l)) if dtype == "bf16" else l
            ll = workloads.f32_to_bf16_bits(l) if dtype == "bf16" else l
            inp = workloads.ChainInputs(ll, ids, q, temp, rng.integers(0, 2**63, size=bs).astype(np.uint64), False,
                                        f"candidates {name} {dtype}")
            assert np.isfinite(lg).any()
            _chain_both_paths(inp, dev, tk, tp)
            check_chain(inp, dev, top_k=tk, top_p=tp)


def test_topk_candidates_unaligned_rows(dev):
    """A strided view whose rows are not 16-byte aligned: the statistics pass
    and the thresholds pass both take scalar loads."""
    base = _random_chain(334, 6, 3, 9010, "f32", "probs")
    V = 9001
    lg = torch.from_numpy(base.logits).to(dev)[:, :, :V]
    l = np.ascontiguousarray(base.logits[:, :, :V])
    q = workloads._softmax_rows(l[:, :3].reshape(-1, V)).reshape(6, 3, V).astype(np.float32)
    ids = np.minimum(base.draft_ids, V - 1).astype(np.int32)
    inp = workloads.ChainInputs(l, ids, q, base.temperature, base.seeds, False, "candidates strided")
    tk = np.array([10, 50, 128, 1, 77, 3], np.int32)
    tp = np.array([1.0, 0.9, 0.6, 1.0, 0.95, 1.0], np.float32)
    got = _chain_both_paths(inp, dev, tk, tp, logits=lg)
    ref = oracle.verify_chain(l, ids, base.temperature, base.seeds, draft_probs=q, top_k=tk, top_p=tp)
    _compare(ref, got, "candidates strided", kind="filtered chain")


def test_topk_candidates_trees(dev):
    inp = _random_tree_inputs(335, 9, 8, 33000, "bf16")
    rng = np.random.default_rng(335)
    tk = rng.choice(np.array([1, 20, 50, 128, 200], np.int32), size=9).astype(np.int32)
    tp = rng.choice(np.array([1.0, 0.9], np.float32), size=9).astype(np.float32)
    outs = []
    for f in (0, sv.FLAG_KF_ROWS):
        out = sv.verify_tree(_t(inp.logits, dev), _t(inp.node_tokens, dev), _t(inp.parent, dev),
                             _t(inp.temperature, dev), _t(inp.seeds, dev), flags=f, top_k=_t(tk, dev),
                             top_p=_t(tp, dev))
        torch.cuda.synchronize()
        outs.append(_np(out))
    _same(outs[0], outs[1], "candidate trees")
    check_tree(inp, dev, top_k=tk, top_p=tp)


# ------------------------------------------------- the give-up path of waits
@pytest.mark.parametrize("drafts", ["probs", "onehot"])
def test_abort_flag_gives_internal_status_and_reset_recovers(dev, drafts):
    """The workspace's abort flag, set from the host before a fused call:
    every bounded wait of the call gives up at its first poll (every kernel
    still ends), the requests whose work waited report REQ_INTERNAL and the
    others are still correct; re-initialising the workspace restores a call
    that matches the oracle in full, with draft probabilities and with
    one-hot drafts."""
    inp = workloads.chain_bf16_mixed(6, bs=32, k=5, V=20000)
    probs = inp.draft_probs if drafts == "probs" else None
    ws = sv.Workspace(sv.chain_workspace_bytes(inp.batch, inp.max_draft, inp.vocab, sv.BF16), dev)
    off = ws.base - ws.buf.data_ptr()
    args = (_t(inp.logits, dev), _t(inp.draft_ids, dev), _t(inp.temperature, dev), _t(inp.seeds, dev))
    onehot = probs is None
    ref = oracle.verify_chain(inp.logits, inp.draft_ids, inp.temperature, inp.seeds, draft_probs=probs, onehot=onehot)
    # a request's status is written once its outputs are final (the race's
    # merge writes OK after the token), so a request that does not report
    # REQ_INTERNAL is complete however the give-ups interleave; three calls,
    # each on a re-initialised workspace
    for rep in range(3):
        print(f"[parity] abort flag set before a fused call ({drafts}, {rep})", flush=True)
        ws.buf[off:off + 4].view(torch.int32).fill_(1)
        out = _np(sv.verify_chain(*args, draft_probs=_t(probs, dev), onehot=onehot, flags=sv.FLAG_FUSED, workspace=ws))
        torch.cuda.synchronize()
        internal = out["status"] == sv.REQ_INTERNAL
        assert internal.any(), "no wait gave up"
        assert int(ws.buf[off:off + 4].view(torch.int32).item()) == 1
        ok = ~internal
        np.testing.assert_array_equal(out["status"][ok], ref["status"][ok])
        margin_ok = ok & (ref["min_margin"] >= MARGIN)
        np.testing.assert_array_equal(out["accept_len"][margin_ok], ref["accept_len"][margin_ok])
        np.testing.assert_array_equal(out["tokens"][margin_ok], ref["tokens"][margin_ok])
        print(f"[parity]   {int(internal.sum())} of {inp.batch} requests reported REQ_INTERNAL; resetting", flush=True)
        ws.reset()
    got = _np(sv.verify_chain(*args, draft_probs=_t(probs, dev), onehot=onehot, flags=sv.FLAG_FUSED, workspace=ws))
    torch.cuda.synchronize()
    assert int(ws.buf[off:off + 4].view(torch.int32).item()) == 0
    _compare(ref, got, "after reset", kind="chain")
