"""GPU parity of the survival top-k draft budget (sv_plan_budget) with the
oracle: the budget and every request's admitted length bit for bit, the
rate within 1e-12 relative; a case whose oracle rate margin (relative gap
between the best rate and the next distinct one) is below 1e-12 may differ
only in the budget's choice among near-equal rates, and is counted."""
import json
import os

import numpy as np
import pytest
import torch

import lossless_draft_verification_amd as sv
import oracle

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d = torch.device("cuda", 0)
    torch.cuda.set_device(d)
    return d


def check(conf, cost, base, dev, num_steps=None, name=""):
    print(f"[plan] {name} bs={conf.shape[0]} K={conf.shape[1]} table={len(cost) - 1}", flush=True)
    ref = oracle.plan_budget(conf, cost, base, num_steps=num_steps)
    out = sv.plan_budget(torch.from_numpy(np.ascontiguousarray(conf)).to(dev), torch.from_numpy(np.asarray(cost, np.float64)).to(dev),
                         base, num_steps=None if num_steps is None else torch.from_numpy(np.asarray(num_steps, np.int32)))
    torch.cuda.synchronize()
    got_b = int(out["budget"].item())
    got_len = out["draft_len"].cpu().numpy()
    got_rate = float(out["rate"].item())
    if ref["margin"] < 1e-12:
        return ref, got_b, got_len, True
    assert got_b == ref["budget"], (name, got_b, ref["budget"])
    np.testing.assert_array_equal(got_len, ref["draft_len"], err_msg=name)
    if np.isfinite(ref["rate"]):
        assert got_rate == pytest.approx(ref["rate"], rel=1e-12), name
    else:
        assert got_rate == ref["rate"], name
    return ref, got_b, got_len, False


def test_page_worked_example_on_gpu(dev):
    from test_oracle_plan import _page_example
    for case, conf, cost, _, _, _ in _page_example():
        ref, b, lens, exempt = check(conf, cost, float(case["batch"]), dev, name=f"page batch {case['batch']}")
        assert not exempt and b == case["admitted"]


@pytest.mark.parametrize("seed,bs,K", [(1, 1, 1), (2, 3, 5), (3, 16, 7), (4, 100, 8), (5, 257, 3), (6, 512, 7),
                                       (7, 512, 16), (8, 1024, 8), (9, 8192, 1), (10, 128, 64), (11, 2048, 4),
                                       (12, 1170, 7), (13, 3, 64)])
def test_random_plans(dev, seed, bs, K):
    rng = np.random.default_rng(seed)
    conf = rng.beta(4, 1.2, size=(bs, K)).astype(np.float32)
    if seed % 2:
        conf = np.round(conf * 8) / 8            # many exact ties
    conf[rng.random((bs, K)) < 0.02] = 1.0
    num_steps = rng.integers(0, K + 1, size=bs) if seed % 3 else None
    n = bs * K
    table = n if seed % 4 else max(1, n // 3)
    steps = np.arange(table + 1)
    cost = 1.0 + np.maximum(0, steps - rng.integers(0, n + 1)) * rng.random() * 5.0 / max(n, 1)
    if seed % 5 == 0:
        cost = 1.0 + np.ceil((steps + 1) / 64) * 0.1   # a step function (padding buckets)
    check(conf, cost, float(bs), dev, num_steps=num_steps, name=f"random {seed}")


def test_edge_inputs(dev):
    conf = np.array([[np.nan, 0.9, 2.0], [1.5, -0.2, 0.5], [0.0, 0.7, 0.7]], np.float32)
    check(conf, np.ones(10), 1.0, dev, num_steps=np.array([3, 5, -1]), name="clamps")
    check(np.full((4, 4), 0.5, np.float32), np.ones(1), 2.0, dev, name="zero table")
    check(np.full((4, 4), 1.0, np.float32), np.linspace(1, 2, 17), 4.0, dev, name="all ones")
    check(np.zeros((8, 3), np.float32), np.ones(25), 8.0, dev, name="all zero")
    # ties between requests and positions decided by the tie rule
    conf = np.array([[1.0, 0.5], [0.5, 0.5], [0.5, 1.0]], np.float32)
    check(conf, np.array([10.0, 1.0, 1.0, 1.0, 1e9, 1e9, 1e9]), 0.0, dev, name="tie rule")


def test_plan_is_deterministic(dev):
    rng = np.random.default_rng(0)
    conf = torch.from_numpy(rng.random((777, 9)).astype(np.float32)).to(dev)
    cost = torch.from_numpy(1.0 + np.arange(777 * 9 + 1) * 1e-4).to(dev)
    a = sv.plan_budget(conf, cost, 777.0)
    b = sv.plan_budget(conf, cost, 777.0)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_workspace_reuse_across_shapes(dev):
    """One caller workspace serves plans of every shape in turn, whatever an
    earlier call or anything else left in it: before some calls it is filled
    with random bytes (so entries of the sorted list past the drafted count
    hold stale or non-finite keys), or with zeros (keys whose score bits are
    NaN); num_steps leaves fewer drafted slots than the table covers."""
    ws = torch.zeros(sv.plan_workspace_bytes(1024, 8), dtype=torch.uint8, device=dev)
    cases = ((31, 1024, 8, None), (32, 3, 5, "random"), (33, 512, 7, None), (34, 1, 1, "zero"),
             (35, 1024, 8, "random"), (36, 512, 7, "zero"), (37, 1000, 8, "random"))
    for seed, bs, K, fill in cases:
        rng = np.random.default_rng(seed)
        conf = rng.beta(4, 1.2, size=(bs, K)).astype(np.float32)
        cost = 1.0 + np.arange(bs * K + 1) * rng.random() * 5.0 / (bs * K)
        num_steps = rng.integers(0, K + 1, size=bs).astype(np.int32) if fill else None
        if fill == "random":
            ws.copy_(torch.from_numpy(rng.integers(0, 256, size=ws.numel(), dtype=np.uint8)).to(dev))
        elif fill == "zero":
            ws.zero_()
        print(f"[plan] workspace reuse bs={bs} K={K} fill={fill}", flush=True)
        ref = oracle.plan_budget(conf, cost, float(bs), num_steps=num_steps)
        out = sv.plan_budget(torch.from_numpy(conf).to(dev), torch.from_numpy(cost).to(dev), float(bs),
                             num_steps=None if num_steps is None else torch.from_numpy(num_steps), workspace=ws)
        torch.cuda.synchronize()
        assert np.isfinite(float(out["rate"].item())) == np.isfinite(ref["rate"])
        if ref["margin"] >= 1e-12:
            assert int(out["budget"].item()) == ref["budget"]
            np.testing.assert_array_equal(out["draft_len"].cpu().numpy(), ref["draft_len"])
            assert float(out["rate"].item()) == pytest.approx(ref["rate"], rel=1e-12)


def test_unaligned_confidences(dev):
    """Confidences whose address is not 16-byte aligned (a view one float
    into a larger buffer) take the word-by-word staging path."""
    for seed, bs, K in ((41, 512, 7), (42, 1024, 8), (43, 33, 6)):
        rng = np.random.default_rng(seed)
        conf = rng.beta(4, 1.2, size=(bs, K)).astype(np.float32)
        cost = 1.0 + np.arange(bs * K + 1) * rng.random() * 5.0 / (bs * K)
        flat = torch.zeros(bs * K + 1, dtype=torch.float32, device=dev)
        flat[1:] = torch.from_numpy(conf.ravel()).to(dev)
        view = flat[1:].view(bs, K)
        assert view.data_ptr() % 16 != 0
        print(f"[plan] unaligned confidences bs={bs} K={K}", flush=True)
        ref = oracle.plan_budget(conf, cost, float(bs))
        out = sv.plan_budget(view, torch.from_numpy(cost).to(dev), float(bs))
        torch.cuda.synchronize()
        if ref["margin"] >= 1e-12:
            assert int(out["budget"].item()) == ref["budget"]
            np.testing.assert_array_equal(out["draft_len"].cpu().numpy(), ref["draft_len"])
