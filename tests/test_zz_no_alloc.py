"""sv_verify_chain_noalloc (the workspace-free variant of sv_verify_chain,
for callers that cannot allocate) against sv_verify_chain, through the C
ABI: the same kernels on the same inputs give the same outputs bit for bit.
Two calls in a row, the second with a smaller input, so the second runs on
the array the first left behind; then the scratch's limits."""
import ctypes

import numpy as np
import pytest
import torch

import lossless_draft_verification_amd as sv
import workloads
from lossless_draft_verification_amd import _lib

pytestmark = pytest.mark.gpu


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


def _both(inp, dev, **kw):
    args = (_t(inp.logits, dev), _t(inp.draft_ids, dev), _t(inp.temperature, dev), _t(inp.seeds, dev))
    q = None if inp.onehot else _t(inp.draft_probs, dev)
    print(f"[no-alloc] {inp.name} bs={inp.batch} k={inp.max_draft} V={inp.vocab} {kw}", flush=True)
    ref = sv.verify_chain(*args, draft_probs=q, onehot=inp.onehot, return_p_draft=True,
                          workspace=sv.Workspace(1 << 20, dev), **kw)
    got = sv.verify_chain_noalloc(*args, draft_probs=q, onehot=inp.onehot, return_p_draft=True, **kw)
    torch.cuda.synchronize()
    for name in ref:
        a, b = ref[name].cpu().numpy(), got[name].cpu().numpy()
        np.testing.assert_array_equal(a, b, err_msg=f"{inp.name}: {name}")
    return got


def test_noalloc_matches_the_workspace_call_twice_then_smaller(dev):
    # the headline shape, then a smaller call on the array it left behind
    big = workloads.chain_bf16_mixed(0)
    out = _both(big, dev)
    assert (out["status"].cpu().numpy() == 0).all()
    small = workloads.chain_fp32(1)
    _both(small, dev)
    _both(workloads.chain_small(0), dev)


def test_noalloc_filtered_and_block(dev):
    inp = workloads.chain_bf16_mixed(2, bs=16)
    tk = torch.full((16,), 50, dtype=torch.int32, device=dev)
    tp = torch.full((16,), 0.9, dtype=torch.float32, device=dev)
    _both(inp, dev, top_k=tk, top_p=tp)
    _both(inp, dev, flags=sv.FLAG_BLOCK)
    _both(inp, dev, flags=sv.FLAG_FUSED)


def test_noalloc_rejects_shapes_beyond_the_scratch(dev):
    inp = workloads.chain_small(0)
    bs = sv.SCRATCH_MAX_BATCH + 1
    logits = torch.zeros((bs, 4, 1000), dtype=torch.float32, device=dev)
    ids = torch.zeros((bs, 3), dtype=torch.int32, device=dev)
    temp = torch.ones(bs, dtype=torch.float32, device=dev)
    seeds = torch.arange(bs, dtype=torch.int64, device=dev)
    q = torch.full((bs, 3, 1000), 1e-3, dtype=torch.float32, device=dev)
    with pytest.raises(sv.SpecVerifyError) as e:
        sv.verify_chain_noalloc(logits, ids, temp, seeds, draft_probs=q)
    assert e.value.status == _lib.ERR_WORKSPACE_TOO_SMALL
    # a vocabulary whose race records exceed the array
    V = 1 << 24
    bs = 64
    logits = torch.zeros((bs, 1, V), dtype=torch.bfloat16, device=dev)
    with pytest.raises(sv.SpecVerifyError) as e:
        sv.verify_chain_noalloc(logits, torch.zeros((bs, 0), dtype=torch.int32, device=dev),
                                torch.ones(bs, dtype=torch.float32, device=dev),
                                torch.arange(bs, dtype=torch.int64, device=dev), onehot=True)
    assert e.value.status == _lib.ERR_WORKSPACE_TOO_SMALL
