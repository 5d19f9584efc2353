"""GPU checks of the benchmark's measurement aids: the read-ceiling stream
(sv_stream_read) touches every byte once (its per-workgroup XOR words fold
to the XOR of the whole buffer), and the prepared tree call equals the
plain one."""
import numpy as np
import pytest
import torch

import lossless_draft_verification_amd as sv
import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d = torch.device("cuda", 0)
    torch.cuda.set_device(d)
    return d


@pytest.mark.parametrize("nbytes,grid", [(16, 1), (4096 * 16, 3), (1000 * 16 * 257, 1536), (1 << 24, 8192)])
def test_stream_read_reads_every_word_once(dev, nbytes, grid):
    print(f"[aids] stream_read bytes={nbytes} grid={grid}", flush=True)
    rng = np.random.default_rng(nbytes + grid)
    words = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).to(dev)
    sink = torch.zeros(grid, dtype=torch.int32, device=dev)
    sv.stream_read(src, sink, grid)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(words))


def test_prepared_tree_equals_the_plain_call(dev):
    t = workloads.tree_fp32(2, bs=12)
    args = [torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (t.logits, t.node_tokens, t.parent, t.temperature)]
    seeds = torch.from_numpy(t.seeds.view(np.int64)).to(dev)
    ref = sv.verify_tree(*args, seeds)
    pt = sv.PreparedTree(*args, seeds, workspace=sv.Workspace(1 << 20, dev))
    pt.launch()
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(ref[k], pt.out[k]), k
    o = oracle.verify_tree(t.logits, t.node_tokens, t.parent, t.temperature, t.seeds)
    near = o["min_margin"] < 1e-6
    assert (pt.out["tokens"].cpu().numpy()[~near] == o["tokens"][~near]).all()
    pt.launch(phase_flag=sv.FLAG_STATS_ONLY)
    pt.launch(phase_flag=sv.FLAG_DECIDE_ONLY)
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(ref[k], pt.out[k]), k
