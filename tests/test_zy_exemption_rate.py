"""The near-tie exemption bound over every GPU parity comparison of the
session (collected after the other GPU modules).

A request is compared with the oracle bit for bit unless one of the oracle's
decisions for it has a relative margin below 1e-6 (or a top-p cut gap below
1e-9), where fp32 and fp64 may legitimately disagree; such requests must be
fewer than 1e-4 of all decisions.  Every kind of call counts: chains (the
standard, one-hot and greedy rules), block-rule chains, trees, and filtered
chains and trees.
"""
import pytest

from _parity import BY_KIND, STATS

pytestmark = pytest.mark.gpu


def test_exemptions_over_the_session_are_below_1e_4_of_decisions():
    if STATS["calls"] == 0:
        pytest.skip("no parity comparison ran in this session")
    for kind, c in sorted(BY_KIND.items()):
        print(f"[parity] {kind}: calls {c['calls']}, decisions {c['decisions']}, exempt requests {c['exempt']}",
              flush=True)
    print(f"[parity] session: calls {STATS['calls']}, requests {STATS['requests']}, decisions {STATS['decisions']}, "
          f"exempt requests {STATS['exempt']}", flush=True)
    assert STATS["exempt"] < 1e-4 * STATS["decisions"], STATS
