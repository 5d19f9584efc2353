"""Counters shared by the GPU parity tests of one pytest session.

Every comparison of a verify call with the oracle adds the oracle's decision
count and the requests exempted for a near-tie (a decision margin below
1e-6, or a top-p cut gap below 1e-9); the last GPU module checks the totals
against the bound of fewer than 1e-4 exemptions per decision.
"""
STATS = {"decisions": 0, "exempt": 0, "calls": 0, "requests": 0}
BY_KIND: dict = {}


def count(kind: str, decisions: int, exempt: int, requests: int):
    STATS["decisions"] += decisions
    STATS["exempt"] += exempt
    STATS["calls"] += 1
    STATS["requests"] += requests
    k = BY_KIND.setdefault(kind, {"decisions": 0, "exempt": 0, "calls": 0})
    k["decisions"] += decisions
    k["exempt"] += exempt
    k["calls"] += 1
