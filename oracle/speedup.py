"""Expected tokens per step and speedup of chain speculative decoding.

[L13] "The math behind the speedup with small numbers": with per-token
acceptance alpha (given the earlier ones were accepted), k drafted tokens
and a draft pass costing c target passes, one step commits on average
1 + alpha + ... + alpha^k tokens and costs 1 + k*c target passes.
A reporting helper only; not part of the decoding path.
"""
from __future__ import annotations


def expected_tokens(alpha: float, k: int) -> float:
    return sum(alpha ** i for i in range(k + 1))


def speedup(alpha: float, k: int, draft_cost: float) -> float:
    return expected_tokens(alpha, k) / (1.0 + k * draft_cost)


def best_k(alpha: float, draft_cost: float, k_max: int = 6) -> int:
    return max(range(1, k_max + 1), key=lambda k: speedup(alpha, k, draft_cost))
