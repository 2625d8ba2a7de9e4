"""Expected tokens per step and speedup of chain speculative decoding.

TEST INFRASTRUCTURE (see the package docstring). Pinned by the printed
numbers of [L13] "The math behind the speedup with small numbers".

Model ([L13] same section): each of the k drafted tokens is accepted with
probability alpha given that every earlier one was; the first rejection ends
the step, and the step always adds the target's own token. Written here from
the distribution of the accepted length L rather than as a geometric sum:

    P(L = j) = alpha^j (1 - alpha)   for j < k     (j accepted, then a miss)
    P(L = k) = alpha^k                             (all k accepted)
    tokens per step = E[L + 1] = sum_j (j + 1) P(L = j)

A step costs one target pass plus k draft passes of relative cost c, so the
speedup over plain decoding (one token per target pass) is E[L + 1] / (1 + k c).
A reporting helper only; not part of the decoding path.
"""
from __future__ import annotations


def accepted_length_pmf(alpha: float, k: int) -> list:
    """[P(L = 0), ..., P(L = k)] for k drafted tokens."""
    pmf = []
    reach = 1.0                      # probability that the first j drafts were accepted
    for _ in range(k):
        pmf.append(reach * (1.0 - alpha))
        reach *= alpha
    pmf.append(reach)
    return pmf


def expected_tokens(alpha: float, k: int) -> float:
    return sum((j + 1) * p for j, p in enumerate(accepted_length_pmf(alpha, k)))


def speedup(alpha: float, k: int, draft_cost: float) -> float:
    return expected_tokens(alpha, k) / (1.0 + k * draft_cost)


def best_k(alpha: float, draft_cost: float, k_max: int = 6) -> int:
    """The draft length in 1..k_max with the highest speedup (smallest on ties)."""
    best, best_s = 1, speedup(alpha, 1, draft_cost)
    for k in range(2, k_max + 1):
        s = speedup(alpha, k, draft_cost)
        if s > best_s:
            best, best_s = k, s
    return best
