"""Sampling-mode (temperature > 0) acceptance over a verified draft tree.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  [L13] "Speculative decoding in four moves": drafted tokens are kept from the
        left while they pass the acceptance test; with sampling that test is
        the rejection-sampling rule, and at the first rejection the target
        supplies the token. The rule makes the output distribution exactly
        the target's own ("Lossless" in the glossary).
  [E2]  "How it works" for the mask builder: after reranking, strict
        speculative sampling selects one branch and corrects it as the target
        distribution requires.

Reading (the pages do not spell out the rule for several branches): the
tree's candidates are chosen deterministically (top-k by draft confidence,
then reranked), so each candidate is proposed with probability one. The
rejection test for a proposal made with probability one accepts candidate x
with probability p(x) / S, where p is the target's distribution at the
current row (softmax of logits / T) and S the mass not yet rejected at that
row. A rejected candidate's token leaves the distribution (S -= p(x)). The
children of a row are tried in row order. When every child is rejected, or
the row has none, the token is drawn from p restricted to the tokens not
rejected, by inverting its cumulative distribution in token-id order.
Taking x1 with probability p(x1), else x2 with p(x2) / (1 - p(x1)), ...,
else the rest, gives every token probability exactly p, at every depth: the
committed stream is distributed as plain sampling from the target.

Random numbers: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC'11), key = the 64-bit seed (low word
first), counter = (step, depth, draw, lane); u = (first output word >> 8) *
2^-24, in [0, 1). step 0 is the prefill's token and step i the i-th verify;
draw j is the test of the j-th child at that depth, 0xFFFF the residual draw;
lane is the sequence's index when several sequences are served together (0
for one). The pages speak of one sequence; the fourth counter word giving
each sequence of a batch its own stream is this implementation's choice.

Precision: everything here is float64 and follows the definitions above
literally (p = exp(l / T - max) / sum, the test u * S < p(x), the residual
target u * S against the running sum of p). An implementation that takes
these decisions in float32 can only differ from them where the two compared
quantities are closer than its rounding error. That error is bounded, in
probability units, by about 2e-7 * (sum over v of p(v) * |l(v) - max| / T)
+ 4e-7: the float32 exponent argument and exp, the normalising sum and the
product u * S. The sum is at most 2 ln V (the entropy plus ln Z), so the
bound stays under 5.1e-6 for V <= 2^17. Every decision therefore carries a
margin (the distance between its two compared quantities), and a decision
whose margin is at most TIE = 1e-5, about twice that bound, is a near-tie:
either outcome is correct there. The walk takes the oracle's own outcome
unless it is told which outcome an implementation took (`follow`), in which
case it takes that one at near-ties and its own everywhere else.
"""
from __future__ import annotations

import numpy as np

MASK32 = 0xFFFFFFFF
PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85
RESIDUAL_DRAW = 0xFFFF
TIE = 1e-5


def philox4x32(ctr, key, rounds: int = 10):
    """Philox4x32-R block function: 4 x 32-bit counter, 2 x 32-bit key."""
    c0, c1, c2, c3 = (int(v) & MASK32 for v in ctr)
    k0, k1 = (int(v) & MASK32 for v in key)
    for r in range(rounds):
        if r:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0) & MASK32, p1 & MASK32, ((p0 >> 32) ^ c3 ^ k1) & MASK32, p0 & MASK32
    return c0, c1, c2, c3


def uniform(seed: int, step: int, depth: int, draw: int, lane: int = 0) -> float:
    """u in [0, 1) with 24 random bits, from the counter (step, depth, draw, lane)."""
    w = philox4x32((step, depth, draw, lane), (seed & MASK32, (seed >> 32) & MASK32))[0]
    return (w >> 8) * (1.0 / 16777216.0)


def probs(logits_row, temperature: float) -> np.ndarray:
    """p = softmax(logits / T), float64."""
    x = np.asarray(logits_row, dtype=np.float64) / float(temperature)
    e = np.exp(x - x.max())
    return e / e.sum()


def residual_draw(p, removed, S: float, u: float):
    """Token drawn from p restricted to the tokens not in `removed` (whose
    mass is S): the first token, in id order, whose running sum of p exceeds
    u * S. Returns (token, margin), the margin being the distance from u * S
    to the nearer end of that token's interval. If rounding leaves the
    running sum short of u * S, the last token left with p > 0 is taken,
    with margin 0."""
    t = u * S
    keep = np.ones(len(p), dtype=bool)
    keep[list(removed)] = False
    cum = 0.0
    last = -1
    for v in range(len(p)):
        if not keep[v]:
            continue
        if p[v] > 0:
            last = v
        before = cum
        cum += float(p[v])
        if cum > t:
            return v, min(t - before, cum - t)
    return last, 0.0


def residual_interval(p, removed, v: int):
    """[cum_before, cum_after) of token v in the restricted running sum."""
    keep = np.ones(len(p), dtype=bool)
    keep[list(removed)] = False
    before = float(np.sum(p[:v][keep[:v]]))
    return before, before + float(p[v])


def _residual(p, removed, S, u, want):
    """The residual draw, taking `want` instead where u * S lies within TIE of
    want's interval (a near-tie with the oracle's own choice)."""
    v, margin = residual_draw(p, removed, S, u)
    if want is not None and want != v and 0 <= want < len(p) and want not in removed:
        lo, hi = residual_interval(p, removed, want)
        t = u * S
        if lo - TIE <= t < hi + TIE and p[want] > 0:
            return want, margin
    return v, margin


def sample_token(logits_row, temperature: float, seed: int, step: int, depth: int = 0,
                 lane: int = 0, follow: int = None):
    """One token drawn from softmax(logits / T) (the prefill's token).
    Returns (token, margin)."""
    p = probs(logits_row, temperature)
    return _residual(p, (), 1.0, uniform(seed, step, depth, RESIDUAL_DRAW, lane), follow)


def walk(token_rows, parent_rows, logits, temperature: float, seed: int, step: int,
         max_depth: int, lane: int = 0, follow=None):
    """Sampling-mode acceptance walk over the verify rows.

    logits[r] are the target's logits at verify row r. Returns (accepted rows
    in order, the token drawn at the last row, margins), margins[d] being the
    smallest margin of the decisions that chose committed token d (every
    child test at that depth and the residual draw if one was made).

    `follow` is another implementation's committed tokens for the same walk;
    at a near-tie the walk takes the outcome those tokens show. Siblings
    carry distinct tokens and a rejected token leaves the residual, so child
    x was accepted exactly when the committed token at its depth is x.
    """
    n = len(token_rows)
    cur, path, depth, margins = 0, [], 0, []
    while True:
        p = probs(logits[cur], temperature)
        want = int(follow[depth]) if follow is not None and depth < len(follow) else None
        S = 1.0
        removed = []
        children = [r for r in range(1, n) if parent_rows[r] == cur] if depth < max_depth else []
        nxt, m_d = -1, np.inf
        for j, r in enumerate(children):
            x = int(token_rows[r])
            us = uniform(seed, step, depth, j, lane) * S
            m_d = min(m_d, abs(us - p[x]))
            take = us < p[x]
            if abs(us - p[x]) <= TIE and want is not None:
                take = want == x
            if take:
                nxt = r
                break
            S -= p[x]
            removed.append(x)
        if nxt < 0:
            v, m = _residual(p, removed, S, uniform(seed, step, depth, RESIDUAL_DRAW, lane), want)
            margins.append(min(m_d, m))
            return path, v, margins
        margins.append(m_d)
        path.append(nxt)
        cur = nxt
        depth += 1


def accept_sample(token_rows, parent_rows, logits, temperature: float, seed: int, step: int,
                  max_depth: int, lane: int = 0):
    """(accepted rows in order, the token drawn at the last row), like the
    greedy walk."""
    path, bonus, _ = walk(token_rows, parent_rows, logits, temperature, seed, step, max_depth, lane)
    return path, bonus


def check_walk(got, token_rows, parent_rows, logits, temperature: float, seed: int, step: int,
               max_depth: int, lane: int = 0):
    """Whether `got` (another implementation's committed tokens for this walk)
    is a correct outcome: equal to the oracle's walk, where every near-tie is
    resolved as `got` resolves it. Returns (ok, the oracle's tokens, the
    smallest decision margin on the walk)."""
    path, bonus, margins = walk(token_rows, parent_rows, logits, temperature, seed, step,
                                max_depth, lane, follow=list(got))
    want = [int(token_rows[r]) for r in path] + [int(bonus)]
    return [int(t) for t in got] == want, want, float(min(margins))
