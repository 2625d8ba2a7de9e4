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
rejected (renormalised by S). Taking x1 with probability p(x1), else x2 with
p(x2) / (1 - p(x1)), ..., else the rest, gives every token probability
exactly p, at every depth: the committed stream is distributed as plain
sampling from the target.

Random numbers: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC'11), key = the 64-bit seed (low word
first), counter = (step, depth, draw, lane); u = (first output word >> 8) *
2^-24, in [0, 1). step 0 is the prefill's token and step i the i-th verify;
draw j is the test of the j-th child at that depth, 0xFFFF the residual draw;
lane is the sequence's index when several sequences are served together (0
for one). The pages speak of one sequence; the fourth counter word giving
each sequence of a batch its own stream is this implementation's choice.

Precision (the GPU takes these decisions in fp32, so the oracle takes them
in the same precision): e(v) = exp((l(v) - max l) / T) in float32, Z = the
float64 sum of e rounded to float32, p(v) = e(v) / Z in float32; the child
test is u * S < p(x) with S in float32; the residual draw walks the tokens
in id order accumulating e(v) in float64 and takes the first v whose running
sum exceeds (u * S) * Z (the product u * S in float32, then times Z in
float64), or the last token left with e(v) > 0 if rounding leaves the sum
short. (In exact arithmetic this is the walk over p = e / Z with target
u * S; counting in units of e spares a division per token.)
"""
from __future__ import annotations

import numpy as np

MASK32 = 0xFFFFFFFF
PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85
RESIDUAL_DRAW = 0xFFFF


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


def uniform(seed: int, step: int, depth: int, draw: int, lane: int = 0) -> np.float32:
    """u in [0, 1) with 24 random bits, from the counter (step, depth, draw, lane)."""
    w = philox4x32((step, depth, draw, lane), (seed & MASK32, (seed >> 32) & MASK32))[0]
    return np.float32((w >> 8) * (1.0 / 16777216.0))


def row_probs(logits_row, temperature: float):
    """(e, Z): e(v) = exp((l(v) - max) / T) in float32 and Z = sum e (float64 sum, float32)."""
    l = np.asarray(logits_row, dtype=np.float32)
    inv_t = np.float32(1.0) / np.float32(temperature)
    e = np.exp((l - l.max()) * inv_t).astype(np.float32)
    z = np.float32(np.sum(e.astype(np.float64)))
    return e, z


def residual_draw(e, z, removed, S: np.float32, u: np.float32) -> int:
    """Token drawn from p = e / Z restricted to tokens not in `removed`."""
    t = float(np.float32(u * S)) * float(z)
    keep = np.ones(len(e), dtype=bool)
    keep[list(removed)] = False
    cum = 0.0
    last = -1
    for v in range(len(e)):
        if not keep[v]:
            continue
        if e[v] > 0:
            last = v
        cum += float(e[v])
        if cum > t:
            return v
    return last


def sample_token(logits_row, temperature: float, seed: int, step: int, depth: int = 0,
                 lane: int = 0) -> int:
    """One token drawn from softmax(logits / T) (the prefill's token)."""
    e, z = row_probs(logits_row, temperature)
    return residual_draw(e, z, (), np.float32(1.0), uniform(seed, step, depth, RESIDUAL_DRAW, lane))


def accept_sample(token_rows, parent_rows, logits, temperature: float, seed: int, step: int,
                  max_depth: int, lane: int = 0):
    """Sampling-mode acceptance walk over the verify rows.

    logits[r] are the target's logits at verify row r. Returns (accepted rows
    in order, the token drawn at the last row) like the greedy walk.
    """
    n = len(token_rows)
    cur, path, depth = 0, [], 0
    while True:
        e, z = row_probs(logits[cur], temperature)
        S = np.float32(1.0)
        removed = []
        children = [r for r in range(1, n) if parent_rows[r] == cur] if depth < max_depth else []
        nxt = -1
        for j, r in enumerate(children):
            x = int(token_rows[r])
            px = np.float32(e[x] / z)
            if np.float32(uniform(seed, step, depth, j, lane) * S) < px:
                nxt = r
                break
            S = np.float32(S - px)
            removed.append(x)
        if nxt < 0:
            return path, residual_draw(e, z, removed, S,
                                       uniform(seed, step, depth, RESIDUAL_DRAW, lane))
        path.append(nxt)
        cur = nxt
        depth += 1
