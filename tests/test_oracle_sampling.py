"""Pins of the sampling-mode oracle (oracle/sampling.py): the published
Philox known answers, the greedy limit, exact residual draws on a small case,
the near-tie allowance, and losslessness: the committed tokens are distributed as the target's own
softmax ([L13] "Speculative decoding in four moves"; glossary "Lossless")."""
import json
import os

import numpy as np
import pytest

from oracle import sampling as S
from oracle import tree as T

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox_kat.json"), encoding="utf-8") as f:
        kat = json.load(f)
    for v in kat["vectors"]:
        ctr = [int(x, 16) for x in v["ctr"]]
        key = [int(x, 16) for x in v["key"]]
        assert [f"0x{w:08x}" for w in S.philox4x32(ctr, key)] == v["out"]


def test_uniform_is_24_bit_and_varies_with_every_counter_word():
    u = [S.uniform(7, s, d, j) for s in range(20) for d in range(5) for j in range(10)]
    arr = np.array(u, dtype=np.float64)
    assert arr.min() >= 0.0 and arr.max() < 1.0
    assert np.all((arr * (1 << 24)) == np.floor(arr * (1 << 24)))
    assert abs(arr.mean() - 0.5) < 0.03
    assert len(set(u)) > 0.99 * len(u)
    assert S.uniform(7, 1, 2, 3) != S.uniform(8, 1, 2, 3)      # the seed is the key
    assert S.uniform(7 << 32, 1, 2, 3) != S.uniform(0, 1, 2, 3)
    # the fourth counter word is the sequence (lane) of a batch: lane 0 is the
    # single-sequence stream, other lanes are streams of their own
    assert S.uniform(7, 1, 2, 3, 0) == S.uniform(7, 1, 2, 3)
    lanes = [S.uniform(7, s, 0, 0, b) for b in range(8) for s in range(50)]
    assert len(set(lanes)) > 0.99 * len(lanes)


def test_residual_draw_small_case():
    p = np.array([1, 2, 3, 4], dtype=np.float64) / 10
    # token 1 rejected: S = 0.8; tokens 0, 2, 3 carry 0.1, 0.3, 0.4
    assert S.residual_draw(p, [1], 0.8, 0.0)[0] == 0
    v, m = S.residual_draw(p, [1], 0.8, 0.2)           # 0.16 in (0.1, 0.4]
    assert v == 2 and abs(m - 0.06) < 1e-12
    v, m = S.residual_draw(p, [1], 0.8, 0.6)           # 0.48 in (0.4, 0.8]
    assert v == 3 and abs(m - 0.08) < 1e-12
    assert S.residual_draw(p, [], 1.0, 0.95)[0] == 3
    # a mass larger than what is left (rounding): the last token left, margin 0
    assert S.residual_draw(p, [3], 0.61, 0.9999) == (2, 0.0)
    assert S.residual_interval(p, [1], 3) == (0.4, 0.8)


def _u(seed, step, depth, draw):
    return S.uniform(seed, step, depth, draw)


def test_near_ties_take_the_followed_outcome_and_nothing_else():
    """A child whose p(x) sits 4e-6 above u (a near-tie): the oracle accepts
    it, and a walk told that the other side rejected it follows that; at
    1e-3 above u the followed rejection is refused. The same for a residual
    draw landing 4e-6 inside a token's interval."""
    seed, step = 3, 9
    u0 = _u(seed, step, 0, 0)
    assert 0.05 < u0 < 0.95
    for gap, tie in ((4e-6, True), (1e-3, False)):
        px = u0 + gap
        # three tokens: x = 0 with p(x) = px, the rest split evenly (T = 1)
        logits = np.log(np.array([[px, (1 - px) / 2, (1 - px) / 2]]))
        tokens, parent = [0, 0], [-1, 0]
        lg = np.repeat(logits, 2, axis=0)
        path, bonus, margins = S.walk(tokens, parent, lg, 1.0, seed, step, max_depth=1)
        assert path == [1] and abs(margins[0] - gap) < 1e-9
        # the other outcome: x rejected, then the residual draw at depth 0
        ur = _u(seed, step, 0, S.RESIDUAL_DRAW)
        alt = 1 + int(ur * (1 - px) >= (1 - px) / 2)
        ok, want, m = S.check_walk([alt], tokens, parent, lg, 1.0, seed, step, 1)
        assert ok == tie and m <= gap + 1e-9
        ok, want, _ = S.check_walk([0, int(bonus)], tokens, parent, lg, 1.0, seed, step, 1)
        assert ok and want == [0, int(bonus)]
    ur = _u(seed, step, 0, S.RESIDUAL_DRAW)
    for gap, tie in ((4e-6, True), (1e-3, False)):
        # no children: the residual draw over p = (ur - gap, the rest / 2, the rest / 2)
        # lands `gap` past the end of token 0's interval
        p0 = ur - gap
        lg = np.log(np.array([[p0, (1 - p0) / 2, (1 - p0) / 2]]))
        v, m = S.residual_draw(S.probs(lg[0], 1.0), [], 1.0, ur)
        assert v == 1 and abs(m - gap) < 1e-9
        ok, _, _ = S.check_walk([0], [0], [-1], lg, 1.0, seed, step, 1)
        assert ok == tie
        # a token whose interval is far from u * S is never accepted
        ok, _, _ = S.check_walk([2], [0], [-1], lg, 1.0, seed, step, 1)
        assert not ok


def _random_tree(rng, n, depth_max):
    parent, depth = [-1], [0]
    for r in range(1, n):
        cands = [p for p in range(r) if depth[p] < depth_max]
        p = int(rng.choice(cands))
        parent.append(p)
        depth.append(depth[p] + 1)
    return parent


def test_low_temperature_is_the_greedy_walk():
    rng = np.random.default_rng(3)
    V = 50
    for trial in range(40):
        n = int(rng.integers(1, 12))
        parent = _random_tree(rng, n, 4)
        logits = (rng.standard_normal((n, V)) * 3).astype(np.float32)
        g = logits.argmax(axis=1)
        # drafted tokens: the greedy choice of the parent row half the time, distinct among siblings
        tokens = [0]
        for r in range(1, n):
            used = {tokens[c] for c in range(1, r) if parent[c] == parent[r]}
            want = int(g[parent[r]]) if rng.random() < 0.5 else int(rng.integers(V))
            while want in used:
                want = (want + 1) % V
            tokens.append(want)
        ref = T.accept(tokens, parent, g)
        got = S.accept_sample(tokens, parent, logits, 1e-4, seed=trial, step=1, max_depth=4)
        assert got == ref


def _chi2_ok(counts, probs, n):
    exp = probs * n
    keep = exp >= 5
    chi2 = float((((counts - exp) ** 2) / np.where(exp > 0, exp, 1))[keep].sum())
    dof = int(keep.sum()) - 1
    return chi2 < dof + 5 * np.sqrt(2 * dof) + 10, chi2, dof


def test_committed_tokens_follow_the_target_distribution():
    """First token ~ p(root); second token, given the first is child c, ~ p(c)."""
    rng = np.random.default_rng(11)
    V = 6
    T_ = 0.9
    # root -> children tokens 2, 0, 5 (rows 1, 2, 3); row 1 -> children 1, 4 (rows 4, 5)
    tokens = [0, 2, 0, 5, 1, 4]
    parent = [-1, 0, 0, 0, 1, 1]
    logits = (rng.standard_normal((6, V)) * 1.5).astype(np.float32)
    p0 = S.probs(logits[0], T_)
    p1 = S.probs(logits[1], T_)
    N = 20000
    first = np.zeros(V)
    second = np.zeros(V)
    n_second = 0
    for step in range(N):
        path, bonus = S.accept_sample(tokens, parent, logits, T_, seed=99, step=step, max_depth=2)
        seq = [tokens[r] for r in path] + [bonus]
        first[seq[0]] += 1
        if path and path[0] == 1:
            second[seq[1]] += 1
            n_second += 1
    ok, chi2, dof = _chi2_ok(first, p0, N)
    assert ok, (chi2, dof, first / N, p0)
    ok, chi2, dof = _chi2_ok(second, p1, n_second)
    assert ok, (chi2, dof, second / n_second, p1)


def test_sample_token_follows_softmax():
    rng = np.random.default_rng(5)
    l = rng.standard_normal(8).astype(np.float32)
    p = S.probs(l, 0.7)
    N = 20000
    c = np.zeros(8)
    for step in range(N):
        c[S.sample_token(l, 0.7, seed=4, step=step)[0]] += 1
    ok, chi2, dof = _chi2_ok(c, p, N)
    assert ok, (chi2, dof)


def test_session_low_temperature_is_greedy_and_sampling_is_seeded():
    import synth
    from oracle.loop import Session, greedy_decode
    from oracle.model import Config, Weights
    w = synth.workloads.get("c1")
    W = Weights(Config(w))
    p = synth.prompt(1, w["prompt_len"], w["vocab"])
    want, _, _ = greedy_decode(w, p, 24, W)
    cold = dict(w, temperature=1e-4, seed=5)
    assert Session(cold, W).generate(p, 24) == want
    hot = dict(w, temperature=1.0, seed=5)
    a = Session(hot, W).generate(p, 24)
    b = Session(hot, W).generate(p, 24)
    c = Session(dict(hot, seed=6), W).generate(p, 24)
    assert a == b and a != c
    assert all(0 <= t < w["vocab"] for t in a)
