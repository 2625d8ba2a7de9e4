"""Pins of the sampling-mode oracle (oracle/sampling.py): the published
Philox known answers, the greedy limit, exact residual draws on a small case,
and losslessness: the committed tokens are distributed as the target's own
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
    e = np.array([1, 2, 3, 4], dtype=np.float32)
    z = np.float32(10)
    # token 1 rejected: S = 0.8; tokens 0, 2, 3 carry 0.1, 0.3, 0.4
    s_left = np.float32(0.8)
    assert S.residual_draw(e, z, [1], s_left, np.float32(0.0)) == 0
    assert S.residual_draw(e, z, [1], s_left, np.float32(0.2)) == 2      # 0.16 in (0.1, 0.4]
    assert S.residual_draw(e, z, [1], s_left, np.float32(0.6)) == 3      # 0.48 in (0.4, 0.8]
    assert S.residual_draw(e, z, [], np.float32(1.0), np.float32(0.95)) == 3
    assert S.residual_draw(e, z, [3], np.float32(0.6), np.float32(0.9999)) == 2   # sum short: last left


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
    e0, z0 = S.row_probs(logits[0], T_)
    p0 = (e0 / z0).astype(np.float64)
    e1, z1 = S.row_probs(logits[1], T_)
    p1 = (e1 / z1).astype(np.float64)
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
    e, z = S.row_probs(l, 0.7)
    p = (e / z).astype(np.float64)
    N = 20000
    c = np.zeros(8)
    for step in range(N):
        c[S.sample_token(l, 0.7, seed=4, step=step)] += 1
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
