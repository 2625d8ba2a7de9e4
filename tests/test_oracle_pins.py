"""Pins of the oracle's tree policy and helpers to values the pages print.

Every expected value here is read from tests/golden/ (the pages' printed
numbers) or follows by hand arithmetic from them.
"""
import itertools
import json
import os
import re

import numpy as np
import pytest

from oracle import speedup
from oracle import tree as T


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ P1
def test_speedup_formula_matches_printed_output(golden_dir):
    g = _load(golden_dir, "eagle_math_output.json")
    for s in g["setups"]:
        k = speedup.best_k(s["alpha"], s["cost"])
        assert k == s["best_k"]
        assert round(speedup.expected_tokens(s["alpha"], k), 2) == s["tokens_per_step"]
        assert round(speedup.speedup(s["alpha"], k, s["cost"]), 2) == s["speedup"]
    h = g["hand"]
    assert speedup.expected_tokens(h["alpha"], h["k"]) == pytest.approx(sum(h["terms"]))
    assert round(speedup.expected_tokens(h["alpha"], h["k"]), 2) == h["tokens"]
    assert 1 + h["k"] * h["cost"] == pytest.approx(h["step_cost"])
    c = g["costly_draft"]
    assert 1 + c["k"] * c["cost"] == pytest.approx(c["step_cost"])
    assert round(speedup.speedup(c["alpha"], c["k"], c["cost"]), 2) == c["speedup"]


# ------------------------------------------------------------------ helpers
def _const_drafter(tree_obj, confs):
    """Toy drafter: the same confidences at every node, tokens = child ranks."""
    def expand(chosen):
        ids = [list(range(len(confs))) for _ in chosen]
        lps = [[np.float32(np.log(c)) for c in confs] for _ in chosen]
        return ids, lps
    return expand


def _path(nodes, i):
    out = []
    while i >= 0:
        out.append(nodes[i].rank)
        i = nodes[i].parent
    return tuple(out[::-1])


def _toy(confs, depth=3, expand=2, budget=6):
    t = T.Tree()
    root_ids = list(range(len(confs)))
    root_lp = [np.float32(np.log(c)) for c in confs]
    T.grow_dynamic(root_ids, root_lp, _const_drafter(t, confs), expand, len(confs), depth, t)
    kept = T.rerank(t.nodes, budget)
    return t, kept


def _parse_practice(golden_dir):
    out = {}
    cur = None
    with open(os.path.join(golden_dir, "practice_dynamic_tree_output.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            m = re.match(r"(\w+): node depths \[([\d, ]+)\], expected accepted drafts ([\d.]+)", line)
            if m:
                cur = m.group(1)
                out[cur] = dict(depths=[int(x) for x in m.group(2).split(",")],
                                total=float(m.group(3)), paths=[])
                continue
            m = re.match(r"\s+path \(([\d, ]*)\)\s+value ([\d.]+)", line)
            path = tuple(int(x) for x in m.group(1).split(",") if x.strip())
            out[cur]["paths"].append((path, float(m.group(2))))
    return out


# ------------------------------------------------------------------ P3
@pytest.mark.parametrize("name,confs", [("predictable", [0.90, 0.06, 0.02]),
                                        ("uncertain", [0.40, 0.30, 0.20])])
def test_practice_script_output(golden_dir, name, confs):
    want = _parse_practice(golden_dir)[name]
    t, kept = _toy(confs)
    got = [(_path(t.nodes, i), float(np.exp(np.float64(t.nodes[i].logv)))) for i in kept]
    assert [p for p, _ in got] == [p for p, _ in want["paths"]]
    for (_, v), (_, w) in zip(got, want["paths"]):
        assert round(v, 3) == pytest.approx(w, abs=1e-9)
    assert sorted(t.nodes[i].depth for i in kept) == want["depths"]
    assert round(sum(v for _, v in got), 2) == pytest.approx(want["total"])
    assert len(t.nodes) == 3 + 2 * 3 + 2 * 3      # 15 nodes generated


# ------------------------------------------------------------------ P4
def test_practice_variants_by_hand():
    """The page's three suggested changes, worked out by hand from its rules."""
    # budget=3: the predictable tree becomes a chain, the uncertain one three siblings
    t, kept = _toy([0.90, 0.06, 0.02], budget=3)
    assert [_path(t.nodes, i) for i in kept] == [(0,), (0, 0), (0, 0, 0)]
    assert sum(np.exp(np.float64(t.nodes[i].logv)) for i in kept) == pytest.approx(0.9 + 0.81 + 0.729, rel=1e-6)
    t, kept = _toy([0.40, 0.30, 0.20], budget=3)
    assert [_path(t.nodes, i) for i in kept] == [(0,), (1,), (2,)]
    # expand=1: uncertain drops to 1.26 (gains (0,2)=.08), predictable gains (0,0,1)=.0486
    t, kept = _toy([0.90, 0.06, 0.02], expand=1)
    total = sum(np.exp(np.float64(t.nodes[i].logv)) for i in kept)
    assert total == pytest.approx(0.9 + 0.81 + 0.729 + 0.06 + 0.054 + 0.0486, rel=1e-6)
    assert (0, 0, 1) in [_path(t.nodes, i) for i in kept]
    t, kept = _toy([0.40, 0.30, 0.20], expand=1)
    total = sum(np.exp(np.float64(t.nodes[i].logv)) for i in kept)
    assert total == pytest.approx(1.26, rel=1e-6)
    # flat drafter: three siblings then the first-generated grandchildren (tie rule)
    t, kept = _toy([0.25, 0.25, 0.25])
    assert [_path(t.nodes, i) for i in kept] == [(0,), (1,), (2,), (0, 0), (0, 1), (0, 2)]
    assert sum(np.exp(np.float64(t.nodes[i].logv)) for i in kept) == pytest.approx(0.9375, rel=1e-6)


# ------------------------------------------------------------------ P2
def test_worked_example(golden_dir):
    g = _load(golden_dir, "worked_tree.json")
    conf = g["confidences"]
    t = T.Tree()

    def label(i):
        n = t.nodes[i]
        prefix = "" if n.parent < 0 else label(n.parent)
        return prefix + list(conf[prefix])[n.rank]

    def expand(chosen):
        kids = [conf[label(e)] for e in chosen]
        return ([list(range(len(c))) for c in kids],
                [[np.float32(np.log(v)) for v in c.values()] for c in kids])

    root = conf[""]
    T.grow_dynamic(list(range(len(root))), [np.float32(np.log(v)) for v in root.values()],
                   expand, g["expand"], g["branch"], g["depth"], t)
    label = {i: label(i) for i in range(len(t.nodes))}
    values = {label[i]: float(np.exp(np.float64(n.logv))) for i, n in enumerate(t.nodes)}
    assert set(values) == set(g["path_values"])
    for k, v in g["path_values"].items():
        assert values[k] == pytest.approx(v, rel=1e-5)
    assert [label[i] for i in t.expanded[-1]] == g["expanded_at_depth_3"]
    order = T.rerank(t.nodes, len(t.nodes))
    assert [label[i] for i in order[:6]] == g["rerank_order_head"]
    kept = T.rerank(t.nodes, g["budget"])
    assert sorted(label[i] for i in kept) == sorted(g["kept"])
    # the kept set is the best connected 5-subset (brute force over all subsets)
    best = max((s for s in itertools.combinations(range(len(t.nodes)), g["budget"])
                if all(t.nodes[i].parent < 0 or t.nodes[i].parent in s for i in s)),
               key=lambda s: sum(values[label[i]] for i in s))
    assert set(best) == set(kept)


# ------------------------------------------------------------------ P5
def test_path_value_arithmetic():
    # EAGLE-2 page, "Path Value Ranks Prefixes": 0.6*0.7 = 0.42 beats 0.2*0.9 = 0.18
    a = np.float32(np.float32(np.log(0.6)) + np.float32(np.log(0.7)))
    b = np.float32(np.float32(np.log(0.2)) + np.float32(np.log(0.9)))
    assert np.exp(a) == pytest.approx(0.42, rel=1e-6) and np.exp(b) == pytest.approx(0.18, rel=1e-6)
    assert a > b
    # lesson, "Pause and think": B->E = 0.08*0.60 = 0.048 < A->D = 0.90*0.20 = 0.18
    be = np.float32(np.float32(np.log(0.08)) + np.float32(np.log(0.6)))
    ad = np.float32(np.float32(np.log(0.9)) + np.float32(np.log(0.2)))
    assert np.exp(be) == pytest.approx(0.048, rel=1e-6) and be < ad


# ------------------------------------------------------------------ P6
@pytest.mark.parametrize("seed", range(20))
def test_rerank_keeps_a_connected_tree(seed):
    rng = np.random.default_rng(seed)
    k_e, k_b, depth = int(rng.integers(1, 4)), int(rng.integers(1, 5)), int(rng.integers(1, 6))
    t = T.Tree()

    def expand(chosen):
        ids = [list(range(k_b)) for _ in chosen]
        lps = []
        for _ in chosen:
            p = rng.dirichlet(np.ones(k_b + 2) * 0.3)[:k_b]
            if rng.random() < 0.2:
                p[:] = p[0]          # force exact ties
            lps.append([np.float32(np.log(x)) if x > 0 else np.float32(-np.inf) for x in p])
        return ids, lps
    p0 = rng.dirichlet(np.ones(k_b + 2))[:k_b]
    T.grow_dynamic(list(range(k_b)), [np.float32(np.log(x)) for x in p0], expand, k_e, k_b, depth, t)
    for m in range(len(t.nodes) + 1):
        kept = set(T.rerank(t.nodes, m))
        assert all(t.nodes[i].parent < 0 or t.nodes[i].parent in kept for i in kept)
    for n in t.nodes:
        if n.parent >= 0:
            assert n.logv <= t.nodes[n.parent].logv


# ------------------------------------------------------------------ P7
def test_fig7_mask(golden_dir):
    g = _load(golden_dir, "fig7_mask.json")
    words = [g["root"]]
    parent = [-1]
    for br in g["branches"]:
        prev = 0
        for wd in br:
            words.append(wd)
            parent.append(prev)
            prev = len(words) - 1
    m = T.tree_mask(parent)
    r = words.index(g["row"])
    seen = {words[j] for j in range(len(words)) if m[r, j]}
    assert seen == set(g["sees"])
    assert not seen & set(g["does_not_see"])


def test_flatten_orders_rows_breadth_first():
    t, kept = _toy([0.40, 0.30, 0.20])
    rows = T.flatten(t.nodes, kept, root_token=99)
    assert rows["token"][0] == 99 and rows["parent"][0] == -1
    assert rows["depth"] == sorted(rows["depth"])
    for r in range(1, len(rows["token"])):
        p = rows["parent"][r]
        assert 0 <= p < r and rows["depth"][p] == rows["depth"][r] - 1


def test_accept_walk_closed_form():
    """L = the longest root path whose tokens equal the greedy continuation."""
    rng = np.random.default_rng(0)
    for _ in range(200):
        n = int(rng.integers(1, 12))
        parent = [-1] + [int(rng.integers(0, r)) for r in range(1, n)]
        tok = [0] * n
        for r in range(1, n):   # siblings get distinct tokens
            used = {tok[c] for c in range(1, r) if parent[c] == parent[r]}
            tok[r] = int(rng.choice([x for x in range(6) if x not in used]))
        cont = [int(x) for x in rng.integers(0, 6, size=8)]   # greedy continuation
        # g at row r = the continuation token after r's path if the path matches it
        g = []
        for r in range(n):
            path = T.ancestors(parent, r)[1:]
            ok = all(tok[p] == cont[i] for i, p in enumerate(path))
            g.append(cont[len(path)] if ok else int(rng.integers(0, 6)))
        path, bonus = T.accept(tok, parent, g)
        seqs = {tuple(tok[p] for p in T.ancestors(parent, r)[1:]) for r in range(n)}
        L = max(l for l in range(len(cont)) if tuple(cont[:l]) in seqs)
        assert L == len(path)
        assert bonus == cont[len(path)]


# ------------------------------------------------------------------ static tree (reading 15)
def test_grow_static_hand_example():
    """EAGLE-1's fixed tree ([L13] "EAGLE-2 and dynamic draft trees": the
    static shape EAGLE-2 replaces) grown by a toy drafter whose child tokens
    encode the parent's token (child = 10 * parent + rank + 1), with
    confidences that differ per expanded node. Expected nodes, parents and
    path values are worked out by hand below, so a swapped parent, a wrong
    rank index or a mis-ordered expansion fails."""
    paths = [(0,), (1,), (2,), (0, 0), (0, 2), (1, 1), (0, 0, 1)]
    probs = {1: [0.7, 0.2, 0.05, 0.05], 2: [0.4, 0.35, 0.2, 0.05],
             11: [0.9, 0.05, 0.03, 0.02]}
    t = T.Tree()

    def expand(chosen):
        ids, lps = [], []
        for e in chosen:
            tok = t.nodes[e].token
            ids.append([10 * tok + r + 1 for r in range(4)])
            lps.append([np.float32(np.log(p)) for p in probs[tok]])
        return ids, lps

    root_p = [0.5, 0.3, 0.15, 0.05]
    T.grow_static([1, 2, 3, 4], [np.float32(np.log(p)) for p in root_p], expand, paths, t)
    # node order follows the list; parents are node indices
    assert [n.token for n in t.nodes] == [1, 2, 3, 11, 13, 22, 112]
    assert [n.parent for n in t.nodes] == [-1, -1, -1, 0, 0, 1, 3]
    assert [n.depth for n in t.nodes] == [1, 1, 1, 2, 2, 2, 3]
    assert [n.rank for n in t.nodes] == [0, 1, 2, 0, 2, 1, 1]
    # expanded per pass: depth 1 nodes with listed children (in list order), then (0, 0)
    assert t.expanded == [[0, 1], [3]]
    # path values: products of the confidences on the path
    want = [0.5, 0.3, 0.15, 0.5 * 0.7, 0.5 * 0.05, 0.3 * 0.35, 0.5 * 0.7 * 0.05]
    assert np.allclose([np.exp(np.float64(n.logv)) for n in t.nodes], want, rtol=1e-6)
    # every node is kept; verify rows are breadth first in list order
    rows = T.flatten(t.nodes, list(range(len(t.nodes))), 0)
    assert rows["token"] == [0, 1, 2, 3, 11, 13, 22, 112]
    assert rows["parent"] == [-1, 0, 0, 0, 1, 1, 2, 4]


def test_grow_static_c2_under_its_prior():
    """The c2 static list grown by a drafter that always returns the prior
    (0.6, 0.2, 0.1, 0.05) over child ranks: every node's log path value is
    the sum of log q over its rank path, the passes expand 4, 5, 4, 2 rows,
    and every expanded row is the parent of at least one listed node."""
    import synth
    q = [0.6, 0.2, 0.1, 0.05]
    lq = [np.float32(np.log(p)) for p in q]
    t = T.Tree()

    def expand(chosen):
        return [[10 * (e + 1) + r for r in range(4)] for e in chosen], [lq] * len(chosen)

    paths = [tuple(p) for p in synth.STATIC_TREE_C2]
    T.grow_static(list(range(4)), lq, expand, paths, t)
    assert len(t.nodes) == 26
    assert [len(x) for x in t.expanded] == [4, 5, 4, 2]
    for i, p in enumerate(paths):
        n = t.nodes[i]
        assert _path(t.nodes, i) == p
        assert n.depth == len(p)
        assert float(n.logv) == pytest.approx(float(np.sum(np.log(np.array(q)[list(p)]))), abs=1e-5)
        if n.parent >= 0:   # child token names its parent node and rank
            assert n.token == 10 * (n.parent + 1) + p[-1]
    for d, exp in enumerate(t.expanded, start=2):
        assert all(t.nodes[e].depth == d - 1 for e in exp)
        assert all(any(n.parent == e for n in t.nodes) for e in exp)


# ------------------------------------------------------------------ P1 (distribution form)
@pytest.mark.parametrize("alpha", [0.0, 0.25, 0.6, 0.8, 1.0])
@pytest.mark.parametrize("k", [0, 1, 3, 5])
def test_accepted_length_distribution_by_enumeration(alpha, k):
    """The speedup oracle's distribution of accepted lengths against an
    enumeration of every accept/reject outcome of k independent drafts (the
    step stops at the first rejection)."""
    pmf = speedup.accepted_length_pmf(alpha, k)
    assert sum(pmf) == pytest.approx(1.0)
    want = [0.0] * (k + 1)
    for outcome in itertools.product([True, False], repeat=k):
        p = 1.0
        for ok in outcome:
            p *= alpha if ok else 1.0 - alpha
        L = next((i for i, ok in enumerate(outcome) if not ok), k)
        want[L] += p
    assert pmf == pytest.approx(want)
