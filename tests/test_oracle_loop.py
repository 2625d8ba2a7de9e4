"""Pins of the oracle's speculative loop to what the pages fix.

* Lossless ([L13] "Speculative decoding in four moves"; [E2] "The Mask
  Preserves Tree Semantics"): the committed stream equals plain greedy decode.
* Tree attention ([E2] Figure 7): every flattened row computes what the same
  path computes as a plain causal chain (target verify and draft rows).
* Acceptance: longest root path matching the greedy continuation, then the
  target's own token.
* Commit: after compaction the KV cache equals the one plain decode builds.
* Brute force on a tiny vocabulary: expansion and rerank equal an exhaustive
  enumeration of draft paths and connected subsets.
"""
import itertools

import numpy as np
import pytest

import synth
from oracle import tree as T
from oracle.loop import Session, greedy_decode
from oracle.model import Config, Draft, Target, Weights, causal_vis


def _prompt(w, seed=1, n=None):
    return synth.prompt(seed, n or w["prompt_len"], w["vocab"])


@pytest.mark.parametrize("name", ["c1", "c2m", "c3m", "c4m", "c5m"])
def test_lossless_stream_equals_greedy(name):
    w = synth.workloads.get(name) if name == "c1" else synth.workloads.mini(name[:2])
    W = Weights(Config(w))
    p = _prompt(w)
    want, _, _ = greedy_decode(w, p, w["gen"], W)
    s = Session(w, W)
    assert s.generate(p) == want


def _rows_from_paths(root, paths):
    """Planted verify rows from token paths (each path's prefixes must be listed first)."""
    index = {(): 0}
    rows = dict(token=[root], parent=[-1], depth=[0], node=[-1])
    for p in paths:
        p = tuple(p)
        index[p] = len(rows["token"])
        rows["token"].append(p[-1])
        rows["parent"].append(index[p[:-1]])
        rows["depth"].append(len(p))
        rows["node"].append(-1)
    return rows


@pytest.mark.parametrize("name", ["c1", "c5m", "c4m"])
def test_planted_tree_accepts_greedy_path_and_compacts_kv(name):
    w = synth.workloads.get(name) if name == "c1" else synth.workloads.mini(name[:2])
    W = Weights(Config(w))
    p = _prompt(w, seed=2)
    D = 4
    want, _, gkv = greedy_decode(w, p, 2 + D + 3, W)
    s = Session(w, W)
    b = s.prefill(p)
    assert b == want[0]
    cont = want[1:]
    V = w["vocab"]
    # greedy path plus decoys: siblings at every depth and a wrong branch
    paths = []
    for d in range(1, D + 1):
        paths.append(tuple(cont[:d]))
        paths.append(tuple(cont[:d - 1]) + ((cont[d - 1] + 1) % V,))
    paths.append(((cont[0] + 2) % V,))
    paths.append(((cont[0] + 2) % V, cont[1]))
    paths.sort(key=len)
    path, bonus, g, _ = s.verify(_rows_from_paths(b, paths))
    assert len(path) == D
    assert bonus == cont[D]
    assert s.committed == want[:D + 2]
    # KV of positions 0..ctx-1 equals plain decode's (bit for bit)
    n = len(p) + D + 1
    for mine, ref in zip(s.kv, gkv):
        assert np.array_equal(mine[:, :n], ref[:, :n])
    # a tree with no matching first token accepts nothing and commits g[root]
    b2 = s.committed[-1]
    path, bonus, g, _ = s.verify(_rows_from_paths(b2, [((want[D + 2] + 1) % V,)]))
    assert path == [] and bonus == want[D + 2]
    # the loop continues correctly from there
    while len(s.committed) < len(want):
        s.draft_tree()
        s.verify()
    assert s.committed[:len(want)] == want


@pytest.mark.parametrize("name", ["c1", "c5m"])
def test_tree_verify_rows_equal_chain_forward(name):
    w = synth.workloads.get(name) if name == "c1" else synth.workloads.mini(name[:2])
    W = Weights(Config(w))
    p = _prompt(w, seed=3)
    s = Session(w, W)
    s.prefill(p)
    t, rows = s.draft_tree()
    ctx = s.ctx
    kv_before = [c.copy() for c in s.kv]
    tgt = Target(Config(w), W)
    M = len(rows["token"])
    slots = ctx + np.arange(M)
    vis = np.zeros((M, kv_before[0].shape[1]), dtype=bool)
    vis[:, :ctx] = True
    for r in range(M):
        vis[r, ctx + np.array(T.ancestors(rows["parent"], r))] = True
    f_tree, _ = tgt.forward(rows["token"], ctx + np.array(rows["depth"]), slots, vis,
                            [c.copy() for c in kv_before])
    lg_tree = tgt.logits(f_tree)
    for r in range(M):
        chain = list(p) + [rows["token"][a] for a in T.ancestors(rows["parent"], r)]
        n = len(chain)
        kv = tgt.new_kv(n)
        f, _ = tgt.forward(chain, np.arange(n), np.arange(n), causal_vis(n, 0, n), kv)
        assert np.array_equal(tgt.logits(f[-1:])[0], lg_tree[r])


def test_draft_tree_rows_equal_chain_drafting():
    """Each tree row's draft distribution equals drafting its path as a chain."""
    w = synth.workloads.get("c1")
    W = Weights(Config(w))
    p = _prompt(w, seed=4)
    s = Session(w, W)
    s.prefill(p)
    t, _ = s.draft_tree()
    cfg = Config(w)
    tgt, dr = Target(cfg, W), Draft(cfg, W)
    n = len(p)
    kv = tgt.new_kv(n)
    f, _ = tgt.forward(p, np.arange(n), np.arange(n), causal_vis(n, 0, n), kv)
    seq = list(p) + [s.committed[0]]
    for e in range(len(t.nodes)):
        path = [e]
        while t.nodes[path[-1]].parent >= 0:
            path.append(t.nodes[path[-1]].parent)
        path = path[::-1]
        # chain: committed rows (f_j, t_{j+1}) then (own output, node token) per step
        S = n + len(path) + 2
        dkv = dr.new_kv(S)
        out = dr.rows(f, seq[1:], np.arange(1, n + 1), np.arange(1, n + 1),
                      causal_vis(n, 1, S, 1), dkv)
        last = out[-1]
        for i, node in enumerate(path):
            pos = n + 1 + i
            vis = np.zeros((1, S), dtype=bool)
            vis[0, 1:pos + 1] = True
            last = dr.rows(last[None], [t.nodes[node].token], np.array([pos]), np.array([pos]),
                           vis, dkv)[0]
        ids, lp, _ = dr.topk(last[None], s.k)
        # the chain's distribution after `path` must give e's children (if e was expanded)
        kids = [c for c in t.nodes if c.parent == e]
        if kids:
            assert [c.token for c in kids] == list(ids[0])
            assert [c.logp for c in kids] == list(lp[0])


def test_budget_zero_is_plain_greedy_and_chain_tree_is_chain_decoding():
    w = synth.workloads.get("c1")
    W = Weights(Config(w))
    p = _prompt(w, seed=6)
    want, _, _ = greedy_decode(w, p, 20, W)
    w0 = dict(w, budget=0)
    s = Session(w0, W)
    assert s.generate(p, 20) == want
    assert all(h["L"] == 0 and len(h["rows"]["token"]) == 1 for h in s.history)
    wc = dict(w, topk=1, budget=w["depth"])
    s = Session(wc, W)
    assert s.generate(p, 20) == want
    for h in s.history:
        assert h["rows"]["parent"] == list(range(-1, w["depth"]))


def _tiny(vocab=8):
    w = synth.workloads.get("c1")
    w.update(name="tiny", hidden=64, n_heads=2, n_kv_heads=2, ffn=96, vocab=vocab,
             n_layers=1, prompt_len=6, gen=4)
    return w


@pytest.mark.parametrize("k", [2, 3])
def test_bruteforce_tiny_vocab(k):
    """Expansion and rerank equal an exhaustive enumeration over all draft paths."""
    w = dict(_tiny(), topk=k, depth=3, budget=5)
    cfg = Config(w)
    W = Weights(cfg)
    # sharpen the draft distribution so paths differ clearly
    s = Session(w, W)
    p = _prompt(w, seed=7)
    s.prefill(p)
    t, rows = s.draft_tree()
    # exhaustive chain drafting of every token path of depth <= 3
    tgt, dr = Target(cfg, W), Draft(cfg, W)
    n = len(p)
    kv = tgt.new_kv(n)
    f, _ = tgt.forward(p, np.arange(n), np.arange(n), causal_vis(n, 0, n), kv)
    seq = list(p) + [s.committed[0]]
    V = w["vocab"]
    logp = {}   # path -> log-prob of its last token given the prefix (chain drafting)
    S = n + 6
    dkv = dr.new_kv(S)
    out = dr.rows(f, seq[1:], np.arange(1, n + 1), np.arange(1, n + 1), causal_vis(n, 1, S, 1), dkv)
    base_k = [c.copy() for c in dkv]

    def dist(prev_out):
        lg = dr.logits(prev_out[None])
        from oracle.numerics import log_softmax, to_f32
        return to_f32(log_softmax(lg))[0], lg[0]
    frontier = {(): out[-1]}
    for d in range(1, 4):
        nxt = {}
        for path, o in frontier.items():
            lp, lg = dist(o)
            for v in range(V):
                logp[path + (v,)] = (np.float32(lp[v]), lg[v])
                if d < 3:
                    ck = [c.copy() for c in base_k]
                    last = out[-1]
                    for i, tok in enumerate(path + (v,)):
                        pos = n + 1 + i
                        vis = np.zeros((1, S), dtype=bool)
                        vis[0, 1:pos + 1] = True
                        last = dr.rows(last[None], [tok], np.array([pos]), np.array([pos]), vis, ck)[0]
                    nxt[path + (v,)] = last
        frontier = nxt
    # top-k children of a path: by (logit desc, id asc)
    def kids(path):
        cand = [(path + (v,)) for v in range(V)]
        return sorted(cand, key=lambda q: (-logp[q][1], q[-1]))[:k]

    def lv(path):
        acc = np.float32(0)
        for i in range(1, len(path) + 1):
            acc = logp[path[:i]][0] if i == 1 else np.float32(acc + logp[path[:i]][0])
        return acc
    gen = list(kids(()))
    frontier = list(gen)
    for d in range(2, 4):
        chosen = sorted(frontier, key=lambda q: (-float(lv(q)), gen.index(q)))[:k]
        frontier = [c for e in chosen for c in kids(e)]
        gen += frontier
    # the oracle's tree generated exactly these paths, with these values
    def tpath(i):
        out_ = []
        while i >= 0:
            out_.append(t.nodes[i].token)
            i = t.nodes[i].parent
        return tuple(out_[::-1])
    assert [tpath(i) for i in range(len(t.nodes))] == gen
    assert [t.nodes[i].logv for i in range(len(t.nodes))] == [lv(q) for q in gen]
    # rerank = the best connected subset of size m by sum of path values
    m = w["budget"]
    vals = [float(np.exp(np.float64(lv(q)))) for q in gen]
    best = max((c for c in itertools.combinations(range(len(gen)), m)
                if all(len(gen[i]) == 1 or gen.index(gen[i][:-1]) in c for i in c)),
               key=lambda c: sum(vals[i] for i in c))
    kept = T.rerank(t.nodes, m)
    assert sum(vals[i] for i in kept) == pytest.approx(sum(vals[i] for i in best), rel=1e-12)
