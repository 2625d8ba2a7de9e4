"""Sampling-mode (temperature > 0) verification on the GPU against the oracle
(oracle/sampling.py, float64 definitions):
* the acceptance walk and the drawn token, taken from the GPU's own verify
  logits, equal the oracle's decisions on the same logits, a decision whose
  two compared quantities lie within the oracle's near-tie allowance (1e-5
  in probability; the GPU decides in float32) counting as correct either
  way (drafted trees,
  and planted trees built from the target's top tokens so that several
  depths are accepted), at c1 (fp32, V=1024) and the reduced c2 (bf16,
  V=32000);
* the c1 stream equals the oracle session's stream with the same seed
  (near-ties again resolved as the GPU resolved them);
* losslessness on the device: over many seeds the prefill's token and the
  first committed token of a verify follow softmax(logits / T) (chi-square).
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _check_walk(got, tree, lg, w, step):
    """The oracle's walk on the GPU's logits, near-ties resolved as `got`
    resolves them; returns the accepted depth."""
    from oracle import sampling as S
    ok, want, margin = S.check_walk(got, tree["token"], tree["parent"], lg, w["temperature"],
                                    w["seed"], step, w["depth"])
    assert ok, (step, got, want, margin)
    return len(want) - 1


def _top_tree(eng, w, p, width, levels):
    """Planted tree whose rows are the target's `width` most likely tokens at
    each row, `levels` deep (built by verifying growing trees from a fresh
    prefill each time; every verify is discarded by the next prefill)."""
    tokens, parent = [0], [-1]
    frontier = [0]
    gap = np.inf
    for _ in range(levels):
        eng.prefill(p)                     # greedy prefill: a fixed root token
        eng.verify({"token": tokens, "parent": parent})
        lg = eng.debug_read("logits")
        nxt = []
        for r in frontier:
            order = np.argsort(-lg[r], kind="stable")
            gap = min(gap, float(lg[r][order[0]] - lg[r][order[1]]))
            for x in order[:width]:
                tokens.append(int(x))
                parent.append(r)
                nxt.append(len(tokens) - 1)
        frontier = nxt
    # smallest top-1 minus top-2 logit gap over the rows that have children
    return {"token": tokens, "parent": parent}, gap


@pytest.fixture(scope="module", params=["c1", "c2r"])
def sampler(request):
    from gpu_helpers import engine
    if request.param == "c1":
        w = dict(synth.workloads.get("c1"), temperature=0.7, seed=1234)
        eng = engine(w)
    else:
        w = dict(synth.workloads.reduced("c2", prompt_len=80, gen=24), temperature=0.6, seed=99)
        eng = engine(w, prefill_chunk=32)
    print(f"sampling setup {w['name']}", flush=True)
    yield w, eng
    eng.close()


def test_drafted_trees_match_oracle_decisions(sampler):
    w, eng = sampler
    p = synth.prompt(2, w["prompt_len"], w["vocab"])
    eng.prefill(p)
    for step in range(1, 7):
        print(f"{w['name']} drafted cycle {step}", flush=True)
        tree = eng.draft_tree()
        new = eng.verify()
        lg = eng.debug_read("logits")
        assert lg.shape == (len(tree["token"]), w["vocab"])
        _check_walk(new, tree, lg, w, step)


def test_planted_top_trees_accept_deep_and_match_oracle(sampler):
    w, eng = sampler
    p = synth.prompt(3, w["prompt_len"], w["vocab"])
    levels = min(3, w["depth"])
    eng.set_sampling(0.0, 0)
    eng.set_debug(True)
    tree, gap = _top_tree(eng, w, p, 2, levels)
    # cold enough that every row's top token outweighs the runner-up ~e^4
    # times, so the first child is accepted at nearly every depth
    cold = max(gap / 4.0, 1e-4)
    eng.set_sampling(cold, w["seed"])
    wc = dict(w, temperature=cold)
    depths = []
    for trial in range(6):
        eng.set_sampling(0.0, 0)
        eng.prefill(p)                     # the same greedy root as the tree's
        eng.set_sampling(cold, w["seed"] + trial)
        print(f"{w['name']} planted trial {trial}", flush=True)
        new = eng.verify(tree)
        lg = eng.debug_read("logits")
        depths.append(_check_walk(new, tree, lg, dict(wc, seed=w["seed"] + trial), 1))
    eng.set_sampling(w["temperature"], w["seed"])
    eng.set_debug(False)
    assert max(depths) >= 2, depths     # the accepting branch is exercised


def test_c1_stream_equals_oracle_session():
    from gpu_helpers import engine
    from oracle.loop import Session
    for seed in (5, 6):
        w = dict(synth.workloads.get("c1"), temperature=0.8, seed=seed)
        eng = engine(w)
        p = synth.prompt(seed, w["prompt_len"], w["vocab"])
        print(f"c1 sampled stream seed {seed}", flush=True)
        got, _ = eng.generate(p, w["gen"])
        eng.close()
        ref = Session(w, follow=got)
        assert ref.generate(p) == got
        print(f"smallest sampling margin {min(ref.sample_margins):.2e}", flush=True)


def _chi2_ok(counts, probs, n):
    exp = probs * n
    keep = exp >= 5
    other = float(counts[~keep].sum())
    other_exp = float(exp[~keep].sum())
    chi2 = float((((counts[keep] - exp[keep]) ** 2) / exp[keep]).sum())
    dof = int(keep.sum()) - 1
    if other_exp >= 5:
        chi2 += (other - other_exp) ** 2 / other_exp
        dof += 1
    return chi2 < dof + 5 * np.sqrt(2 * max(dof, 1)) + 10, chi2, dof


def test_first_tokens_follow_target_softmax():
    from gpu_helpers import engine
    from oracle import sampling as S
    from oracle.model import Config, Target, Weights, causal_vis
    T = 1.0
    w = dict(synth.workloads.get("c1"), temperature=T, seed=0)
    eng = engine(w)
    p = synth.prompt(7, w["prompt_len"], w["vocab"])
    # the prefill's token: the last prompt row's softmax (c1 is fp32; the
    # oracle's logits agree with the GPU's to ~1e-6)
    cfg = Config(w)
    tgt = Target(cfg, Weights(cfg))
    n = len(p)
    f, _ = tgt.forward(p, np.arange(n), np.arange(n), causal_vis(n, 0, n), tgt.new_kv(n))
    p_pre = S.probs(tgt.logits(f[-1:])[0], T)
    # the first verified token: the root row after a greedy prefill, whose
    # distribution comes from the GPU's own logits
    eng.set_sampling(0.0, 0)
    eng.set_debug(True)
    eng.prefill(p)
    eng.verify({"token": [0], "parent": [-1]})
    p_root = S.probs(eng.debug_read("logits")[0], T)
    top = [int(x) for x in np.argsort(-p_root, kind="stable")[:3]]
    planted = {"token": [0] + top, "parent": [-1, 0, 0, 0]}
    N = 1500
    pre_counts = np.zeros(w["vocab"])
    ver_counts = np.zeros(w["vocab"])
    print("c1 chi-square sampling", flush=True)
    for s in range(N):
        eng.set_sampling(T, 1000 + s)
        eng.prefill(p)
        pre_counts[eng.committed()[0]] += 1
        eng.set_sampling(0.0, 0)
        eng.prefill(p)                      # greedy root
        eng.set_sampling(T, 50000 + s)
        ver_counts[eng.verify(planted)[0]] += 1
    eng.close()
    ok, chi2, dof = _chi2_ok(pre_counts, p_pre, N)
    assert ok, ("prefill", chi2, dof)
    ok, chi2, dof = _chi2_ok(ver_counts, p_root, N)
    assert ok, ("verify", chi2, dof)
