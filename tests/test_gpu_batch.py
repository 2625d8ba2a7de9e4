"""Several sequences served by one context (eagle_config.batch > 1). Each
lane must compute what a batch-1 context computes for its own sequence: the
method is defined per sequence ([L13] "Speculative decoding in four moves",
[E2] "Putting It Together"), and a batch only runs the lanes' rows through
one pass over the weights.

* c1 (fp32), batch 3, prompts of different lengths: every lane's drafted
  tree and committed tokens equal the oracle session's for its prompt, cycle
  by cycle; a lane prefilled again between cycles starts its new sequence
  while the other lanes carry on; batch-1 calls are refused.
* c1 greedy streams over a whole generation (batch 4) and plain decoding
  (budget 0, batch 2) equal the oracle's greedy decode of each prompt.
* c1 sampling (T = 0.8, batch 2): lane b's stream equals the oracle session
  that draws from stream `lane = b`.
* reduced c2 (bf16, static tree, EAGLE-1) and reduced c4 (bf16, GQA, dynamic
  tree, EAGLE-3), batch 3 with ragged prompts: verify logits and features of
  every lane match the oracle within the bf16 tolerance, the tree policy is
  bit-exact on the GPU's own log-probabilities, and each lane's stream passes
  the teacher-forced check.
* full-size c2 at batch 4 and 6 (launched as the benchmark runs it): tree policy
  and acceptance bit-exact per lane, and each lane's stream equals a batch-1
  engine's stream on the same prompt up to a near-tie.
* sampling in a batch on reduced c2 (EAGLE-1) and c4 (EAGLE-3): each lane's
  tokens equal the oracle's rejection-sampling walk on that lane's GPU
  logits with the lane's own draw stream.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _max_ctx(w, B):
    # lanes cycle together until the slowest has `gen` tokens: a fast lane
    # can commit depth + 1 tokens in each of those cycles
    return w["prompt_len"] + (w["depth"] + 1) * w["gen"] + w["depth"] + 2


def run_lanes(eng, prompts, gen):
    """Prefill every lane, then cycle all lanes until each holds >= gen tokens."""
    for b, p in enumerate(prompts):
        eng.prefill(p, lane=b)
    while min(len(eng.committed(b)) for b in range(len(prompts))) < gen:
        eng.draft_tree(want=False)
        eng.verify_batch()
    return [eng.committed(b) for b in range(len(prompts))]


def _ragged_prompts(w, B, seed0=1):
    n = w["prompt_len"]
    lens = [n, max(4, n - 13), max(4, n // 2 + 3), max(4, n - 5)][:B]
    return [synth.prompt(seed0 + b, lens[b], w["vocab"]) for b in range(B)]


def test_c1_lanes_equal_oracle_sessions_cycle_by_cycle():
    import speculative_decoding_draft_amd as E
    from gpu_helpers import engine, gpu_tree_check
    from oracle.loop import Session
    w = dict(synth.workloads.get("c1"), batch=3)
    eng = engine(w, max_ctx=_max_ctx(w, 3))
    prompts = _ragged_prompts(w, 3)
    refs = [Session(w) for _ in prompts]
    print("c1 batch 3 prefill", flush=True)
    for b, p in enumerate(prompts):
        assert eng.prefill(p, lane=b) == refs[b].prefill(p), b

    def cycle(tag):
        eng.draft_tree(want=False)
        rows = []
        for b, ref in enumerate(refs):
            tree = eng.read_tree(b)
            gpu_tree_check(tree, w["topk"], w["depth"], w["budget"])
            t, r = ref.draft_tree()
            assert tree["node_token"] == [n.token for n in t.nodes], (tag, b)
            ref_lp = np.array([n.logp for n in t.nodes], dtype=np.float64)
            assert np.abs(tree["node_logp"] - ref_lp).max() < 1e-3, (tag, b)
            assert tree["token"] == r["token"] and tree["parent"] == r["parent"], (tag, b)
            rows.append(r)
        news = eng.verify_batch()
        for b, ref in enumerate(refs):
            path, bonus, _, _ = ref.verify()
            assert news[b] == [rows[b]["token"][r] for r in path] + [bonus], (tag, b)
            assert eng.committed(b) == ref.committed, (tag, b)

    for cyc in range(4):
        print(f"c1 batch 3 cycle {cyc}", flush=True)
        cycle(cyc)
    # lane 1 starts a new sequence; lanes 0 and 2 carry on
    p_new = synth.prompt(9, 17, w["vocab"])
    refs[1] = Session(w)
    assert eng.prefill(p_new, lane=1) == refs[1].prefill(p_new)
    for cyc in range(4, 7):
        print(f"c1 batch 3 cycle {cyc} (lane 1 restarted)", flush=True)
        cycle(cyc)
    # batch-1 calls are refused at batch 3
    with pytest.raises(E.EagleError) as ei:
        eng.verify()
    assert ei.value.status == E.E_STATE
    with pytest.raises(E.EagleError) as ei:
        eng.generate(prompts[0], 4)
    assert ei.value.status == E.E_STATE
    with pytest.raises(E.EagleError) as ei:
        eng.prefill(prompts[0], lane=3)
    assert ei.value.status == E.E_INVALID
    eng.close()


@pytest.mark.parametrize("budget", [16, 0])
def test_c1_batch_streams_equal_greedy_decode(budget):
    from gpu_helpers import engine
    from oracle.loop import greedy_decode
    B = 4 if budget else 2
    w = dict(synth.workloads.get("c1"), batch=B, budget=budget)
    eng = engine(w, max_ctx=_max_ctx(w, B))
    prompts = _ragged_prompts(w, B, seed0=11)
    print(f"c1 batch {B} budget {budget} streams", flush=True)
    got = run_lanes(eng, prompts, w["gen"])
    eng.close()
    for b, p in enumerate(prompts):
        want, margins, _ = greedy_decode(w, p, w["gen"])
        mism = [i for i in range(len(want)) if got[b][i] != want[i]]
        if mism:   # only at a near-tie, after which the streams part ways
            assert margins[mism[0]] < 1e-3, (b, mism[0], margins[mism[0]])


def test_c1_batch_sampling_streams_equal_oracle_sessions():
    from gpu_helpers import engine
    from oracle.loop import Session
    B = 2
    w = dict(synth.workloads.get("c1"), batch=B, temperature=0.8, seed=5)
    eng = engine(w, max_ctx=_max_ctx(w, B))
    prompts = _ragged_prompts(w, B, seed0=21)
    print("c1 batch 2 sampling", flush=True)
    got = run_lanes(eng, prompts, w["gen"])
    eng.close()
    for b, p in enumerate(prompts):
        # near-ties of the sampling decisions resolved as the GPU resolved them
        want = Session(w, lane=b, follow=got[b]).generate(p)
        n = min(len(want), len(got[b]))
        assert n >= w["gen"]
        assert got[b][:n] == want[:n], b
    # the two lanes draw from different streams: the same prompt in both
    # lanes gives two different sampled streams (with overwhelming odds)
    eng = engine(w, max_ctx=_max_ctx(w, B))
    same = run_lanes(eng, [prompts[0], prompts[0]], w["gen"])
    eng.close()
    assert same[0][:w["gen"]] == got[0][:w["gen"]]
    assert same[1][:w["gen"]] != same[0][:w["gen"]]


def _rel_rows(got, ref):
    return float((np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)).max())


@pytest.mark.parametrize("name", ["c2", "c4"])
def test_bf16_batch_lanes_match_oracle(name):
    from gpu_helpers import engine, gpu_tree_check, stream_check
    from oracle.loop import Session
    from oracle.model import Config, Weights
    B = 3
    w = dict(synth.workloads.reduced(name, prompt_len=80, gen=24), batch=B)
    static = w["static"] if w["tree"] == "static" else None
    eng = engine(w, max_ctx=_max_ctx(w, B), prefill_chunk=32)
    W = Weights(Config(w))
    prompts = _ragged_prompts(w, B, seed0=31)
    print(f"{w['name']} batch {B} cycle", flush=True)
    refs = [Session(w, W) for _ in prompts]
    for b, p in enumerate(prompts):
        gb = eng.prefill(p, lane=b)
        assert gb == refs[b].prefill(p) or refs[b].prefill_margin < 1e-3, b
    eng.set_debug(True)
    eng.draft_tree(want=False)
    trees = [eng.read_tree(b) for b in range(B)]
    for tree in trees:
        gpu_tree_check(tree, w["topk"], w["depth"], w["budget"], static)
    eng.verify_batch()
    gl, gf = eng.debug_read("logits"), eng.debug_read("features")
    mv = len(trees[0]["token"])
    assert gl.shape[0] == B * mv and gf.shape[0] == B * mv
    for b, ref in enumerate(refs):
        ref.draft_tree()
        tree = trees[b]
        ref.verify(dict(token=tree["token"], parent=tree["parent"], depth=tree["depth"],
                        node=tree["node"]))
        rel = _rel_rows(gl[b * mv:(b + 1) * mv], ref.last_logits)
        f_rel = _rel_rows(gf[b * mv:(b + 1) * mv], ref.last_features)
        print(f"{w['name']} lane {b}: verify logits rel err {rel:.2e}, features {f_rel:.2e}",
              flush=True)
        assert rel < 1e-3 and f_rel < 1e-3, b
    eng.set_debug(False)
    print(f"{w['name']} batch {B} streams", flush=True)
    got = run_lanes(eng, prompts, w["gen"])
    eng.close()
    for b, p in enumerate(prompts):
        near = stream_check(w, p, got[b][:w["gen"]], W)
        print(f"{w['name']} lane {b}: {w['gen']} tokens, near-ties {near}", flush=True)
        assert near <= 2, b


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B", [4, 6])
def test_full_c2_batch_lanes_equal_batch1(B):
    # B = 4: 108 verify rows (one 128-row pass of q|k|v); B = 6: 162 rows
    # (the 256-row weight tiles with activations copied into LDS)
    import torch
    from gpu_helpers import engine, gpu_tree_check
    from oracle.tree import accept
    w = synth.workloads.get("c2")
    cycles = 3
    max_ctx = w["prompt_len"] + 32 * (w["depth"] + 1) + w["depth"] + 2
    lens = [w["prompt_len"], 400, 256, 511, 300, 450][:B]
    prompts = [synth.prompt(41 + b, lens[b], w["vocab"]) for b in range(B)]
    print(f"c2 full size, batch {B}", flush=True)
    eng = engine(dict(w, batch=B), max_ctx=max_ctx)
    for b, p in enumerate(prompts):
        eng.prefill(p, lane=b)
    eng.set_debug(True)
    mv = 1 + len(w["static"])
    spec = [[eng.committed(b)[0]] for b in range(B)]
    margins = [[] for _ in range(B)]
    for cyc in range(cycles):
        eng.draft_tree(want=False)
        trees = [eng.read_tree(b) for b in range(B)]
        news = eng.verify_batch()
        g, mg = eng.debug_read("argmax"), eng.debug_read("margin")
        for b in range(B):
            gpu_tree_check(trees[b], w["topk"], w["depth"], w["budget"], w["static"])
            gb = g[b * mv:(b + 1) * mv]
            path, bonus = accept(trees[b]["token"], trees[b]["parent"], gb)
            assert news[b] == [trees[b]["token"][r] for r in path] + [bonus], (cyc, b)
            spec[b] += news[b]
            margins[b] += [float(mg[b * mv + r]) for r in [0] + path]
        print(f"c2 batch {B} cycle {cyc}: accepted {[len(n) - 1 for n in news]}", flush=True)
    eng.close()
    del eng
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    # the same prompts one at a time on a batch-1 engine
    one = engine(w, max_ctx=max_ctx)
    one.set_debug(True)
    for b, p in enumerate(prompts):
        ref = [one.prefill(p)]
        ref_margin = []
        while len(ref) < len(spec[b]):
            tree = one.draft_tree()
            new = one.verify()
            mg = one.debug_read("margin")
            path, _ = accept(tree["token"], tree["parent"], one.debug_read("argmax"))
            ref += new
            ref_margin += [float(mg[r]) for r in [0] + path]
        n = min(len(ref), len(spec[b]))
        same = 0
        for i in range(1, n):
            if spec[b][i] != ref[i]:
                assert min(margins[b][i - 1], ref_margin[i - 1]) < 1e-3, (b, i)
                break
            same += 1
        print(f"c2 lane {b} (prompt {lens[b]}): batch {B} == batch 1 on {same}/{n - 1} tokens",
              flush=True)
    one.close()


@pytest.mark.parametrize("name", ["c2", "c4"])
def test_bf16_batch_sampling_decisions_match_oracle(name):
    """Sampling in a batch (reduced c2: static tree, EAGLE-1; reduced c4:
    dynamic tree, EAGLE-3): every lane's committed tokens equal the oracle's
    rejection-sampling walk over that lane's tree, on the GPU's own verify
    logits of that lane, with the lane's own draw stream (counter word 3 =
    lane)."""
    from gpu_helpers import engine
    from oracle import sampling as S
    B = 3 if name == "c2" else 2
    w = dict(synth.workloads.reduced(name, prompt_len=60, gen=16), batch=B, temperature=0.7,
             seed=77)
    eng = engine(w, max_ctx=_max_ctx(w, B), prefill_chunk=32)
    prompts = _ragged_prompts(w, B, seed0=51)
    print(f"{w['name']} batch {B} sampling", flush=True)
    for b, p in enumerate(prompts):
        eng.prefill(p, lane=b)
    for step in range(1, 5):
        eng.draft_tree(want=False)
        trees = [eng.read_tree(b) for b in range(B)]
        news = eng.verify_batch()
        lg = eng.debug_read("logits")
        mv = len(trees[0]["token"])
        assert lg.shape == (B * mv, w["vocab"])
        for b, tree in enumerate(trees):
            ok, want, margin = S.check_walk(news[b], tree["token"], tree["parent"],
                                            lg[b * mv:(b + 1) * mv], w["temperature"], w["seed"],
                                            step, w["depth"], lane=b)
            assert ok, (step, b, news[b], want, margin)
        print(f"{w['name']} sampled cycle {step}: accepted {[len(n) - 1 for n in news]}", flush=True)
    eng.close()
