"""Parity at the full sizes of the 7B / 8B / 70B workloads (all layers, the
full prompt lengths), with the engine sized and launched as the benchmark
runs it (default prefill chunking).

The oracle cannot follow a 32- to 80-layer model over thousands of positions
in seconds, so at the full prompt lengths the checks are exact properties
and oracle recomputations of sampled outputs:
* tree policy, bit-exact: the oracle's expansion / rerank / flattening,
  rerun on the GPU's own draft log-probabilities, gives the GPU's nodes,
  path values and verify rows ([E2] "Putting It Together");
* acceptance, bit-exact: the oracle's walk over the GPU's tree and target
  argmax gives exactly the tokens the GPU committed ([L13] "Speculative
  decoding in four moves");
* lossless on the GPU itself: the speculative stream equals plain greedy
  decode (root-only planted trees) on the same engine, up to the first
  position where either side's top-1/top-2 margin is below 1e-3;
* tree attention: a kept row's logits equal those of the same path verified
  as a chain ([E2] "The Mask Preserves Tree Semantics in One Target Pass");
* LM head: the oracle's logits from the GPU's own final features on
  sampled rows (the full vocabulary, 128256 rows at the 8B shape);
and the oracle's teacher-forced greedy choices over the GPU's stream: at the
configs' own prompt and generation lengths (512 + 256, 1536 + 512 and
3584 + 512 tokens for c2, c3, c4; the 70B shape's 1024 + 256, about eight
minutes of CPU work, when EAGLE_ORACLE_LONG=c5 is set), and for the 70B shape
by default with every layer but a short prompt.
"""
import os

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

CONFIGS = ["c2", "c3", "c4", "c5"]
# configs whose full-length oracle pass fits the default test run
FULL_LENGTH_DEFAULT = ("c2", "c3", "c4")
CYCLES = 3
TOL = 1e-3


@pytest.fixture(scope="module", params=CONFIGS)
def setup(request):
    import torch
    from gpu_helpers import engine
    name = request.param
    w = synth.workloads.get(name)
    # sized like the benchmark: room for many cycles of depth + 1 tokens
    max_new = max(w["gen"], 32 * (w["depth"] + 1))
    max_ctx = w["prompt_len"] + max_new + w["depth"] + 2
    print(f"setup {name}: full size, max_ctx {max_ctx}", flush=True)
    eng = engine(w, max_ctx=max_ctx)
    yield w, eng
    eng.close()
    del eng
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _static(w):
    return w["static"] if w.get("tree") == "static" else None


def test_full_tree_acceptance_and_lossless(setup):
    from gpu_helpers import gpu_tree_check
    from oracle.tree import accept
    w, eng = setup
    p = synth.prompt(1, w["prompt_len"], w["vocab"])
    print(f"{w['name']}: prefill {len(p)}", flush=True)
    b = eng.prefill(p)
    spec, spec_margin = [b], []
    for cyc in range(CYCLES):
        tree = eng.draft_tree()
        gpu_tree_check(tree, w["topk"], w["depth"], w["budget"], _static(w))
        assert len(tree["token"]) == 1 + (len(w["static"]) if _static(w) else w["budget"])
        new = eng.verify()
        g, mg = eng.debug_read("argmax"), eng.debug_read("margin")
        path, bonus = accept(tree["token"], tree["parent"], g)
        assert new == [tree["token"][r] for r in path] + [bonus]
        spec += new
        spec_margin += [float(mg[r]) for r in [0] + path]
        print(f"{w['name']}: cycle {cyc}: {len(tree['node_token'])} nodes, accepted {len(path)}",
              flush=True)
    # plain greedy decode on the same engine: root-only trees, one token per verify
    assert eng.prefill(p) == b
    plain, plain_margin = [b], []
    for _ in range(len(spec) - 1):
        new = eng.verify(dict(token=[plain[-1]], parent=[-1]))
        assert len(new) == 1
        plain += new
        plain_margin.append(float(eng.debug_read("margin")[0]))
    same = 0
    for i in range(1, len(spec)):
        if spec[i] != plain[i]:
            assert min(spec_margin[i - 1], plain_margin[i - 1]) < TOL, \
                f"token {i}: speculative {spec[i]} plain {plain[i]}"
            break
        same += 1
    print(f"{w['name']}: speculative == plain greedy on {same}/{len(spec) - 1} tokens", flush=True)


def test_full_tree_rows_equal_chains_and_lm_head(setup):
    from oracle.model import Config, Weights, matmul_t
    w, eng = setup
    p = synth.prompt(2, w["prompt_len"], w["vocab"])
    eng.prefill(p)
    tree = eng.draft_tree()
    rows = dict(token=list(tree["token"]), parent=list(tree["parent"]))
    eng.set_debug(True)
    try:
        eng.prefill(p)
        eng.verify(rows)
        lt, ft = eng.debug_read("logits"), eng.debug_read("features")
        # LM head: oracle logits from the GPU's final features on sampled rows
        W = Weights(Config(w), cache_bytes=4 << 30)
        from synth import GLOBAL, LM_HEAD
        wlm = W.get(LM_HEAD, GLOBAL)
        sample = [0, len(rows["token"]) // 2, len(rows["token"]) - 1]
        ref = matmul_t(ft[sample].astype(np.float64), wlm)
        err = np.abs(lt[sample] - ref).max(axis=1) / np.abs(ref).max(axis=1)
        print(f"{w['name']}: LM head rel err {err.max():.2e} on rows {sample}", flush=True)
        assert err.max() < TOL
        # the deepest rows, each verified again as a chain from the root
        depth = np.array(tree["depth"])
        for r in [int(i) for i in np.argsort(-depth, kind="stable")[:3]]:
            chain = [r]
            while rows["parent"][chain[-1]] > 0:
                chain.append(rows["parent"][chain[-1]])
            chain = [0] + chain[::-1]
            eng.prefill(p)
            eng.verify(dict(token=[rows["token"][c] for c in chain],
                            parent=[-1] + list(range(len(chain) - 1))))
            lc = eng.debug_read("logits")
            for j, c in enumerate(chain):
                e = np.abs(lc[j] - lt[c]).max() / np.abs(lt[c]).max()
                assert e < TOL, (r, c, e)
            print(f"{w['name']}: row {r} (depth {depth[r]}) == chain", flush=True)
    finally:
        eng.set_debug(False)


@pytest.mark.timeout(900)
def test_full_depth_teacher_forced(setup):
    """Every layer, a 40-token prompt: each generated token is the oracle's
    greedy choice on the GPU's own prefix, or sits at a margin < 1e-3 (for
    the configs whose full-length pass is not in the default run)."""
    from gpu_helpers import stream_check
    from oracle.model import Config, Weights
    w, eng = setup
    if w["name"] in FULL_LENGTH_DEFAULT:
        pytest.skip(f"{w['name']}: covered at full length by test_full_length_stream_teacher_forced")
    p = synth.prompt(3, 40, w["vocab"])
    got, stats = eng.generate(p, 8)
    print(f"{w['name']}: oracle teacher-forced pass over {len(p) + len(got)} tokens", flush=True)
    W = Weights(Config(w), cache_bytes=4 << 30)
    near = stream_check(w, p, got, W)
    print(f"{w['name']}: {len(got)} tokens, near-ties {near}", flush=True)
    assert near <= 1




@pytest.mark.timeout(1500)
def test_full_length_stream_teacher_forced(setup):
    """The spec check at the config's own size: the committed stream of
    a full-length generation (prompt seed 1) is, token by token, the oracle's
    greedy choice on the GPU's own prefix ([L13] "Speculative decoding in four
    moves": the speculative output equals plain greedy decoding), except at
    positions whose oracle top-1/top-2 margin is below 1e-3, which are counted.
    By induction, a stream that passes at every position is the greedy stream."""
    from gpu_helpers import progress, stream_check
    from oracle.model import Config, Weights
    w, eng = setup
    name = w["name"]
    extra = [c for c in os.environ.get("EAGLE_ORACLE_LONG", "").split(",") if c]
    if name not in FULL_LENGTH_DEFAULT and name not in extra:
        pytest.skip(f"{name}: full-length oracle pass is long; set EAGLE_ORACLE_LONG={name}")
    p = synth.prompt(1, w["prompt_len"], w["vocab"])
    got, stats = eng.generate(p, w["gen"])
    progress(f"{name}: generated {len(got)} tokens in {stats['cycles']} cycles; oracle "
             f"teacher-forced pass over {len(p) + len(got) - 1} tokens")
    W = Weights(Config(w), cache_bytes=4 << 30)
    near = stream_check(w, p, got, W, label=name)
    progress(f"{name}: full-length stream: {len(got)} tokens equal the oracle's greedy choice, "
             f"near-ties {near}")
