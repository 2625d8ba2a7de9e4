"""Shared set-up of GPU tests: a loaded engine with seeded synthetic weights."""
import numpy as np
import torch

import synth
import speculative_decoding_draft_amd as E


def engine(w: dict, max_ctx: int = None, prefill_chunk: int = 0) -> "E.Engine":
    eng = E.Engine(w, max_ctx=max_ctx, prefill_chunk=prefill_chunk)
    synth.fill_weights(eng.table, eng.weights.data_ptr(), w["weight_seed"], eng.stream.cuda_stream)
    torch.cuda.synchronize()
    return eng.load()


def gpu_tree_check(tree: dict, k: int, depth: int, budget: int, static=None):
    """Re-run the oracle's tree policy on the GPU's own nodes and
    log-probabilities; the selection and the verify rows must match."""
    from oracle import tree as T
    nt, npar = tree["node_token"], tree["node_parent"]
    lp = tree["node_logp"]
    kids = {}
    for i, p in enumerate(npar):
        kids.setdefault(p, []).append(i)
    t = T.Tree()

    def expand(chosen):
        ids, lps = [], []
        for e in chosen:
            ch = kids.get(e, [])
            assert len(ch) > 0, f"oracle expands node {e}, the GPU did not"
            ids.append([nt[c] for c in ch])
            lps.append([lp[c] for c in ch])
        return ids, lps
    if static is not None:
        # static tree: GPU nodes follow the list; give each parent a rank-indexed list
        rank = [p[-1] for p in static]

        def rank_list(children):
            ids, lps = [0] * k, [np.float32(-np.inf)] * k
            for c in children:
                ids[rank[c]], lps[rank[c]] = nt[c], lp[c]
            return ids, lps

        def expand_static(chosen):
            out = [rank_list(kids.get(e, [])) for e in chosen]
            return [o[0] for o in out], [o[1] for o in out]
        r_ids, r_lps = rank_list(kids[-1])
        T.grow_static(r_ids, r_lps, expand_static, [tuple(p) for p in static], t)
        kept = list(range(len(t.nodes)))
    else:
        root = kids[-1]
        T.grow_dynamic([nt[c] for c in root], [lp[c] for c in root], expand, k, k, depth, t)
        kept = T.rerank(t.nodes, budget)
    assert [n.token for n in t.nodes] == list(nt)
    assert [n.parent for n in t.nodes] == list(npar)
    assert np.array_equal(np.array([n.logv for n in t.nodes], dtype=np.float32), tree["node_logv"])
    rows = T.flatten(t.nodes, kept, tree["token"][0])
    assert rows["token"] == tree["token"]
    assert rows["parent"] == tree["parent"]
    assert rows["node"] == tree["node"]
    return rows


def progress(msg: str):
    """Print a progress line and, when the run keeps a gpurun_out/ folder in
    the working directory, append it to gpurun_out/test_progress.log (long
    oracle passes otherwise print nothing for minutes under pytest -q)."""
    import os
    import time
    print(msg, flush=True)
    if os.path.isdir("gpurun_out"):
        with open(os.path.join("gpurun_out", "test_progress.log"), "a") as f:
            f.write(f"{time.strftime('%H:%M:%S')} {msg}\n")


def stream_check(w, prompt, stream, weights=None, tol=1e-3, label=None):
    """Teacher-forced check: every token is the oracle's greedy choice on the
    GPU's own prefix, or sits where the oracle's top-1/top-2 margin < tol.
    Returns the number of such near-tie positions (a mismatch elsewhere fails)."""
    from oracle.loop import teacher_forced
    on_layer = None
    if label is not None:
        def on_layer(i):
            if i % 4 == 3:
                progress(f"{label}: oracle layer {i + 1}/{w['n_layers']}")
    g, margin = teacher_forced(w, prompt, stream, weights, on_layer=on_layer)
    near = 0
    for i, tok in enumerate(stream):
        if tok != int(g[i]):
            assert margin[i] < tol, f"token {i}: gpu {tok} oracle {int(g[i])} margin {margin[i]}"
            near += 1
    return near
