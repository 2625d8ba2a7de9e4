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
    root = kids[-1]
    if static is not None:
        ids0 = {}
        # static: children are listed by rank; rebuild rank-indexed lists
        raise NotImplementedError
    T.grow_dynamic([nt[c] for c in root], [lp[c] for c in root], expand, k, k, depth, t)
    assert [n.token for n in t.nodes] == list(nt)
    assert [n.parent for n in t.nodes] == list(npar)
    assert np.array_equal(np.array([n.logv for n in t.nodes], dtype=np.float32), tree["node_logv"])
    kept = T.rerank(t.nodes, budget)
    rows = T.flatten(t.nodes, kept, tree["token"][0])
    assert rows["token"] == tree["token"]
    assert rows["parent"] == tree["parent"]
    assert rows["node"] == tree["node"]
    return rows
