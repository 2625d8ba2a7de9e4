"""Workload shapes for the five configurations and their reduced variants.

c1  tiny fp32 Llama-style target, EAGLE-1 head, dynamic tree k=4 D=3 m=16
c2  Llama-2-7B shape, bf16, EAGLE-1 head, static 26-node tree of depth 5
c3  Llama-2-7B shape, bf16, EAGLE-1 head, dynamic tree k=10 D=6 m=60
c4  Llama-3-8B shape (GQA 32/8, vocab 128256), EAGLE-3 head, k=8 D=7 m=64
c5  Llama-2-70B shape (GQA 64/8), bf16, EAGLE-1 head, k=10 D=6 m=60

A "reduced" workload keeps hidden size, heads, vocabulary and tree of a
config but has few layers and a short context, so the CPU oracle can run the
whole speculative loop on it in seconds to minutes.
"""
from __future__ import annotations

import copy

# Static EAGLE-1 tree of c2 as child-rank paths, breadth first (26 nodes,
# per-depth counts 4, 8, 7, 5, 2). Built from a context-free prior over child
# ranks (0.6, 0.2, 0.1, 0.05): the 26 best rank paths of depth <= 5 ranked by
# the sum of log prior, ties by depth then lexicographic order.
STATIC_TREE_C2 = [
    (0,), (1,), (2,), (3,),
    (0, 0), (0, 1), (1, 0), (0, 2), (2, 0), (1, 1), (0, 3), (3, 0),
    (0, 0, 0), (0, 0, 1), (0, 1, 0), (1, 0, 0), (0, 0, 2), (0, 2, 0), (2, 0, 0),
    (0, 0, 0, 0), (0, 0, 1, 0), (0, 1, 0, 0), (1, 0, 0, 0), (0, 0, 0, 1),
    (0, 0, 0, 0, 0), (0, 0, 1, 0, 0),
]

_BASE = dict(rope_base=10000.0, rms_eps=1e-5, head="e1", feat_layers=(0, 0, 0),
             tree="dynamic", static=None, weight_seed=0, prompt_seeds=(1, 2, 3))

WORKLOADS = {
    "c1": dict(_BASE, name="c1", n_layers=2, hidden=256, n_heads=4, n_kv_heads=4,
               ffn=688, vocab=1024, dtype="f32", topk=4, depth=3, budget=16,
               prompt_len=32, gen=64),
    "c2": dict(_BASE, name="c2", n_layers=32, hidden=4096, n_heads=32,
               n_kv_heads=32, ffn=11008, vocab=32000, dtype="bf16",
               tree="static", static=STATIC_TREE_C2, topk=4, depth=5, budget=26,
               prompt_len=512, gen=256),
    "c3": dict(_BASE, name="c3", n_layers=32, hidden=4096, n_heads=32,
               n_kv_heads=32, ffn=11008, vocab=32000, dtype="bf16", topk=10,
               depth=6, budget=60, prompt_len=1536, gen=512),
    "c4": dict(_BASE, name="c4", n_layers=32, hidden=4096, n_heads=32,
               n_kv_heads=8, ffn=14336, vocab=128256, dtype="bf16",
               rope_base=500000.0, head="e3", feat_layers=(2, 16, 29), topk=8,
               depth=7, budget=64, prompt_len=3584, gen=512),
    "c5": dict(_BASE, name="c5", n_layers=80, hidden=8192, n_heads=64,
               n_kv_heads=8, ffn=28672, vocab=32000, dtype="bf16", topk=10,
               depth=6, budget=60, prompt_len=1024, gen=256),
}


def get(name: str) -> dict:
    return copy.deepcopy(WORKLOADS[name])


def reduced(name: str, n_layers: int = 2, prompt_len: int = 80, gen: int = 24) -> dict:
    """Config `name` with few layers and a short context (same H, heads, V, tree)."""
    w = get(name)
    w["name"] = name + "r"
    w["n_layers"] = n_layers if w["head"] == "e1" else max(3, n_layers)
    if w["head"] == "e3":
        w["feat_layers"] = (0, 1, 2)
    w["prompt_len"] = min(prompt_len, w["prompt_len"])
    w["gen"] = min(gen, w["gen"])
    return w


def mini(name: str, prompt_len: int = 24, gen: int = 16) -> dict:
    """Config `name` shrunk to a toy width (H=256, V=512) with the same
    structure: GQA ratio, head type, dtype and tree parameters."""
    w = get(name)
    ratio = w["n_heads"] // w["n_kv_heads"]
    w.update(name=name + "m", hidden=256, n_heads=8, n_kv_heads=max(1, 8 // ratio),
             ffn=344, vocab=512, prompt_len=prompt_len, gen=gen)
    w["n_layers"] = 3 if w["head"] == "e3" else 2
    if w["head"] == "e3":
        w["feat_layers"] = (0, 1, 2)
    return w
