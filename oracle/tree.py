"""EAGLE-2 tree policy: path values, expansion, global rerank, flattening.

Sources:
  [E2] "Path Value Ranks Prefixes, Not Isolated Tokens": V_i is the product of
       the draft confidences c_j on the root-to-node path; each round expands
       the top-k leaves by V.
  [E2] "Global Reranking Separates Exploration from Verification": after
       expansion keep the m best V over every generated node, shallower
       first on ties, which leaves a connected tree that is then flattened.
  [E2] "The Mask Preserves Tree Semantics in One Target Pass": each flattened
       row sees the root, its ancestors and itself.
  [E2] "Where It Breaks": rank in log space to avoid prefix-product underflow.
  [L13] "EAGLE-2 and dynamic draft trees", "Worked example, step by step" and
       "Practice: try it yourself" (frontier = newest depth; expand the best
       few; rerank everything generated; keep a budget).

Readings taken where the pages leave a choice open:
  * Path values are kept as log V = sum of fp32 log-probabilities, each sum
    rounded to fp32 in root-to-leaf order.
  * Expansion candidates are the nodes of the newest depth ("frontier").
  * Expand width k_e and branching k_b are separate parameters (the worked
    example uses 2 and 2, the practice script 2 and 3, the configs k and k).
  * Ties: expansion by (log V desc, generation order asc); rerank by (log V
    desc, depth asc, generation order asc) -- the page's stable "largest"
    selection keeps generation order among equals.
  * Verify rows: row 0 is the root (the last committed token); then the kept
    nodes by (depth asc, rerank order).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class Node:
    token: int
    parent: int          # index of the parent node, -1 = the root
    depth: int           # 1 for children of the root
    logv: np.float32     # log of the path value
    logp: np.float32     # log of this node's own draft confidence
    gen: int             # generation order (index in the node list)
    rank: int            # child rank within its parent's top-k


@dataclass
class Tree:
    nodes: list = field(default_factory=list)
    expanded: list = field(default_factory=list)   # per draft pass: expanded node ids


def _child(nodes, parent, token, logp, rank, depth):
    base = np.float32(0.0) if parent < 0 else nodes[parent].logv
    lv = np.float32(base + np.float32(logp)) if parent >= 0 else np.float32(logp)
    nodes.append(Node(int(token), parent, depth, lv, np.float32(logp), len(nodes), rank))


def grow_dynamic(root_ids, root_logp, expand, k_e: int, k_b: int, depth: int,
                 t: Tree = None) -> Tree:
    """Grow the EAGLE-2 tree.

    root_ids/root_logp: the root row's top-k_b draft tokens and log-probs.
    expand(node_ids) -> (ids [n, k_b], logp [n, k_b]): the drafter run on the
    rows that expand those nodes, in the given order. `t` (optional) is the
    tree object to grow, so the drafter callback can read its nodes.
    """
    t = Tree() if t is None else t
    for r in range(k_b):
        _child(t.nodes, -1, root_ids[r], root_logp[r], r, 1)
    for d in range(2, depth + 1):
        frontier = [n.gen for n in t.nodes if n.depth == d - 1]
        chosen = sorted(frontier, key=lambda i: (-float(t.nodes[i].logv), i))[:k_e]
        t.expanded.append(chosen)
        ids, lps = expand(chosen)
        for e, row_ids, row_lp in zip(chosen, ids, lps):
            for r in range(k_b):
                _child(t.nodes, e, row_ids[r], row_lp[r], r, d)
    return t


def grow_static(root_ids, root_logp, expand, paths, t: Tree = None) -> Tree:
    """EAGLE-1 static tree given as child-rank paths (breadth first).

    Node order follows `paths`; at depth d the expanded nodes are the
    depth-(d-1) paths that have listed children, in list order, and only the
    listed child ranks are kept.
    """
    t = Tree() if t is None else t
    index = {}
    for p in paths:
        if len(p) == 1:
            index[p] = len(t.nodes)
            _child(t.nodes, -1, root_ids[p[0]], root_logp[p[0]], p[0], 1)
    max_depth = max(len(p) for p in paths)
    for d in range(2, max_depth + 1):
        parents = []
        for p in paths:
            if len(p) == d - 1 and any(len(q) == d and q[:-1] == p for q in paths):
                parents.append(p)
        chosen = [index[p] for p in parents]
        t.expanded.append(chosen)
        ids, lps = expand(chosen)
        row_of = {p: i for i, p in enumerate(parents)}
        for q in paths:
            if len(q) == d:
                i = row_of[q[:-1]]
                index[q] = len(t.nodes)
                _child(t.nodes, index[q[:-1]], ids[i][q[-1]], lps[i][q[-1]], q[-1], d)
    return t


def rerank(nodes, m: int):
    """The m best nodes by (log V desc, depth asc, generation asc), in that order."""
    order = sorted(range(len(nodes)),
                   key=lambda i: (-float(nodes[i].logv), nodes[i].depth, i))
    return order[:m]


def flatten(nodes, kept, root_token: int):
    """Verify rows: root, then kept nodes by (depth asc, order in `kept`).

    Returns dict(token, parent, depth, node) per row; parent is a row index
    (-1 for the root row), node the node index (-1 for the root row).
    """
    pos_in_kept = {n: i for i, n in enumerate(kept)}
    body = sorted(kept, key=lambda n: (nodes[n].depth, pos_in_kept[n]))
    row_of = {n: r + 1 for r, n in enumerate(body)}
    token = [int(root_token)] + [nodes[n].token for n in body]
    parent = [-1] + [0 if nodes[n].parent < 0 else row_of[nodes[n].parent] for n in body]
    depth = [0] + [nodes[n].depth for n in body]
    return dict(token=token, parent=parent, depth=depth, node=[-1] + body)


def ancestors(parent_rows, r: int):
    """Rows on the path from the root to row r, root first, r last."""
    out = [r]
    while parent_rows[out[-1]] >= 0:
        out.append(parent_rows[out[-1]])
    return out[::-1]


def tree_mask(parent_rows):
    """Boolean [n, n]: row i sees row j iff j is i or an ancestor of i."""
    n = len(parent_rows)
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        m[i, ancestors(parent_rows, i)] = True
    return m


def accept(token_rows, parent_rows, g):
    """Greedy acceptance walk ([L13] "Speculative decoding in four moves").

    From the root row, follow the child whose drafted token equals the
    target's greedy choice g at the current row; stop when none does.
    Returns (accepted rows in order, bonus token = g at the last row).
    """
    cur, path = 0, []
    while True:
        nxt = [c for c in range(1, len(token_rows))
               if parent_rows[c] == cur and token_rows[c] == int(g[cur])]
        if not nxt:
            return path, int(g[cur])
        cur = nxt[0]
        path.append(cur)
