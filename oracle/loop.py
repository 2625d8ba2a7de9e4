"""Plain greedy decode and the EAGLE / EAGLE-2 speculative loop.

Sources:
  [L13] "Speculative decoding in four moves": draft, verify in one pass,
        accept from the left while drafted == target's greedy choice, correct
        with the target's token at the first rejection (at least one token
        per pass).
  [L13] "Resolving the uncertainty by feeding back the token": the draft row
        pairs feature f_t with the sampled token t_{t+1}.
  [E3]  section 2.3: features [B,S,H] and tokens shifted by one; every
        deeper draft level is one more draft step on the current leaves.
  [E2]  "Putting It Together": drafter -> expander -> reranker -> mask
        builder -> target and verifier -> next verified state.

Conventions (positions are 0-based; the target KV holds positions 0..ctx-1):
  * the root of a cycle is the last committed token b, at position ctx;
  * a draft row (s, t) sits at t's position p and uses draft KV slot p;
    committed draft rows fill slots 1..ctx (the first prompt token never
    enters the draft); tree rows use slots after ctx and are discarded;
  * a tree node of depth d sits at position ctx + d;
  * after verify the root and the L accepted rows become positions
    ctx..ctx+L (KV compaction), the bonus token becomes the next root, and
    the L+1 new (true feature, token) pairs are drafted again ("catch-up").
"""
from __future__ import annotations

import numpy as np

from .model import Config, Draft, Target, Weights, argmax_lowest, causal_vis
from . import sampling as SMP
from . import tree as T


class Session:
    """Oracle state for one sequence: target + draft KV, committed tokens.
    `lane` is the sequence's index in a batch; it only selects the stream of
    random draws in sampling mode (oracle/sampling.py). `follow`, in sampling
    mode, is another implementation's committed stream: at a sampling
    decision that is a near-tie (oracle/sampling.py) the session takes the
    outcome that stream shows, and its own everywhere else."""

    def __init__(self, w: dict, weights: Weights = None, max_new: int = None, lane: int = 0,
                 follow=None):
        self.w = dict(w)
        self.cfg = Config(w)
        self.W = weights if weights is not None else Weights(self.cfg)
        self.target = Target(self.cfg, self.W)
        self.draft = Draft(self.cfg, self.W)
        self.k = int(w["topk"])
        self.depth = int(w["depth"])
        self.budget = int(w["budget"])
        self.static = w.get("static") if w.get("tree") == "static" else None
        self.max_new = int(max_new if max_new is not None else w["gen"])
        # sampling mode (oracle/sampling.py) when temperature > 0
        self.temperature = float(w.get("temperature", 0.0))
        self.seed = int(w.get("seed", 0))
        self.lane = int(lane)
        self.follow = None if follow is None else [int(t) for t in follow]
        self.sample_margins = []
        self.n_verify = 0
        self.history = []

    # ------------------------------------------------------------ helpers
    def _draft_feats(self, f_rows, kept):
        """Features s for committed draft rows: f (EAGLE-1) or FC([l;m;h]) (EAGLE-3)."""
        if self.cfg.head == "e1":
            return f_rows
        lmh = np.concatenate([kept[i] for i in self.cfg.feat_layers], axis=1)
        return self.draft.fuse(lmh)

    def _catch_up(self, s, tokens, first: int):
        """Draft rows for newly committed pairs (s_i, t_i) at positions first+i."""
        M = len(tokens)
        slots = np.arange(first, first + M)
        vis = causal_vis(M, first, self.dkv[0].shape[0], prefix_from=1)
        out = self.draft.rows(s, tokens, slots, slots, vis, self.dkv)
        self.root_out = out[-1]
        ids, lp, lg = self.draft.topk(out[-1:], self.k)
        self.root_ids, self.root_logp, self.root_logits = ids[0], lp[0], lg[0]

    # ------------------------------------------------------------ prefill
    def prefill(self, prompt):
        prompt = [int(t) for t in prompt]
        n = len(prompt)
        extra = self.budget + self.depth * max(self.k, 1) + self.depth + 8
        n_slots = n + self.max_new + extra
        self.kv = self.target.new_kv(n_slots)
        self.dkv = self.draft.new_kv(n_slots)
        keep = self.cfg.feat_layers if self.cfg.head == "e3" else ()
        pos = np.arange(n)
        f, kept = self.target.forward(prompt, pos, pos, causal_vis(n, 0, n_slots), self.kv, keep)
        last = self.target.logits(f[-1:])
        g, margin = argmax_lowest(last)
        b = int(g[0])
        self.n_verify = 0
        if self.temperature > 0:   # sampling mode: the prefill's token is draw step 0
            want = self.follow[0] if self.follow else None
            b, m = SMP.sample_token(last[0], self.temperature, self.seed, 0, lane=self.lane,
                                    follow=want)
            self.sample_margins = [m]
        self.prefill_margin = float(margin[0])
        self.tokens = prompt + [b]
        self.committed = [b]
        # draft rows j = 1..n: (f_j, t_{j+1}) at positions 1..n
        self._catch_up(self._draft_feats(f, kept), self.tokens[1:], 1)
        self.ctx = n
        return b

    # ------------------------------------------------------------ one cycle
    def draft_tree(self):
        """Grow the draft tree and flatten the kept nodes into verify rows."""
        ctx, k = self.ctx, self.k
        row_out, row_slot = {}, {}
        next_slot = [ctx + 1]
        n_slots = self.dkv[0].shape[0]

        def path_nodes(nodes, e):
            out = [e]
            while nodes[out[-1]].parent >= 0:
                out.append(nodes[out[-1]].parent)
            return out

        t = T.Tree()
        # draft logits of the row expanding each node (-1: the root row), kept
        # so that tests can tell near-ties from real differences
        self.row_logits = {-1: self.root_logits}

        def expand(chosen):
            nodes = t.nodes
            M = len(chosen)
            slots = np.arange(next_slot[0], next_slot[0] + M)
            next_slot[0] += M
            vis = np.zeros((M, n_slots), dtype=bool)
            vis[:, 1:ctx + 1] = True
            s, toks, pos = [], [], []
            for i, e in enumerate(chosen):
                row_slot[e] = slots[i]
                par = nodes[e].parent
                s.append(self.root_out if par < 0 else row_out[par])
                toks.append(nodes[e].token)
                pos.append(ctx + nodes[e].depth)
                for a in path_nodes(nodes, e):
                    vis[i, row_slot[a]] = True
            out = self.draft.rows(np.stack(s), toks, np.array(pos), slots, vis, self.dkv)
            for i, e in enumerate(chosen):
                row_out[e] = out[i]
            ids, lp, lg = self.draft.topk(out, k)
            for i, e in enumerate(chosen):
                self.row_logits[e] = lg[i]
            return ids, lp

        if self.budget == 0:
            kept = []
        elif self.static is not None:
            T.grow_static(self.root_ids, self.root_logp, expand, self.static, t)
            kept = list(range(len(t.nodes)))
        else:
            T.grow_dynamic(self.root_ids, self.root_logp, expand, k, k, self.depth, t)
            kept = T.rerank(t.nodes, self.budget)
        rows = T.flatten(t.nodes, kept, self.tokens[-1])
        self.tree = t
        self.rows = rows
        return t, rows

    def verify(self, rows=None):
        """Target pass over the flattened tree, acceptance, commit, catch-up."""
        rows = self.rows if rows is None else rows
        ctx = self.ctx
        M = len(rows["token"])
        n_slots = self.kv[0].shape[1]
        slots = ctx + np.arange(M)
        pos = ctx + np.array(rows["depth"])
        vis = np.zeros((M, n_slots), dtype=bool)
        vis[:, :ctx] = True
        for r in range(M):
            for a in T.ancestors(rows["parent"], r):
                vis[r, ctx + a] = True
        keep = self.cfg.feat_layers if self.cfg.head == "e3" else ()
        f, kept = self.target.forward(rows["token"], pos, slots, vis, self.kv, keep)
        logits = self.target.logits(f)
        self.last_logits, self.last_features = logits, f
        g, margin = argmax_lowest(logits)
        self.n_verify += 1
        if self.temperature > 0:
            want = None if self.follow is None else self.follow[len(self.committed):]
            path, bonus, m = SMP.walk(rows["token"], rows["parent"], logits, self.temperature,
                                      self.seed, self.n_verify, self.depth, lane=self.lane,
                                      follow=want)
            self.sample_margins += m
        else:
            path, bonus = T.accept(rows["token"], rows["parent"], g)
        L = len(path)
        new = [rows["token"][r] for r in path] + [bonus]
        # KV compaction: row path[j-1] -> position ctx + j (read all, then write)
        if L:
            src = ctx + np.array(path)
            dst = ctx + 1 + np.arange(L)
            for c in self.kv:
                c[:, dst] = c[:, src].copy()
        feat_rows = [0] + path
        kept_rows = {i: v[feat_rows] for i, v in kept.items()}
        s = self._draft_feats(f[feat_rows], kept_rows)
        self.history.append(dict(ctx=ctx, L=L, g=g, margin=margin, rows=rows, new=new))
        self._catch_up(s, new, ctx + 1)
        self.ctx = ctx + L + 1
        self.tokens += new
        self.committed += new
        return path, bonus, g, margin

    def generate(self, prompt, max_new=None):
        max_new = self.max_new if max_new is None else max_new
        self.prefill(prompt)
        while len(self.committed) < max_new:
            self.draft_tree()
            self.verify()
        return self.committed[:max_new]


def greedy_decode(w: dict, prompt, max_new: int, weights: Weights = None):
    """Plain one-token-at-a-time greedy decode with a KV cache (the reference result)."""
    cfg = Config(w)
    W = weights if weights is not None else Weights(cfg)
    tgt = Target(cfg, W)
    prompt = [int(t) for t in prompt]
    n = len(prompt)
    S = n + max_new + 1
    kv = tgt.new_kv(S)
    pos = np.arange(n)
    f, _ = tgt.forward(prompt, pos, pos, causal_vis(n, 0, S), kv)
    g, mg = argmax_lowest(tgt.logits(f[-1:]))
    out, margins = [int(g[0])], [float(mg[0])]
    while len(out) < max_new:
        p = n + len(out) - 1
        vis = np.zeros((1, S), dtype=bool)
        vis[0, :p + 1] = True
        f, _ = tgt.forward([out[-1]], np.array([p]), np.array([p]), vis, kv)
        g, mg = argmax_lowest(tgt.logits(f))
        out.append(int(g[0]))
        margins.append(float(mg[0]))
    return out, margins, kv


def teacher_forced(w: dict, prompt, stream, weights: Weights = None, on_layer=None):
    """One causal pass over prompt + stream[:-1]: the greedy choice and the
    top-1/top-2 margin at every generated position, given that prefix.
    Every row of a causal pass computes what one-token-at-a-time decoding
    computes for it, so this equals greedy decode's choices on that prefix."""
    cfg = Config(w)
    W = weights if weights is not None else Weights(cfg)
    tgt = Target(cfg, W)
    seq = [int(t) for t in prompt] + [int(t) for t in stream[:-1]]
    n = len(seq)
    kv = tgt.new_kv(n)
    pos = np.arange(n)
    f, _ = tgt.forward(seq, pos, pos, causal_vis(n, 0, n), kv, on_layer=on_layer)
    rows = f[len(prompt) - 1:]
    g, margin = argmax_lowest(tgt.logits(rows))
    return g, margin
