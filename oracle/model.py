"""Llama-style target model and EAGLE draft heads, written out plainly.

Target layer (Llama style; the configurations name RMSNorm, RoPE and SwiGLU):
    x  = RMSNorm(h) * gain
    q, k, v = x Wq^T, x Wk^T, x Wv^T      (GQA: query head j reads kv head j // G)
    q, k  <- rotate-half RoPE at the token's position, theta_i = base^(-2i/d)
    o  = softmax(q k^T / sqrt(d) over the visible keys) v
    h += o Wo^T
    h += (SiLU(x2 Wg^T) * (x2 Wu^T)) Wd^T,   x2 = RMSNorm(h) * gain
and the feature f = RMSNorm(h_last) * gain feeds the LM head: logits = f W_lm^T.

EAGLE-1 draft head ([L13] "The big idea: draft at the feature level" and
"Resolving the uncertainty by feeding back the token"; [E3] section 2.3
"Draft 的计算流程"): the row (feature s, token t) forms [E[t]; s] (2H), an FC
maps it back to H, one decoder layer of the target's shape (own weights, own
KV cache) gives f_hat, and the shared frozen LM head turns f_hat into draft
probabilities. The embedding E and the LM head are the target's.

EAGLE-3 draft head ([E3] section 4.3 "多层 feature fusion"): committed rows use
g = FC([l; m; h]) (3H -> H) from three target layers; tree rows use the
parent row's own output a in place of g. The decoder layer reads [E[t]; s]
(2H wide input norm and QKV) with residual stream starting at s; its output
is a, and logits = a W_lm^T.

Parity unpinned: the draft heads' wiring. The pages give the data flow but
not every detail ([E3] lists only "FC 12288->4096, 1 decoder layer" for
EAGLE-3; the concat order and whether the FC output passes through the
layer's input norm are not stated). The readings taken here (concat
[E[t]; s]; E1 FC 2H->H feeding a full Llama layer; E3 with a 2H-wide input
norm and QKV and the residual stream starting at s) are checked only for
internal consistency: tree drafting equals chain drafting along each path,
and the lossless loop. No printed value exists to pin them to.
"""
from __future__ import annotations

import math
from collections import OrderedDict

import numpy as np

import synth
from synth import (ATTN_NORM, DRAFT, EMBED, FC, FFN_NORM, FINAL_NORM, GLOBAL,
                   LM_HEAD, TARGET, WDOWN, WGATE, WK, WO, WQ, WUP, WV)

from .numerics import apply_rope, kv_store, log_softmax, operand, rmsnorm, rope_tables, silu, to_f32


class Config:
    """Model shape and numerics of one workload (see synth.workloads)."""

    def __init__(self, w: dict):
        self.w = dict(w)
        for key in ("n_layers", "hidden", "n_heads", "n_kv_heads", "ffn", "vocab"):
            setattr(self, key, int(w[key]))
        self.rope_base = float(w["rope_base"])
        self.eps = float(w["rms_eps"])
        self.dtype = w["dtype"]
        self.head = w["head"]
        self.feat_layers = tuple(int(x) for x in w["feat_layers"])
        self.head_dim = self.hidden // self.n_heads
        self.group = self.n_heads // self.n_kv_heads
        self.seed = int(w.get("weight_seed", 0))

    def shape(self, kind: int, group: int):
        H, d, F, V = self.hidden, self.head_dim, self.ffn, self.vocab
        qd, kvd = self.n_heads * d, self.n_kv_heads * d
        e3 = self.head == "e3" and group == DRAFT
        kin = 2 * H if e3 else H      # K-dim of the EAGLE-3 decoder's norm and QKV
        return {
            EMBED: (V, H), LM_HEAD: (V, H), FINAL_NORM: (H,),
            FC: (H, 3 * H) if self.head == "e3" else (H, 2 * H),
            ATTN_NORM: (kin,), WQ: (qd, kin), WK: (kvd, kin), WV: (kvd, kin),
            WO: (H, qd), FFN_NORM: (H,), WGATE: (F, H), WUP: (F, H), WDOWN: (H, F),
        }[kind]


class Weights:
    """Weight tensors regenerated from the seeded generator (cached as fp32).

    A byte budget bounds the cache, so 7B-70B shapes are rebuilt layer by
    layer instead of being held whole. Evicted arrays are kept for reuse by
    the next tensor of the same shape (layers repeat shapes), because writing
    into fresh memory costs more than generating the values.
    """

    def __init__(self, cfg: Config, cache_bytes: int = 24 << 30):
        self.cfg = cfg
        self.cache = OrderedDict()
        self.spare = []          # evicted arrays, reusable as output buffers
        self.budget = cache_bytes
        self.used = 0            # bytes in cache and spare

    def _buffer(self, shape, nb):
        for i, a in enumerate(self.spare):
            if a.shape == tuple(shape):
                return self.spare.pop(i)
        while self.used + nb > self.budget and (self.cache or self.spare):
            if self.spare:
                self.used -= self.spare.pop(0).nbytes
            else:
                _, old = self.cache.popitem(last=False)
                if old.shape == tuple(shape):
                    return old
                self.spare.append(old)
        self.used += nb
        return np.empty(shape, dtype=np.float32)

    def get(self, kind: int, group: int, layer: int = 0) -> np.ndarray:
        key = (kind, group, layer)
        if key in self.cache:
            self.cache.move_to_end(key)
            return self.cache[key]
        shape = tuple(self.cfg.shape(kind, group))
        nb = int(np.prod(shape)) * 4
        if nb > self.budget:
            return synth.tensor_values(self.cfg.seed, kind, group, layer, shape, self.cfg.dtype)
        out = self._buffer(shape, nb)
        arr = synth.tensor_values(self.cfg.seed, kind, group, layer, shape, self.cfg.dtype, out=out)
        self.cache[key] = arr
        return arr


_F64 = {}


def _f64_buffer(shape) -> np.ndarray:
    """A persistent fp64 scratch array (reused across calls, so the weight
    chunks below are widened into memory that is already mapped)."""
    n = int(np.prod(shape))
    buf = _F64.get("w")
    if buf is None or buf.size < n:
        buf = np.empty(n, dtype=np.float64)
        _F64["w"] = buf
    return buf[:n].reshape(shape)


def matmul_t(x, w32, chunk: int = 2048):
    """x @ w^T in fp64 (x [M,K] fp64, w [N,K] fp32), processed in row blocks of w."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty((x.shape[0], w32.shape[0]), dtype=np.float64)
    for n0 in range(0, w32.shape[0], chunk):
        wc = w32[n0:n0 + chunk]
        w64 = _f64_buffer(wc.shape)
        np.copyto(w64, wc)          # exact widening of fp32 to fp64
        out[:, n0:n0 + chunk] = x @ w64.T
    return out


def attention(q, kc, vc, vis, scale: float):
    """softmax(q k^T * scale over visible keys) v, per head, GQA.

    q [M, nq, d]; kc, vc [S, nkv, d]; vis bool [M, S] (row i sees key slot j).
    """
    M, nq, d = q.shape
    nkv = kc.shape[1]
    G = nq // nkv
    out = np.empty((M, nq, d), dtype=np.float64)
    for j in range(nkv):
        qj = q[:, j * G:(j + 1) * G, :].reshape(M * G, d)
        s = (qj @ kc[:, j, :].T) * scale                       # [M*G, S]
        s = np.where(np.repeat(vis, G, axis=0), s, -np.inf)
        s = s - np.max(s, axis=1, keepdims=True)
        p = np.exp(s)
        p = p / np.sum(p, axis=1, keepdims=True)
        out[:, j * G:(j + 1) * G, :] = (p @ vc[:, j, :]).reshape(M, G, d)
    return out


def decoder_layer(cfg: Config, W: Weights, group: int, layer: int, h, pos,
                  kc, vc, slots, vis, x_in=None):
    """One Llama decoder layer over M rows; writes the rows' K/V to `slots`.

    h: residual stream [M, H]; x_in: input of the first norm when it is not h
    (the EAGLE-3 decoder reads [E[t]; s]). kc, vc: this layer's cache
    [S, nkv, d], updated in place before attention (a row sees itself).
    """
    dt, d = cfg.dtype, cfg.head_dim
    M = h.shape[0]
    src = h if x_in is None else x_in
    x = operand(rmsnorm(src, W.get(ATTN_NORM, group, layer), cfg.eps), dt)
    q = to_f32(matmul_t(x, W.get(WQ, group, layer))).reshape(M, cfg.n_heads, d)
    k = to_f32(matmul_t(x, W.get(WK, group, layer))).reshape(M, cfg.n_kv_heads, d)
    v = to_f32(matmul_t(x, W.get(WV, group, layer))).reshape(M, cfg.n_kv_heads, d)
    cos, sin = rope_tables(pos, d, cfg.rope_base)
    q = to_f32(apply_rope(q, cos, sin))
    k = to_f32(apply_rope(k, cos, sin))
    kc[slots] = kv_store(k, dt)
    vc[slots] = kv_store(v, dt)
    o = to_f32(attention(operand(q, dt), kc, vc, vis, 1.0 / math.sqrt(d)))
    h = to_f32(h + to_f32(matmul_t(operand(o.reshape(M, -1), dt), W.get(WO, group, layer))))
    x2 = operand(rmsnorm(h, W.get(FFN_NORM, group, layer), cfg.eps), dt)
    a = to_f32(matmul_t(x2, W.get(WGATE, group, layer)))
    b = to_f32(matmul_t(x2, W.get(WUP, group, layer)))
    m = operand(silu(a) * b, dt)
    return to_f32(h + to_f32(matmul_t(m, W.get(WDOWN, group, layer))))


class Target:
    """The frozen target model."""

    def __init__(self, cfg: Config, W: Weights):
        self.cfg, self.W = cfg, W

    def new_kv(self, n_slots: int):
        c = self.cfg
        shp = (c.n_layers, n_slots, c.n_kv_heads, c.head_dim)
        return np.zeros(shp), np.zeros(shp)

    def forward(self, tokens, pos, slots, vis, kv, keep=(), on_layer=None):
        """Rows (token, position) -> (f [M,H] post final norm, {layer: h after it}).
        on_layer(i), when given, is called after layer i (progress of long passes)."""
        c = self.cfg
        h = self.W.get(EMBED, GLOBAL)[np.asarray(tokens)].astype(np.float64)
        kept = {}
        for layer in range(c.n_layers):
            h = decoder_layer(c, self.W, TARGET, layer, h, pos, kv[0][layer], kv[1][layer],
                              slots, vis)
            if layer in keep:
                kept[layer] = h.copy()
            if on_layer is not None:
                on_layer(layer)
        f = to_f32(rmsnorm(h, self.W.get(FINAL_NORM, GLOBAL), c.eps))
        return f, kept

    def logits(self, f):
        return to_f32(matmul_t(operand(f, self.cfg.dtype), self.W.get(LM_HEAD, GLOBAL)))


class Draft:
    """EAGLE-1 or EAGLE-3 draft head sharing the target's embedding and LM head.

    Parity unpinned (the wiring; see the module docstring): its tree rows
    are pinned to chain drafting, not to values printed on the pages."""

    def __init__(self, cfg: Config, W: Weights):
        self.cfg, self.W = cfg, W

    def new_kv(self, n_slots: int):
        c = self.cfg
        shp = (n_slots, c.n_kv_heads, c.head_dim)
        return np.zeros(shp), np.zeros(shp)

    def fuse(self, lmh):
        """EAGLE-3: g = FC([l; m; h]) for committed rows (lmh [M, 3H])."""
        return to_f32(matmul_t(operand(lmh, self.cfg.dtype), self.W.get(FC, GLOBAL)))

    def rows(self, s, tokens, pos, slots, vis, kv):
        """Draft rows (s, t) at positions pos -> output feature (f_hat or a) [M, H]."""
        c = self.cfg
        e = self.W.get(EMBED, GLOBAL)[np.asarray(tokens)].astype(np.float64)
        if c.head == "e1":
            x_in = np.concatenate([e, operand(s, c.dtype)], axis=1)
            h = to_f32(matmul_t(x_in, self.W.get(FC, GLOBAL)))
            return decoder_layer(c, self.W, DRAFT, 0, h, pos, kv[0], kv[1], slots, vis)
        x_in = np.concatenate([e, s], axis=1)
        return decoder_layer(c, self.W, DRAFT, 0, to_f32(s), pos, kv[0], kv[1], slots, vis,
                             x_in=x_in)

    def logits(self, out):
        return to_f32(matmul_t(operand(out, self.cfg.dtype), self.W.get(LM_HEAD, GLOBAL)))

    def topk(self, out, k: int):
        """Per row: k best ids by (logit desc, id asc) and their log-probabilities.

        Draft confidence is the full-vocabulary softmax probability
        ([E2] "Calibration Makes Acceptance Estimation Cheap"); logp is
        l - max - log(sum exp(l - max)) rounded to fp32.
        """
        lg = self.logits(out)
        lp = to_f32(log_softmax(lg))
        ids = np.empty((lg.shape[0], k), dtype=np.int64)
        for r in range(lg.shape[0]):
            order = np.lexsort((np.arange(lg.shape[1]), -lg[r]))
            ids[r] = order[:k]
        return ids, np.take_along_axis(lp, ids, axis=1).astype(np.float32), lg


def argmax_lowest(logits):
    """Greedy choice per row with ties to the lowest id, and top-1 minus top-2."""
    lg = np.atleast_2d(logits)
    g = np.argmax(lg, axis=1)             # numpy returns the first maximum
    srt = np.sort(lg, axis=1)
    return g, srt[:, -1] - srt[:, -2]


def causal_vis(n_rows: int, first_slot: int, n_slots: int, prefix_from: int = 0):
    """Row i sees slots [prefix_from, first_slot + i]."""
    vis = np.zeros((n_rows, n_slots), dtype=bool)
    for i in range(n_rows):
        vis[i, prefix_from:first_slot + i + 1] = True
    return vis
