"""Python binding of libeagle.so: one EAGLE / EAGLE-2 draft-and-verify cycle
on an MI355X (gfx950), for one sequence or a batch of lanes.

Argument marshalling only: every step of the cycle runs in the library's
HIP kernels. PyTorch provides device memory (three uint8 tensors sized by
``eagle_query``) and the HIP stream. There is no CPU fallback: if the
library is not built, importing `lib()` raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libeagle.so")

MAX_STATIC, MAX_DEPTH, MAX_VERIFY, MAX_NODES, MAX_TOPK, MAX_BATCH = 64, 16, 128, 1024, 16, 8
F32, BF16 = 0, 1
OK, E_INVALID, E_STATE, E_CAPACITY, E_BUFFER, E_HIP, E_DEVICE = range(7)
HEAD_E1, HEAD_E3 = 0, 1
TREE_DYNAMIC, TREE_STATIC = 0, 1
STATUS = {0: "EAGLE_OK", 1: "EAGLE_E_INVALID", 2: "EAGLE_E_STATE", 3: "EAGLE_E_CAPACITY",
          4: "EAGLE_E_BUFFER", 5: "EAGLE_E_HIP", 6: "EAGLE_E_DEVICE"}

i32, i64, u64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float


class Config(ctypes.Structure):
    _fields_ = [("n_layers", i32), ("hidden", i32), ("n_heads", i32), ("n_kv_heads", i32),
                ("ffn", i32), ("vocab", i32), ("rope_base", f32), ("rms_eps", f32),
                ("dtype", i32), ("head", i32), ("feat_layers", i32 * 3), ("tree", i32),
                ("topk", i32), ("expand", i32), ("depth", i32), ("budget", i32),
                ("n_static", i32), ("static_parent", i32 * MAX_STATIC),
                ("static_rank", i32 * MAX_STATIC), ("max_ctx", i32), ("prefill_chunk", i32),
                ("temperature", f32), ("seed_lo", ctypes.c_uint32), ("seed_hi", ctypes.c_uint32),
                ("batch", i32)]


class Sizes(ctypes.Structure):
    _fields_ = [("weight_bytes", u64), ("kv_bytes", u64), ("scratch_bytes", u64),
                ("n_tensors", i32), ("verify_rows", i32), ("max_nodes", i32), ("kv_page", i32),
                ("ctx_headroom", i32)]


class Tensor(ctypes.Structure):
    _fields_ = [("kind", i32), ("group", i32), ("layer", i32), ("dtype", i32),
                ("rows", i64), ("cols", i64), ("offset", u64)]


class Buffers(ctypes.Structure):
    _fields_ = [("weights", ctypes.c_void_p), ("weight_bytes", u64),
                ("kv", ctypes.c_void_p), ("kv_bytes", u64),
                ("scratch", ctypes.c_void_p), ("scratch_bytes", u64)]


class Tree(ctypes.Structure):
    _fields_ = [("n_rows", i32), ("token", i32 * MAX_VERIFY), ("parent", i32 * MAX_VERIFY),
                ("depth", i32 * MAX_VERIFY), ("logv", f32 * MAX_VERIFY),
                ("node", i32 * MAX_VERIFY), ("n_nodes", i32),
                ("node_token", i32 * MAX_NODES), ("node_parent", i32 * MAX_NODES),
                ("node_depth", i32 * MAX_NODES), ("node_logv", f32 * MAX_NODES),
                ("node_logp", f32 * MAX_NODES)]


# profile classes, in the order of the EAGLE_PROF_* constants
PROF_CLASSES = ["gemm", "attention", "lmhead", "rows", "tree", "kv", "swiglu", "draft"]
PROF_ALL = 0xFFFFFFFF


class Profile(ctypes.Structure):
    _n = len(PROF_CLASSES)
    _fields_ = [("launches", i64 * _n), ("ms", ctypes.c_double * _n), ("bytes", ctypes.c_double * _n)]


class Stats(ctypes.Structure):
    _fields_ = [("cycles", i64), ("committed", i64), ("accept_hist", i64 * (MAX_DEPTH + 1)),
                ("seconds", ctypes.c_double)]


_lib = None


def lib():
    """The loaded libeagle.so (torch is imported first so the library binds
    to the HIP runtime torch already loaded)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp = ctypes.c_void_p
        L.eagle_query.argtypes = [P(Config), P(Sizes)]
        L.eagle_tensor_info.argtypes = [P(Config), i32, P(Tensor)]
        L.eagle_load.argtypes = [P(Config), P(Buffers), vp, P(vp)]
        L.eagle_prefill.argtypes = [vp, P(i32), i32, P(i32)]
        L.eagle_prefill_lane.argtypes = [vp, i32, P(i32), i32, P(i32)]
        L.eagle_draft_tree.argtypes = [vp, P(Tree)]
        L.eagle_read_tree.argtypes = [vp, i32, P(Tree)]
        L.eagle_verify.argtypes = [vp, P(Tree), P(i32), P(i32)]
        L.eagle_verify_batch.argtypes = [vp, P(i32), P(i32)]
        L.eagle_generate.argtypes = [vp, P(i32), i32, i32, P(i32), P(i32), P(Stats)]
        L.eagle_committed.argtypes = [vp, P(i32), i32, P(i32)]
        L.eagle_committed_lane.argtypes = [vp, i32, P(i32), i32, P(i32)]
        L.eagle_debug_read.argtypes = [vp, i32, vp, u64, P(i32)]
        L.eagle_set_debug.argtypes = [vp, i32]
        L.eagle_set_sampling.argtypes = [vp, f32, ctypes.c_uint32, ctypes.c_uint32]
        L.eagle_profile_enable.argtypes = [vp, ctypes.c_uint32, i32]
        L.eagle_profile_read.argtypes = [vp, P(Profile)]
        L.eagle_free.argtypes = [vp]
        L.eagle_free.restype = None
        L.eagle_last_error.argtypes = [vp]
        L.eagle_last_error.restype = ctypes.c_char_p
        L.eagle_status_string.argtypes = [i32]
        L.eagle_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


class EagleError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def make_config(w: dict, max_ctx: int = None, prefill_chunk: int = 0) -> Config:
    """eagle_config for a workload dict (see synth.workloads)."""
    c = Config()
    c.n_layers, c.hidden, c.n_heads = w["n_layers"], w["hidden"], w["n_heads"]
    c.n_kv_heads, c.ffn, c.vocab = w["n_kv_heads"], w["ffn"], w["vocab"]
    c.rope_base, c.rms_eps = float(w["rope_base"]), float(w["rms_eps"])
    c.dtype = BF16 if w["dtype"] == "bf16" else F32
    c.head = HEAD_E3 if w["head"] == "e3" else HEAD_E1
    for i, v in enumerate(w.get("feat_layers", (0, 0, 0))):
        c.feat_layers[i] = int(v)
    c.topk, c.expand, c.depth, c.budget = w["topk"], w.get("expand", 0), w["depth"], w["budget"]
    if w.get("tree") == "static":
        c.tree = TREE_STATIC
        paths = [tuple(p) for p in w["static"]]
        index = {p: i for i, p in enumerate(paths)}
        c.n_static = len(paths)
        for i, p in enumerate(paths):
            c.static_parent[i] = index[p[:-1]] if len(p) > 1 else -1
            c.static_rank[i] = p[-1]
    else:
        c.tree = TREE_DYNAMIC
    if max_ctx is None:
        max_ctx = w["prompt_len"] + w["gen"] + w["depth"] + 2
    c.max_ctx = int(max_ctx)
    c.prefill_chunk = int(prefill_chunk)
    c.temperature = float(w.get("temperature", 0.0))
    seed = int(w.get("seed", 0))
    c.seed_lo, c.seed_hi = seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF
    c.batch = int(w.get("batch", 1))
    return c


def query(cfg: Config) -> Sizes:
    s = Sizes()
    rc = lib().eagle_query(ctypes.byref(cfg), ctypes.byref(s))
    if rc:
        raise EagleError(rc, "eagle_query rejected the configuration")
    return s


def tensor_table(cfg: Config):
    n = query(cfg).n_tensors
    out = []
    for i in range(n):
        t = Tensor()
        rc = lib().eagle_tensor_info(ctypes.byref(cfg), i, ctypes.byref(t))
        if rc:
            raise EagleError(rc, f"eagle_tensor_info({i})")
        out.append(dict(kind=t.kind, group=t.group, layer=t.layer, dtype=t.dtype,
                        rows=t.rows, cols=t.cols, offset=t.offset))
    return out


def _i32p(a):
    return a.ctypes.data_as(ctypes.POINTER(i32))


class Engine:
    """One context over torch-allocated device buffers.

    Usage: e = Engine(workload); fill e.weights per e.table; e.load();
    then e.prefill / e.draft_tree / e.verify, or e.generate.
    """

    def __init__(self, w: dict, max_ctx: int = None, prefill_chunk: int = 0, device: str = "cuda"):
        import torch
        self.w = dict(w)
        self.cfg = make_config(w, max_ctx, prefill_chunk)
        self.sizes = query(self.cfg)
        self.table = tensor_table(self.cfg)
        self.weights = torch.empty(self.sizes.weight_bytes, dtype=torch.uint8, device=device)
        self.kv = torch.empty(self.sizes.kv_bytes, dtype=torch.uint8, device=device)
        self.scratch = torch.empty(self.sizes.scratch_bytes, dtype=torch.uint8, device=device)
        self.stream = torch.cuda.current_stream()
        self.ctx = None

    # ------------------------------------------------------------ plumbing
    def _check(self, rc, what):
        if rc:
            msg = lib().eagle_last_error(self.ctx).decode() if self.ctx else ""
            raise EagleError(rc, f"{what}: {msg}")

    def load(self):
        b = Buffers(self.weights.data_ptr(), self.sizes.weight_bytes, self.kv.data_ptr(),
                    self.sizes.kv_bytes, self.scratch.data_ptr(), self.sizes.scratch_bytes)
        ctx = ctypes.c_void_p()
        rc = lib().eagle_load(ctypes.byref(self.cfg), ctypes.byref(b),
                              ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(ctx))
        if rc:
            raise EagleError(rc, "eagle_load")
        self.ctx = ctx
        return self

    def close(self):
        if self.ctx:
            lib().eagle_free(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------ calls
    def prefill(self, prompt, lane: int = 0) -> int:
        p = np.ascontiguousarray(prompt, dtype=np.int32)
        b = i32()
        self._check(lib().eagle_prefill_lane(self.ctx, lane, _i32p(p), len(p), ctypes.byref(b)),
                    "eagle_prefill_lane")
        return int(b.value)

    def draft_tree(self, want: bool = True):
        """Drafts every lane's tree; returns lane 0's (or None)."""
        t = Tree() if want else None
        self._check(lib().eagle_draft_tree(self.ctx, ctypes.byref(t) if want else None),
                    "eagle_draft_tree")
        return tree_to_dict(t) if want else None

    def read_tree(self, lane: int):
        t = Tree()
        self._check(lib().eagle_read_tree(self.ctx, lane, ctypes.byref(t)), "eagle_read_tree")
        return tree_to_dict(t)

    def verify_batch(self):
        """Verifies every lane's drafted tree; returns each lane's committed tokens."""
        B = max(self.cfg.batch, 1)
        out = (i32 * (B * (MAX_DEPTH + 1)))()
        n = (i32 * B)()
        self._check(lib().eagle_verify_batch(self.ctx, out, n), "eagle_verify_batch")
        return [list(out[b * (MAX_DEPTH + 1):b * (MAX_DEPTH + 1) + n[b]]) for b in range(B)]

    def verify(self, planted: dict = None):
        tp = None
        if planted is not None:
            tp = Tree()
            n = len(planted["token"])
            tp.n_rows = n
            for r in range(n):
                tp.token[r] = int(planted["token"][r])
                tp.parent[r] = int(planted["parent"][r])
        out = (i32 * (MAX_DEPTH + 1))()
        n = i32()
        self._check(lib().eagle_verify(self.ctx, ctypes.byref(tp) if tp is not None else None,
                                       out, ctypes.byref(n)), "eagle_verify")
        return list(out[:n.value])

    def generate(self, prompt, max_new: int):
        p = np.ascontiguousarray(prompt, dtype=np.int32)
        out = np.zeros(max_new, dtype=np.int32)
        n = i32()
        st = Stats()
        self._check(lib().eagle_generate(self.ctx, _i32p(p), len(p), max_new, _i32p(out),
                                         ctypes.byref(n), ctypes.byref(st)), "eagle_generate")
        stats = dict(cycles=st.cycles, committed=st.committed, seconds=st.seconds,
                     accept_hist=list(st.accept_hist))
        return out[:n.value].tolist(), stats

    def committed(self, lane: int = 0):
        n = i32()
        self._check(lib().eagle_committed_lane(self.ctx, lane, None, 0, ctypes.byref(n)),
                    "eagle_committed_lane")
        out = np.zeros(max(n.value, 1), dtype=np.int32)
        self._check(lib().eagle_committed_lane(self.ctx, lane, _i32p(out), n.value, ctypes.byref(n)),
                    "eagle_committed_lane")
        return out[:n.value].tolist()

    def profile(self, on=True, every: int = 1):
        """Enable profiling: True for every class, False to stop, or an iterable of
        class names (PROF_CLASSES) to bracket only those launches; one launch in
        `every` of each class is bracketed."""
        if on is True:
            mask = PROF_ALL
        elif not on:
            mask = 0
        else:
            mask = 0
            for name in on:
                mask |= 1 << PROF_CLASSES.index(name)
        self._check(lib().eagle_profile_enable(self.ctx, ctypes.c_uint32(mask), int(every)),
                    "eagle_profile_enable")

    def profile_read(self) -> dict:
        p = Profile()
        self._check(lib().eagle_profile_read(self.ctx, ctypes.byref(p)), "eagle_profile_read")
        return {name: dict(launches=p.launches[i], ms=p.ms[i], bytes=p.bytes[i])
                for i, name in enumerate(PROF_CLASSES)}

    def set_sampling(self, temperature: float, seed: int = 0):
        """Temperature (0 = greedy) and seed of the draws, from the next call."""
        self._check(lib().eagle_set_sampling(self.ctx, float(temperature), seed & 0xFFFFFFFF,
                                             (seed >> 32) & 0xFFFFFFFF), "eagle_set_sampling")

    def set_debug(self, on: bool = True):
        self._check(lib().eagle_set_debug(self.ctx, 1 if on else 0), "eagle_set_debug")

    def debug_read(self, what: str):
        """'features' [rows,H] f32, 'logits' [rows,V] f32, 'argmax' [rows] i32, 'margin' [rows] f32."""
        code = {"features": 0, "logits": 1, "argmax": 2, "margin": 3}[what]
        width = {0: self.cfg.hidden, 1: self.cfg.vocab, 2: 1, 3: 1}[code]
        dt = np.int32 if code == 2 else np.float32
        rows = i32()
        B = max(self.cfg.batch, 1)
        rows_cap = B * MAX_VERIFY if code else max(B * self.sizes.verify_rows, 1024)
        buf = np.zeros(rows_cap * width, dtype=dt)
        self._check(lib().eagle_debug_read(self.ctx, code, buf.ctypes.data, buf.nbytes,
                                           ctypes.byref(rows)), "eagle_debug_read")
        return buf[:rows.value * width].reshape(rows.value, width) if width > 1 else buf[:rows.value]


def tree_to_dict(t: Tree) -> dict:
    n, m = t.n_rows, t.n_nodes
    return dict(token=list(t.token[:n]), parent=list(t.parent[:n]), depth=list(t.depth[:n]),
                logv=np.array(t.logv[:n], dtype=np.float32), node=list(t.node[:n]),
                node_token=list(t.node_token[:m]), node_parent=list(t.node_parent[:m]),
                node_depth=list(t.node_depth[:m]),
                node_logv=np.array(t.node_logv[:m], dtype=np.float32),
                node_logp=np.array(t.node_logp[:m], dtype=np.float32))


# ---------------------------------------------------------------- kernel ops
def op_pack(src, dst, N: int, K: int, stream=None):
    """eagle_op_pack: fragment-pack the bf16 weight src [N, K] into dst."""
    L = lib()
    L.eagle_op_pack.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i32, i32, ctypes.c_void_p]
    st = stream.cuda_stream if stream is not None else _torch_stream()
    rc = L.eagle_op_pack(src.data_ptr(), dst.data_ptr(), N, K, st)
    if rc:
        raise EagleError(rc, "eagle_op_pack")


def op_linear(dtype: int, epilogue: int, x, w, y, M: int, N: int, K: int, workspace=None,
              stream=None):
    """eagle_op_linear on torch tensors (device pointers)."""
    L = lib()
    L.eagle_op_linear_workspace.argtypes = [i32, i32, i32, i32, i32]
    L.eagle_op_linear_workspace.restype = u64
    L.eagle_op_linear.argtypes = [i32, i32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  i32, i32, i32, ctypes.c_void_p, u64, ctypes.c_void_p]
    need = L.eagle_op_linear_workspace(dtype, epilogue, M, N, K)
    ws_ptr, ws_bytes = (workspace.data_ptr(), workspace.numel()) if workspace is not None else (None, 0)
    if need > ws_bytes:
        raise EagleError(4, f"linear workspace needs {need} bytes")
    st = stream.cuda_stream if stream is not None else _torch_stream()
    rc = L.eagle_op_linear(dtype, epilogue, x.data_ptr(), w.data_ptr(), y.data_ptr(), M, N, K,
                           ws_ptr, ws_bytes, st)
    if rc:
        raise EagleError(rc, "eagle_op_linear")


def op_norm_linear_workspace(epilogue: int, M: int, N: int, H: int) -> int:
    L = lib()
    L.eagle_op_norm_linear_workspace.argtypes = [i32, i32, i32, i32]
    L.eagle_op_norm_linear_workspace.restype = u64
    return int(L.eagle_op_norm_linear_workspace(epilogue, M, N, H))


def op_norm_linear(epilogue: int, h, part, S: int, gain, eps: float, w, y, M: int, N: int, H: int,
                   workspace, stream=None):
    """eagle_op_norm_linear on torch tensors (device pointers): h += planes,
    then the projection of RMSNorm(h) * gain (bf16)."""
    L = lib()
    L.eagle_op_norm_linear.argtypes = [i32, ctypes.c_void_p, ctypes.c_void_p, i32, ctypes.c_void_p,
                                       f32, ctypes.c_void_p, ctypes.c_void_p, i32, i32, i32,
                                       ctypes.c_void_p, u64, ctypes.c_void_p]
    need = op_norm_linear_workspace(epilogue, M, N, H)
    if need == 0:
        raise EagleError(1, "eagle_op_norm_linear: bad shape")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        raise EagleError(4, f"norm_linear workspace needs {need} bytes")
    st = stream.cuda_stream if stream is not None else _torch_stream()
    rc = L.eagle_op_norm_linear(epilogue, h.data_ptr(), part.data_ptr() if part is not None else None,
                                S, gain.data_ptr(), eps, w.data_ptr(), y.data_ptr(), M, N, H,
                                workspace.data_ptr(), workspace.numel() * workspace.element_size(), st)
    if rc:
        raise EagleError(rc, "eagle_op_norm_linear")


NOALLOC_SCRATCH_BYTES = 32 << 20   # EAGLE_OP_NOALLOC_SCRATCH_BYTES


def op_linear_noalloc(dtype: int, epilogue: int, x, w, y, M: int, N: int, K: int, stream=None):
    """eagle_op_linear_noalloc: eagle_op_linear with the library's own fixed
    device array as its workspace (no allocation anywhere)."""
    L = lib()
    L.eagle_op_linear_noalloc.argtypes = [i32, i32, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, i32, i32, i32, ctypes.c_void_p]
    st = stream.cuda_stream if stream is not None else _torch_stream()
    rc = L.eagle_op_linear_noalloc(dtype, epilogue, x.data_ptr(), w.data_ptr(), y.data_ptr(),
                                   M, N, K, st)
    if rc:
        raise EagleError(rc, "eagle_op_linear_noalloc")


def op_linear_workspace(dtype, epilogue, M, N, K) -> int:
    L = lib()
    L.eagle_op_linear_workspace.argtypes = [i32, i32, i32, i32, i32]
    L.eagle_op_linear_workspace.restype = u64
    return int(L.eagle_op_linear_workspace(dtype, epilogue, M, N, K))


def op_lmhead(dtype: int, k: int, x, w, M: int, V: int, H: int, ids, vals, logits=None,
              workspace=None, stream=None):
    L = lib()
    L.eagle_op_lmhead_workspace.argtypes = [i32, i32, i32]
    L.eagle_op_lmhead_workspace.restype = u64
    L.eagle_op_lmhead.argtypes = [i32, i32, ctypes.c_void_p, ctypes.c_void_p, i32, i32, i32,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, u64, ctypes.c_void_p]
    need = L.eagle_op_lmhead_workspace(M, V, k)
    if workspace is None or workspace.numel() < need:
        raise EagleError(4, f"lmhead workspace needs {need} bytes")
    st = stream.cuda_stream if stream is not None else _torch_stream()
    rc = L.eagle_op_lmhead(dtype, k, x.data_ptr(), w.data_ptr(), M, V, H, ids.data_ptr(),
                           vals.data_ptr(), logits.data_ptr() if logits is not None else None,
                           workspace.data_ptr(), workspace.numel(), st)
    if rc:
        raise EagleError(rc, "eagle_op_lmhead")


def op_attention_workspace(dtype, M, n_heads, head_dim, key_end) -> int:
    L = lib()
    L.eagle_op_attention_workspace.argtypes = [i32, i32, i32, i32, i32]
    L.eagle_op_attention_workspace.restype = u64
    return int(L.eagle_op_attention_workspace(dtype, M, n_heads, head_dim, key_end))


def op_attention(dtype: int, q, kv, page_table, n_kv_heads: int, n_heads: int, head_dim: int,
                 M: int, pre_lo: int, prehi, tree_mask, tree_base: int, n_tree: int, key_end: int,
                 scale: float, out, workspace=None, stream=None):
    """eagle_op_attention on torch tensors (device pointers)."""
    L = lib()
    vp = ctypes.c_void_p
    L.eagle_op_attention.argtypes = [i32, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, i32, i32,
                                     i32, f32, vp, vp, u64, vp]
    st = stream.cuda_stream if stream is not None else _torch_stream()
    ws_ptr, ws_bytes = (workspace.data_ptr(), workspace.numel()) if workspace is not None else (None, 0)
    rc = L.eagle_op_attention(dtype, q.data_ptr(), kv.data_ptr(), page_table.data_ptr(), n_kv_heads,
                              n_heads, head_dim, M, pre_lo, prehi.data_ptr(),
                              tree_mask.data_ptr(), tree_base,
                              n_tree, key_end, scale, out.data_ptr(), ws_ptr, ws_bytes, st)
    if rc:
        raise EagleError(rc, "eagle_op_attention")


def op_lmhead_workspace(M, V, k) -> int:
    L = lib()
    L.eagle_op_lmhead_workspace.argtypes = [i32, i32, i32]
    L.eagle_op_lmhead_workspace.restype = u64
    return int(L.eagle_op_lmhead_workspace(M, V, k))


def _torch_stream():
    import torch
    return torch.cuda.current_stream().cuda_stream
