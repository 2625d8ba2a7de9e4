"""Seeded synthetic inputs shared by the CPU oracle and the GPU harness.

Holds input generation only (weights, prompts, workload shapes); none of the
decoding method's arithmetic lives here. The generator is defined in
``synth.c`` and is bit-reproducible: SplitMix64 counters, an Irwin-Hall(8)
sum of 16-bit lanes, and a single correctly rounded multiply (std 0.02).

Tensor streams: every weight tensor has its own stream id from
:func:`stream_id`, so any tensor (or any slice of one) can be regenerated on
its own, which lets the oracle rebuild a 70B-shaped model layer by layer.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .workloads import WORKLOADS, STATIC_TREE_C2, reduced  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# Tensor kinds. The numbering is the one the C library's tensor table uses
# (enum eagle_tensor_kind in include/eagle.h).
EMBED, LM_HEAD, FINAL_NORM, ATTN_NORM, WQ, WK, WV, WO, FFN_NORM, WGATE, WUP, \
    WDOWN, FC = range(13)
KIND_NAMES = ["embed", "lm_head", "final_norm", "attn_norm", "wq", "wk", "wv",
              "wo", "ffn_norm", "wgate", "wup", "wdown", "fc"]
NORM_KINDS = (FINAL_NORM, ATTN_NORM, FFN_NORM)

# Layer groups of a tensor.
GLOBAL, TARGET, DRAFT = 0, 1, 2

PROMPT_STREAM = 7


def stream_id(kind: int, group: int, layer: int = 0) -> int:
    """Generator stream of one weight tensor (norm gains are constant 1)."""
    if group == GLOBAL:
        return 1 + kind
    if group == DRAFT:
        return 500 + kind
    return 1000 + 16 * layer + kind


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (OpenMP). Returns the path."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        import subprocess
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-ffp-contract=off",
                               "-shared", "-fPIC", "-o", tmp, src])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()   # rebuilds only when synth.c is newer than the library
        lib = ctypes.CDLL(_LIB_PATH)
        u64, p = ctypes.c_uint64, ctypes.c_void_p
        lib.synth_normal_f32.argtypes = [u64, u64, u64, u64, p]
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, u64, p]
        lib.synth_normal_bf16_f32.argtypes = [u64, u64, u64, u64, p]
        lib.synth_tokens.argtypes = [u64, u64, u64, ctypes.c_uint32, p]
        lib.synth_key.argtypes = [u64, u64]
        lib.synth_key.restype = u64
        lib.synth_mix.argtypes = [u64]
        lib.synth_mix.restype = u64
        _lib = lib
    return _lib


def _out(n, dtype, out):
    if out is None:
        return np.empty(n, dtype=dtype)
    assert out.dtype == dtype and out.flags.c_contiguous and out.size == n
    return out.reshape(n)


def normal_f32(seed: int, sid: int, n: int, offset: int = 0, out=None) -> np.ndarray:
    out = _out(n, np.float32, out)
    _load().synth_normal_f32(seed, sid, offset, n, out.ctypes.data)
    return out


def normal_bf16_bits(seed: int, sid: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    _load().synth_normal_bf16(seed, sid, offset, n, out.ctypes.data)
    return out


def normal_bf16_f32(seed: int, sid: int, n: int, offset: int = 0, out=None) -> np.ndarray:
    """The bf16 values of normal_bf16_bits, as float32 (one pass)."""
    out = _out(n, np.float32, out)
    _load().synth_normal_bf16_f32(seed, sid, offset, n, out.ctypes.data)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def tensor_values(seed: int, kind: int, group: int, layer: int, shape,
                  dtype: str, out=None) -> np.ndarray:
    """Values of one weight tensor as float32 (bf16-representable if bf16),
    written into `out` (float32, that shape) when given."""
    n = int(np.prod(shape))
    if kind in NORM_KINDS:
        if out is None:
            return np.ones(shape, dtype=np.float32)
        out[...] = 1.0
        return out
    sid = stream_id(kind, group, layer)
    if dtype == "bf16":
        return normal_bf16_f32(seed, sid, n, out=out).reshape(shape)
    return normal_f32(seed, sid, n, out=out).reshape(shape)


def prompt(seed: int, n: int, vocab: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().synth_tokens(seed, PROMPT_STREAM, n, vocab, out.ctypes.data)
    return out


def mix(x: int) -> int:
    return int(_load().synth_mix(x))


# ---------------------------------------------------------------- device twin
_GPU_LIB_PATH = os.path.join(_HERE, "libsynth_gpu.so")
_gpu_lib = None


def build_gpu(force: bool = False) -> str:
    """Compile libsynth_gpu.so (hipcc, gfx950)."""
    src = os.path.join(_HERE, "synth_gpu.hip")
    if force or not os.path.exists(_GPU_LIB_PATH) or \
            os.path.getmtime(_GPU_LIB_PATH) < os.path.getmtime(src):
        import subprocess
        tmp = _GPU_LIB_PATH + ".tmp"
        subprocess.check_call(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3",
                               "-shared", "-fPIC", "-Xclang", "-target-feature",
                               "-Xclang", "-packed-fp32-ops", "-o", tmp, src])
        os.replace(tmp, _GPU_LIB_PATH)
    return _GPU_LIB_PATH


def _load_gpu():
    global _gpu_lib
    if _gpu_lib is None:
        import torch  # noqa: F401  (binds the HIP runtime torch ships first)
        if not os.path.exists(_GPU_LIB_PATH):
            raise RuntimeError("libsynth_gpu.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_GPU_LIB_PATH)
        u64, p = ctypes.c_uint64, ctypes.c_void_p
        lib.synth_gpu_fill.argtypes = [u64, u64, u64, u64, ctypes.c_int, p, p]
        lib.synth_gpu_fill_const_f32.argtypes = [u64, ctypes.c_float, p, p]
        _gpu_lib = lib
    return _gpu_lib


def gpu_fill(dst_ptr: int, n: int, seed: int, sid: int, dtype: str, stream_ptr: int,
             offset: int = 0) -> None:
    rc = _load_gpu().synth_gpu_fill(seed, sid, offset, n, 1 if dtype == "bf16" else 0,
                                    dst_ptr, stream_ptr)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_fill failed: hipError {rc}")


def gpu_fill_const(dst_ptr: int, n: int, value: float, stream_ptr: int) -> None:
    rc = _load_gpu().synth_gpu_fill_const_f32(n, value, dst_ptr, stream_ptr)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_fill_const_f32 failed: hipError {rc}")


def fill_weights(table, base_ptr: int, seed: int, stream_ptr: int) -> None:
    """Write every tensor of a weight table (list of dicts with kind, group,
    layer, dtype (0 fp32 / 1 bf16), rows, cols, offset) into device memory at
    base_ptr: norm gains are 1, every matrix is its own seeded stream."""
    for t in table:
        n = int(t["rows"]) * int(t["cols"])
        dst = base_ptr + int(t["offset"])
        if t["kind"] in NORM_KINDS:
            gpu_fill_const(dst, n, 1.0, stream_ptr)
        else:
            gpu_fill(dst, n, seed, stream_id(t["kind"], t["group"], t["layer"]),
                     "bf16" if t["dtype"] == 1 else "f32", stream_ptr)
