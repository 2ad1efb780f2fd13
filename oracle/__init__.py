"""Float64 CPU oracle for grouped-query attention at decode time.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  It shares no code with the HIP path and never imports it.

The arithmetic lives in ``gqa_oracle.c`` (plain loops, float64, two-pass
softmax).  This module only builds that file with gcc, loads it with ctypes
and converts inputs to contiguous float64 arrays (bf16 and fp32 values are
exactly representable in float64, so nothing is re-sampled or rounded).

Definition followed ("GQA (Grouped-Query Attention) 분석", section "Grouped
broadcast"; "Same GQA, Different Execution Cost Across Backends", section 1):

    g(h)       = floor(h / (H / G))
    out[b,h,s] = softmax(scale * Q[b,h,s] . K[b,g(h),0..last]^T) . V[b,g(h),0..last]
    last       = min(seq_lens[b], T) - sq + s        (causal among new tokens)

Parity status of every function is pinned by ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgqa_oracle.so")
_lock = threading.Lock()
_lib = None

_dptr = ctypes.POINTER(ctypes.c_double)
_i32ptr = ctypes.POINTER(ctypes.c_int32)


def compile_c(src: str, out_path: str) -> str:
    """gcc -O2 (no fast-math, no FMA contraction) a C source into a .so."""
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=gnu11",
           "-Wall", "-Wextra", "-fPIC", "-shared", "-o", tmp, src,
           "-lpthread", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def build(force: bool = True) -> str:
    """Compile gqa_oracle.c into libgqa_oracle.so next to it."""
    global _lib
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    compile_c(_SRC, _LIB_PATH)
    _lib = None
    return _LIB_PATH


def load_library(path: str):
    """Bind an oracle build at ``path`` (used to run the pins on variants)."""
    return _bind(path)


SOURCE_PATH = _SRC


def _bind(path: str):
    lib = ctypes.CDLL(path)
    lib.gqa_oracle_kv_head.argtypes = [ctypes.c_int] * 3
    lib.gqa_oracle_kv_head.restype = ctypes.c_int
    lib.gqa_oracle_decode_f64.argtypes = [ctypes.c_int] * 6 + [
        _dptr, _dptr, _dptr, _i32ptr, ctypes.c_double, _dptr, _dptr,
        ctypes.c_int]
    lib.gqa_oracle_decode_f64.restype = ctypes.c_int
    lib.gqa_oracle_decode_row_f64.argtypes = [ctypes.c_int] * 5 + [
        _dptr, _dptr, _dptr, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_double, _dptr]
    lib.gqa_oracle_decode_row_f64.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or \
                    os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build(force=True)
            _lib = _bind(_LIB_PATH)
    return _lib


def _f64(x) -> np.ndarray:
    """Any CPU tensor/array -> contiguous float64 numpy (exact for bf16/fp32)."""
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach()
        if x.device.type != "cpu":
            raise ValueError("oracle inputs must be CPU tensors")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def kv_head(h: int, H: int, G: int, lib=None) -> int:
    """KV head read by query head h: floor(h / (H/G))."""
    return int((lib or _load()).gqa_oracle_kv_head(int(h), int(H), int(G)))


def decode_f64(q, k, v, seq_lens=None, scale=None, threads: int = 1,
               return_probs: bool = False, lib=None):
    """Full oracle.  q: [B,H,sq,D]; k, v: [B,G,T,D]; seq_lens: [B] or None.

    Returns out [B,H,sq,D] float64 (and probs [B,H,sq,T] if asked).
    """
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    if qd.ndim != 4 or kd.ndim != 4 or vd.shape != kd.shape:
        raise ValueError("expected q[B,H,sq,D], k/v[B,G,T,D]")
    B, H, sq, D = qd.shape
    Bk, G, T, Dk = kd.shape
    if Bk != B or Dk != D:
        raise ValueError("q and k/v shapes disagree")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, H, sq, D), dtype=np.float64)
    probs = np.zeros((B, H, sq, T), dtype=np.float64) if return_probs else None
    sl = None
    if seq_lens is not None:
        sl = _i32(seq_lens)
        if sl.shape != (B,):
            raise ValueError("seq_lens must be [B]")
    lib = lib or _load()
    rc = lib.gqa_oracle_decode_f64(
        B, H, G, sq, T, D,
        qd.ctypes.data_as(_dptr), kd.ctypes.data_as(_dptr), vd.ctypes.data_as(_dptr),
        sl.ctypes.data_as(_i32ptr) if sl is not None else None,
        float(scale), out.ctypes.data_as(_dptr),
        probs.ctypes.data_as(_dptr) if probs is not None else None,
        int(threads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (H % G != 0 or bad sizes)")
    return (out, probs) if return_probs else out


def decode_row_f64(q_row, k_b, v_b, H: int, sq: int, h: int, s: int,
                   seq_len_b: int, scale: float, lib=None):
    """One output row for query head h, new-token index s of one sequence.

    q_row: [D]; k_b, v_b: that sequence's [G,T,D] cache.  Returns [D] float64.
    """
    qd, kd, vd = _f64(q_row), _f64(k_b), _f64(v_b)
    G, T, D = kd.shape
    out = np.zeros(D, dtype=np.float64)
    rc = (lib or _load()).gqa_oracle_decode_row_f64(
        int(H), int(G), int(sq), int(T), int(D),
        qd.ctypes.data_as(_dptr), kd.ctypes.data_as(_dptr), vd.ctypes.data_as(_dptr),
        int(h), int(s), int(seq_len_b), float(scale), out.ctypes.data_as(_dptr))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out
