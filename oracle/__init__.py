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


# ---------------------------------------------------------------------------
# Cache variants.  Both are the plain definition applied to the cache they
# describe: the rows are put where the variant says, with numpy indexing, and
# the float64 oracle above runs on the result.
# ---------------------------------------------------------------------------
def append_rows(k_new, v_new, k_cache, v_cache, seq_lens=None):
    """The caches after storing the sq new tokens of every (b, g): token s goes
    to row L_b - sq + s (L_b = min(seq_lens[b], T), which counts the new
    tokens); a token whose row would be negative is dropped.  Appending to the
    cache before attending is the incremental decode loop of "GQA
    (Grouped-Query Attention) 분석", section "동작 원리", items 2 and 3.
    Returns new float64 arrays; the inputs are not modified."""
    kn, vn = _f64(k_new), _f64(v_new)
    kc, vc = _f64(k_cache).copy(), _f64(v_cache).copy()
    B, G, T, D = kc.shape
    sq = kn.shape[2]
    if kn.shape != (B, G, sq, D) or vn.shape != kn.shape or vc.shape != kc.shape:
        raise ValueError("expected k_new/v_new [B,G,sq,D] and caches [B,G,T,D]")
    lens = [T] * B if seq_lens is None else [min(max(int(x), 0), T) for x in _i32(seq_lens)]
    for b in range(B):
        for s in range(sq):
            row = lens[b] - sq + s
            if row >= 0:
                kc[b, :, row, :] = kn[b, :, s, :]
                vc[b, :, row, :] = vn[b, :, s, :]
    return kc, vc


def decode_append_f64(q, k_new, v_new, k_cache, v_cache, seq_lens=None, scale=None,
                      threads: int = 1):
    """Append (see append_rows), then decode.  Returns (out, k_after, v_after)."""
    kc, vc = append_rows(k_new, v_new, k_cache, v_cache, seq_lens)
    return decode_f64(q, kc, vc, seq_lens, scale, threads=threads), kc, vc


def gather_pages(pages, block_table, seq_lens=None):
    """The contiguous [B, G, T, D] cache a paged one describes: row t of
    sequence b is row t % page_size of page block_table[b, t // page_size]
    of pages [num_pages, G, page_size, D]; T = page_size * max_pages.  Only
    the pages that hold rows below L_b are looked up; the other rows are NaN
    (the definition never reads them)."""
    pg = _f64(pages)
    bt = _i32(block_table).astype(np.int64)
    num_pages, G, ps, D = pg.shape
    B, max_pages = bt.shape
    T = ps * max_pages
    lens = [T] * B if seq_lens is None else [min(max(int(x), 0), T) for x in _i32(seq_lens)]
    out = np.full((B, G, T, D), np.nan, dtype=np.float64)
    for b in range(B):
        for i in range((lens[b] + ps - 1) // ps):
            p = int(bt[b, i])
            if not 0 <= p < num_pages:
                raise ValueError("block_table[%d, %d] = %d is not a page" % (b, i, p))
            out[b, :, i * ps:(i + 1) * ps, :] = pg[p]
    return out


def decode_paged_f64(q, k_pages, v_pages, block_table, seq_lens=None, scale=None,
                     threads: int = 1):
    """Decode over a paged cache: gather_pages, then the oracle."""
    k = gather_pages(k_pages, block_table, seq_lens)
    v = gather_pages(v_pages, block_table, seq_lens)
    return decode_f64(q, k, v, seq_lens, scale, threads=threads)


# ---------------------------------------------------------------------------
# Quantized cache: fp8 E4M3 codes with one scale per KV head.  The pages
# name KV quantization only as a change of element precision that composes
# with GQA ("GQA (Grouped-Query Attention) 분석", section "장단점"); the
# format read here is the OCP FP8 E4M3 ("E4M3FN") code -- sign bit, 4
# exponent bits with bias 7, 3 mantissa bits, subnormals, no infinities,
# S.1111.111 = NaN -- and the cache value is decode(code) * scale[g].
# ---------------------------------------------------------------------------
def fp8_e4m3_value(code: int) -> float:
    """The real number an E4M3 code stands for (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)          # subnormal: 0.m * 2^-6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_FP8_TABLE = np.array([fp8_e4m3_value(c) for c in range(256)], dtype=np.float64)


def dequant_fp8(codes, scale) -> np.ndarray:
    """codes [B, G, T, D] (uint8), scale [G] -> float64 cache values."""
    c = np.asarray(codes.cpu().numpy() if hasattr(codes, "cpu") else codes).astype(np.int64)
    sc = _f64(scale)
    if c.ndim != 4 or sc.shape != (c.shape[1],):
        raise ValueError("expected codes [B,G,T,D] and scale [G]")
    return _FP8_TABLE[c] * sc[None, :, None, None]


def decode_fp8_f64(q, k_codes, v_codes, k_scale, v_scale, seq_lens=None, scale=None,
                   threads: int = 1):
    """Decode over an fp8 cache: dequantize every code (dequant_fp8), then
    the float64 oracle."""
    return decode_f64(q, dequant_fp8(k_codes, k_scale), dequant_fp8(v_codes, v_scale), seq_lens,
                      scale, threads=threads)


def dequant_int8(codes, scale) -> np.ndarray:
    """codes [B, G, T, D] (int8, two's complement), scale [G] -> float64
    cache values code * scale[g] (an int8 cache with one scale per KV head;
    the pages name KV quantization as composable with GQA -- "GQA
    (Grouped-Query Attention) 분석", section "장단점" -- without a format)."""
    c = np.asarray(codes.cpu().numpy() if hasattr(codes, "cpu") else codes)
    if c.dtype != np.int8:
        raise ValueError("int8 codes expected")
    sc = _f64(scale)
    if c.ndim != 4 or sc.shape != (c.shape[1],):
        raise ValueError("expected codes [B,G,T,D] and scale [G]")
    return c.astype(np.float64) * sc[None, :, None, None]


def decode_int8_f64(q, k_codes, v_codes, k_scale, v_scale, seq_lens=None, scale=None,
                    threads: int = 1):
    """Decode over an int8 cache: dequantize every code (dequant_int8), then
    the float64 oracle."""
    return decode_f64(q, dequant_int8(k_codes, k_scale), dequant_int8(v_codes, v_scale), seq_lens,
                      scale, threads=threads)
