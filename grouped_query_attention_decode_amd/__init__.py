"""Python binding of libgqa: grouped-query attention at decode time on MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libgqa.so`` (built by ``grouped_query_attention_decode_amd.build``);
torch supplies device memory and the current stream.  If the library is
missing or fails to load, every call raises -- there is no fallback.

    out = decode(q, k_cache, v_cache, seq_lens=None, scale=None, out=None)

q [B,H,sq,D], k_cache / v_cache [B,G,T,D] (contiguous, on one GPU, all
float32, all bfloat16 or all float16), seq_lens [B] int32 on the same GPU or None,
out [B,H,sq,D] float32.  Query head h reads KV head h // (H/G)
("GQA (Grouped-Query Attention) 분석", section "Grouped broadcast").

    out = decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens)   # bf16
    out = decode_paged(q, k_pages, v_pages, block_table, seq_lens)     # bf16

decode_append stores the sq new tokens' K/V (k_new / v_new [B,G,sq,D]) at
cache rows L-sq .. L-1 and attends in the same pass; decode_paged reads a
page pool [num_pages, G, page_size, D] through block_table [B, max_pages].
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

__all__ = ["decode", "decode_append", "decode_paged", "decode_fp8", "decode_int8", "plan", "workspace_bytes",
           "paged_workspace_bytes", "append_workspace_bytes", "decode_noalloc", "workspace_clear",
           "version", "library_path",
           "load_library", "GqaError", "PATH_AUTO", "PATH_VALU", "PATH_MFMA", "PATH_MFMA_QK",
           "MERGE_AUTO", "MERGE_IN_KERNEL", "MERGE_COMBINE",
           "EXPORTED_SYMBOLS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgqa.so")

GQA_OK, GQA_ERR_INVALID_ARG, GQA_ERR_UNSUPPORTED, GQA_ERR_ALLOC, GQA_ERR_HIP = range(5)
GQA_F32, GQA_BF16, GQA_FP8_E4M3, GQA_F16, GQA_INT8 = 0, 1, 2, 3, 4
PATH_AUTO, PATH_VALU, PATH_MFMA, PATH_MFMA_QK = 0, 1, 2, 3
MERGE_AUTO, MERGE_IN_KERNEL, MERGE_COMBINE = 0, 1, 2

# Every symbol include/gqa.h declares.
EXPORTED_SYMBOLS = ("gqa_decode", "gqa_workspace_bytes", "gqa_append_workspace_bytes", "gqa_decode_ws",
                    "gqa_workspace_clear", "gqa_decode_noalloc",
                    "gqa_decode_ex", "gqa_decode_fp8", "gqa_decode_int8", "gqa_decode_append",
                    "gqa_paged_workspace_bytes",
                    "gqa_decode_paged", "gqa_plan", "gqa_last_error", "gqa_version")


class GqaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("libgqa status %d: %s" % (status, message))
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("G", ctypes.c_int32),
                ("sq", ctypes.c_int32), ("T", ctypes.c_int32), ("D", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32)]


class PagedShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("G", ctypes.c_int32),
                ("sq", ctypes.c_int32), ("D", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32)]


class Options(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("workgroups", ctypes.c_int32),
                ("merge", ctypes.c_int32), ("reserved", ctypes.c_int32 * 5)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("workgroups", ctypes.c_int32),
                ("rows_per_group", ctypes.c_int32), ("row_blocks", ctypes.c_int32),
                ("row_block", ctypes.c_int32), ("combine", ctypes.c_int32),
                ("waves_per_group", ctypes.c_int32), ("reserved", ctypes.c_int32 * 1),
                ("workspace_bytes", ctypes.c_uint64)]


_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Load libgqa.so (after torch, so that both share one HIP runtime)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libgqa.so is not built (%s); run "
                "`python -m grouped_query_attention_decode_amd.build` "
                "or __graft_entry__.build()" % LIB_PATH)
        import torch  # noqa: F401  (loads torch's HIP runtime first)
        lib = ctypes.CDLL(LIB_PATH)
        vp, sp = ctypes.c_void_p, ctypes.POINTER(Shape)
        i32p = ctypes.c_void_p
        lib.gqa_decode.argtypes = [sp, vp, vp, vp, i32p, ctypes.c_float, vp, vp]
        lib.gqa_decode.restype = ctypes.c_int
        lib.gqa_workspace_bytes.argtypes = [sp]
        lib.gqa_workspace_bytes.restype = ctypes.c_size_t
        lib.gqa_append_workspace_bytes.argtypes = [sp]
        lib.gqa_append_workspace_bytes.restype = ctypes.c_size_t
        lib.gqa_decode_ws.argtypes = [sp, vp, vp, vp, i32p, ctypes.c_float, vp, vp,
                                      ctypes.c_size_t, vp]
        lib.gqa_decode_ws.restype = ctypes.c_int
        lib.gqa_workspace_clear.argtypes = [vp, ctypes.c_size_t, vp]
        lib.gqa_workspace_clear.restype = ctypes.c_int
        lib.gqa_decode_ex.argtypes = [sp, vp, vp, vp, i32p, ctypes.c_float, vp, vp,
                                      ctypes.c_size_t, ctypes.POINTER(Options), vp]
        lib.gqa_decode_ex.restype = ctypes.c_int
        lib.gqa_decode_noalloc.argtypes = [sp, vp, vp, vp, i32p, ctypes.c_float, vp,
                                           ctypes.POINTER(Options), vp]
        lib.gqa_decode_noalloc.restype = ctypes.c_int
        lib.gqa_decode_fp8.argtypes = [sp, vp, vp, vp, vp, vp, i32p, ctypes.c_float, vp, vp,
                                       ctypes.c_size_t, ctypes.POINTER(Options), vp]
        lib.gqa_decode_fp8.restype = ctypes.c_int
        lib.gqa_decode_int8.argtypes = lib.gqa_decode_fp8.argtypes
        lib.gqa_decode_int8.restype = ctypes.c_int
        lib.gqa_decode_append.argtypes = [sp, vp, vp, vp, vp, vp, i32p, ctypes.c_float, vp, vp,
                                          ctypes.c_size_t, ctypes.POINTER(Options), vp]
        lib.gqa_decode_append.restype = ctypes.c_int
        psp = ctypes.POINTER(PagedShape)
        lib.gqa_paged_workspace_bytes.argtypes = [psp]
        lib.gqa_paged_workspace_bytes.restype = ctypes.c_size_t
        lib.gqa_decode_paged.argtypes = [psp, vp, vp, vp, i32p, i32p, ctypes.c_float, vp, vp,
                                         ctypes.c_size_t, ctypes.POINTER(Options), vp]
        lib.gqa_decode_paged.restype = ctypes.c_int
        lib.gqa_plan.argtypes = [sp, ctypes.POINTER(Options), ctypes.POINTER(PlanInfo)]
        lib.gqa_plan.restype = ctypes.c_int
        lib.gqa_last_error.argtypes = []
        lib.gqa_last_error.restype = ctypes.c_char_p
        lib.gqa_version.argtypes = []
        lib.gqa_version.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _check(status: int):
    if status != GQA_OK:
        msg = load_library().gqa_last_error().decode(errors="replace")
        raise GqaError(status, msg)


def _dtype_code(dt) -> int:
    import torch
    if dt == torch.float32:
        return GQA_F32
    if dt == torch.bfloat16:
        return GQA_BF16
    if dt == torch.float16:
        return GQA_F16
    if dt == torch.int8:
        return GQA_INT8
    if dt in (torch.uint8, torch.float8_e4m3fn):
        return GQA_FP8_E4M3
    return 99  # rejected by the library as unsupported


def make_shape(B, H, G, sq, T, D, q_dtype=GQA_BF16, kv_dtype=GQA_BF16, out_dtype=GQA_F32):
    return Shape(B, H, G, sq, T, D, q_dtype, kv_dtype, out_dtype)


def _options(path=PATH_AUTO, workgroups=0, merge=0):
    o = Options()
    o.path = int(path)
    o.workgroups = int(workgroups)
    o.merge = int(merge)
    return o


def plan(shape: Shape, path=PATH_AUTO, workgroups=0, merge=0) -> dict:
    """The planner's launch decisions for ``shape`` (host only)."""
    lib = load_library()
    info = PlanInfo()
    opts = _options(path, workgroups, merge)
    _check(lib.gqa_plan(ctypes.byref(shape), ctypes.byref(opts), ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in PlanInfo._fields_ if name != "reserved"}


def workspace_bytes(shape: Shape) -> int:
    return int(load_library().gqa_workspace_bytes(ctypes.byref(shape)))


def workspace_clear(workspace, stream=None):
    """Zero the arrival counters of a caller workspace (a uint8 GPU tensor)
    on ``stream`` (default: torch's current stream): before its first use,
    or after queued work on it did not complete."""
    import torch
    if not workspace.is_cuda:
        raise ValueError("workspace must be a GPU tensor")
    if stream is None:
        stream = torch.cuda.current_stream(workspace.device)
    with torch.cuda.device(workspace.device):
        _check(load_library().gqa_workspace_clear(
            workspace.data_ptr(), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
            ctypes.c_void_p(stream.cuda_stream)))


def append_workspace_bytes(shape: Shape) -> int:
    """Device scratch bytes gqa_decode_append needs for ``shape``."""
    return int(load_library().gqa_append_workspace_bytes(ctypes.byref(shape)))


def version() -> str:
    return load_library().gqa_version().decode()


def shape_of(q, k_cache, out_dtype=None) -> Shape:
    B, H, sq, D = q.shape
    _, G, T, _ = k_cache.shape
    import torch
    return make_shape(B, H, G, sq, T, D, _dtype_code(q.dtype), _dtype_code(k_cache.dtype),
                      _dtype_code(out_dtype or torch.float32))


def decode(q, k_cache, v_cache, seq_lens=None, scale=None, out=None, *,
           path=PATH_AUTO, workgroups=0, merge=0, workspace=None, stream=None):
    """Grouped-query attention for one decode step (see module docstring).

    Runs asynchronously on ``stream`` (default: torch's current stream).
    ``workspace``: optional uint8 GPU tensor of at least
    ``workspace_bytes(shape_of(q, k_cache))`` bytes, zero-filled before its
    first use (each call leaves it zeroed); default: library-owned.
    ``workgroups``: kernel grid size (0 = the planner's choice).
    ``merge``: MERGE_AUTO, MERGE_IN_KERNEL or MERGE_COMBINE (matrix-core path).
    """
    import torch
    lib = load_library()
    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,H,sq,D] and k_cache/v_cache [B,G,T,D]")
    if q.shape[0] != k_cache.shape[0] or q.shape[3] != k_cache.shape[3]:
        raise ValueError("q and the caches disagree on B or D")
    if v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must share a dtype")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    dev = q.device
    if k_cache.device != dev or v_cache.device != dev:
        raise ValueError("all tensors must be on one device")
    if seq_lens is not None:
        if seq_lens.dtype != torch.int32 or seq_lens.device != dev or \
                seq_lens.shape != (q.shape[0],) or not seq_lens.is_contiguous():
            raise ValueError("seq_lens must be a contiguous int32 [B] tensor on q's device")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    else:
        if out.shape != q.shape or out.device != dev or not out.is_contiguous():
            raise ValueError("out must be a contiguous [B,H,sq,D] tensor on q's device")
    D = q.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    shape = shape_of(q, k_cache, out.dtype)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    opts = _options(path, workgroups, merge)
    ws_ptr, ws_len = None, 0
    if workspace is not None:
        if not workspace.is_cuda or workspace.device != dev:
            raise ValueError("workspace must be on q's device")
        ws_ptr, ws_len = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        st = lib.gqa_decode_ex(
            ctypes.byref(shape), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            seq_lens.data_ptr() if seq_lens is not None else None,
            ctypes.c_float(scale), out.data_ptr(), ws_ptr, ctypes.c_size_t(ws_len),
            ctypes.byref(opts), sptr)
    _check(st)
    return out


def decode_noalloc(q, k_cache, v_cache, seq_lens=None, scale=None, out=None, *,
                   path=PATH_AUTO, workgroups=0, merge=0, stream=None):
    """As ``decode``, through gqa_decode_noalloc: no device memory is
    allocated (``out`` must then be given); the library's fixed 64 MiB
    scratch serves as workspace, so calls that overlap on one device race."""
    import torch
    lib = load_library()
    if out is None:
        raise ValueError("decode_noalloc allocates nothing: pass out")
    out = _common_checks(q, (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)), seq_lens, out)
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must share a shape and dtype")
    dev = q.device
    scale = 1.0 / math.sqrt(q.shape[3]) if scale is None else scale
    shape = shape_of(q, k_cache, out.dtype)
    stream = torch.cuda.current_stream(dev) if stream is None else stream
    opts = _options(path, workgroups, merge)
    with torch.cuda.device(dev):
        st = lib.gqa_decode_noalloc(
            ctypes.byref(shape), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            seq_lens.data_ptr() if seq_lens is not None else None, ctypes.c_float(scale),
            out.data_ptr(), ctypes.byref(opts), ctypes.c_void_p(stream.cuda_stream))
    _check(st)
    return out


def _common_checks(q, tensors, seq_lens, out):
    import torch
    dev = q.device
    for name, t in tensors:
        if not t.is_cuda or t.device != dev:
            raise ValueError("%s must be a GPU tensor on q's device" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if seq_lens is not None:
        if seq_lens.dtype != torch.int32 or seq_lens.device != dev or \
                seq_lens.shape != (q.shape[0],) or not seq_lens.is_contiguous():
            raise ValueError("seq_lens must be a contiguous int32 [B] tensor on q's device")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    elif out.shape != q.shape or out.device != dev or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B,H,sq,D] tensor on q's device")
    return out


def _ws(workspace, dev):
    if workspace is None:
        return None, 0
    if not workspace.is_cuda or workspace.device != dev:
        raise ValueError("workspace must be on q's device")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens=None, scale=None, out=None, *,
                  path=PATH_AUTO, workgroups=0, merge=0, workspace=None, stream=None):
    """Store the new tokens' K/V (k_new / v_new [B,G,sq,D]) at cache rows
    L-sq .. L-1 (L = seq_lens[b], which counts them) and return the decode
    attention over rows 0 .. L-1 -- one pass (bf16)."""
    import torch
    lib = load_library()
    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,H,sq,D] and k_cache/v_cache [B,G,T,D]")
    B, H, sq, D = q.shape
    G = k_cache.shape[1]
    if k_new.shape != (B, G, sq, D) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [B,G,sq,D]")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_new, v_new and the caches must share a dtype")
    out = _common_checks(q, (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                             ("v_cache", v_cache)), seq_lens, out)
    dev = q.device
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    shape = shape_of(q, k_cache, out.dtype)
    stream = torch.cuda.current_stream(dev) if stream is None else stream
    ws_ptr, ws_len = _ws(workspace, dev)
    opts = _options(path, workgroups, merge)
    with torch.cuda.device(dev):
        st = lib.gqa_decode_append(
            ctypes.byref(shape), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
            k_cache.data_ptr(), v_cache.data_ptr(),
            seq_lens.data_ptr() if seq_lens is not None else None, ctypes.c_float(scale),
            out.data_ptr(), ws_ptr, ctypes.c_size_t(ws_len), ctypes.byref(opts),
            ctypes.c_void_p(stream.cuda_stream))
    _check(st)
    return out


def paged_shape_of(q, k_pages, block_table, out_dtype=None) -> PagedShape:
    import torch
    B, H, sq, D = q.shape
    num_pages, G, page_size, Dk = k_pages.shape
    if Dk != D or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("expected k_pages [num_pages,G,page_size,D] and block_table [B,max_pages]")
    return PagedShape(B, H, G, sq, D, page_size, num_pages, block_table.shape[1],
                      _dtype_code(q.dtype), _dtype_code(k_pages.dtype),
                      _dtype_code(out_dtype or torch.float32))


def paged_workspace_bytes(shape: PagedShape) -> int:
    return int(load_library().gqa_paged_workspace_bytes(ctypes.byref(shape)))


def decode_paged(q, k_pages, v_pages, block_table, seq_lens=None, scale=None, out=None, *,
                 path=PATH_AUTO, workgroups=0, merge=0, workspace=None, stream=None):
    """Decode attention over a paged cache: k_pages / v_pages
    [num_pages, G, page_size, D], block_table [B, max_pages] int32 (row t of
    sequence b is row t % page_size of page block_table[b, t // page_size]).
    Pages of bf16 or fp16, or of 8-bit codes (uint8 / float8_e4m3fn for E4M3,
    int8) read with unit scales: fold one K scale into ``scale`` and multiply
    the output by one V scale."""
    import torch
    lib = load_library()
    if q.dim() != 4 or k_pages.dim() != 4 or v_pages.shape != k_pages.shape:
        raise ValueError("expected q [B,H,sq,D] and k_pages/v_pages [num_pages,G,page_size,D]")
    if v_pages.dtype != k_pages.dtype:
        raise ValueError("k_pages and v_pages must share a dtype")
    if block_table.dtype != torch.int32:
        raise ValueError("block_table must be int32")
    out = _common_checks(q, (("q", q), ("k_pages", k_pages), ("v_pages", v_pages),
                             ("block_table", block_table)), seq_lens, out)
    dev = q.device
    scale = 1.0 / math.sqrt(q.shape[3]) if scale is None else scale
    shape = paged_shape_of(q, k_pages, block_table, out.dtype)
    stream = torch.cuda.current_stream(dev) if stream is None else stream
    ws_ptr, ws_len = _ws(workspace, dev)
    opts = _options(path, workgroups, merge)
    with torch.cuda.device(dev):
        st = lib.gqa_decode_paged(
            ctypes.byref(shape), q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
            block_table.data_ptr(), seq_lens.data_ptr() if seq_lens is not None else None,
            ctypes.c_float(scale), out.data_ptr(), ws_ptr, ctypes.c_size_t(ws_len),
            ctypes.byref(opts), ctypes.c_void_p(stream.cuda_stream))
    _check(st)
    return out


def decode_fp8(q, k_codes, v_codes, k_scale=None, v_scale=None, seq_lens=None, scale=None, out=None,
               *, workgroups=0, merge=0, workspace=None, stream=None):
    """Decode over an fp8 E4M3 cache: k_codes / v_codes [B,G,T,D] uint8 (or
    torch.float8_e4m3fn), k_scale / v_scale [G] float32 on the GPU or None
    (1.0); the value of code c in KV head g is e4m3(c) * scale[g]."""
    return _decode_codes("gqa_decode_fp8", q, k_codes, v_codes, k_scale, v_scale, seq_lens, scale, out,
                         workgroups, merge, workspace, stream)


def decode_int8(q, k_codes, v_codes, k_scale=None, v_scale=None, seq_lens=None, scale=None, out=None,
                *, workgroups=0, merge=0, workspace=None, stream=None):
    """Decode over an int8 cache: k_codes / v_codes [B,G,T,D] torch.int8,
    k_scale / v_scale [G] float32 on the GPU or None (1.0); the value of code
    c in KV head g is c * scale[g]."""
    return _decode_codes("gqa_decode_int8", q, k_codes, v_codes, k_scale, v_scale, seq_lens, scale, out,
                         workgroups, merge, workspace, stream)


def _decode_codes(entry, q, k_codes, v_codes, k_scale, v_scale, seq_lens, scale, out, workgroups, merge,
                  workspace, stream):
    import torch
    lib = load_library()
    if q.dim() != 4 or k_codes.dim() != 4 or v_codes.shape != k_codes.shape:
        raise ValueError("expected q [B,H,sq,D] and k_codes/v_codes [B,G,T,D]")
    if k_codes.element_size() != 1 or v_codes.element_size() != 1:
        raise ValueError("k_codes / v_codes must hold one byte per element")
    G = k_codes.shape[1]
    ts = [("q", q), ("k_codes", k_codes), ("v_codes", v_codes)]
    for name, sc in (("k_scale", k_scale), ("v_scale", v_scale)):
        if sc is not None:
            if sc.dtype != torch.float32 or sc.shape != (G,):
                raise ValueError("%s must be a float32 [G] tensor" % name)
            ts.append((name, sc))
    out = _common_checks(q, ts, seq_lens, out)
    dev = q.device
    scale = 1.0 / math.sqrt(q.shape[3]) if scale is None else scale
    shape = shape_of(q, k_codes, out.dtype)
    stream = torch.cuda.current_stream(dev) if stream is None else stream
    ws_ptr, ws_len = _ws(workspace, dev)
    opts = _options(PATH_AUTO, workgroups, merge)
    with torch.cuda.device(dev):
        st = getattr(lib, entry)(
            ctypes.byref(shape), q.data_ptr(), k_codes.data_ptr(), v_codes.data_ptr(),
            k_scale.data_ptr() if k_scale is not None else None,
            v_scale.data_ptr() if v_scale is not None else None,
            seq_lens.data_ptr() if seq_lens is not None else None, ctypes.c_float(scale),
            out.data_ptr(), ws_ptr, ctypes.c_size_t(ws_len), ctypes.byref(opts),
            ctypes.c_void_p(stream.cuda_stream))
    _check(st)
    return out
