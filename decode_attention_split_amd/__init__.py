"""Thin Python binding of libdas.so (split-KV decode attention for MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/das.h``.  PyTorch supplies
device memory and the current HIP stream.  The functions carry the C names.

If ``libdas.so`` has not been built, every call raises: there is no CPU
fallback.

Streams: every call launches on ``stream`` (default: torch's current
stream).  Tensors a call allocates itself (workspace, out, lse) are created
on that stream; inputs and caller-supplied outputs must be ready on it (the
caller orders them, as with any torch work on a side stream).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdas.so")
# The debug build: the same library with every LDS buffer filled with NaN
# bytes when it stops being live (a read that races its write then returns
# NaN instead of stale values).  Tests only; nothing here loads it by itself.
DEBUG_LIB_PATH = os.path.join(_HERE, "libdas_debug.so")

DAS_OK, DAS_EINVAL, DAS_ENOTSUP, DAS_EWORKSPACE, DAS_ELAUNCH = 0, -1, -2, -3, -4
DAS_F32, DAS_BF16, DAS_E4M3, DAS_INT4 = 0, 1, 2, 3
DAS_PAGED_HND, DAS_PAGED_NHD = 0, 1
DAS_MAX_SPLITS = 4096
DAS_CHUNK_QUANTUM = 128
DAS_WORKSPACE_COUNTER_BYTES = 65536 * 4

EXPORTED = ("das_plan", "das_plan_kv", "das_decode_workspace_bytes", "das_decode_attention",
            "das_split_kv_decode", "das_decode_attention_fp8", "das_split_kv_decode_fp8",
            "das_decode_attention_int4", "das_split_kv_decode_int4", "das_decode_attention_paged",
            "das_lse_combine", "das_merge_attn_states", "das_decode_attention_noalloc",
            "das_strerror")
DAS_NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


class DasError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {das_strerror(status)} (status {status})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdas.so and declare the C signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = open_library(path)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """Load a build of the library at ``path`` (libdas.so, or the debug
    build libdas_debug.so) with the C signatures declared, without making it
    the one the entry points below call.  Raises if it is missing."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950) first")
    lib = ctypes.CDLL(path)
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pi32 = ctypes.POINTER(ctypes.c_int32)
    lib.das_plan.argtypes = [i32, i32, i32, i32, i32, i32, i32, pi32, pi32]
    lib.das_plan.restype = ctypes.c_int
    lib.das_plan_kv.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, pi32, pi32]
    lib.das_plan_kv.restype = ctypes.c_int
    lib.das_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.das_decode_workspace_bytes.restype = sz
    decode_args = [p, p, p, p, i32, i32, i32, i32, i32, ctypes.c_float, p, i32, p, i32, p, sz, p]
    for name in ("das_decode_attention", "das_split_kv_decode"):
        getattr(lib, name).argtypes = decode_args
        getattr(lib, name).restype = ctypes.c_int
    fp8_args = [p, p, p, p, p, p, i32, i32, i32, i32, i32, ctypes.c_float, p, i32, p, i32, p, sz, p]
    for name in ("das_decode_attention_fp8", "das_split_kv_decode_fp8",
                 "das_decode_attention_int4", "das_split_kv_decode_int4"):
        getattr(lib, name).argtypes = fp8_args
        getattr(lib, name).restype = ctypes.c_int
    lib.das_decode_attention_paged.argtypes = [p, p, p, i32, p, p, p, i32, i32, i32, i32, p, i32,
                                               i32, i32, i32, ctypes.c_float, p, i32, p, i32, p,
                                               sz, p]
    lib.das_decode_attention_paged.restype = ctypes.c_int
    lib.das_decode_attention_noalloc.argtypes = [p, p, p, p, i32, i32, i32, i32, i32,
                                                 ctypes.c_float, p, i32, p, i32, p]
    lib.das_decode_attention_noalloc.restype = ctypes.c_int
    lib.das_lse_combine.argtypes = [p, i32, i32, i32, i32, i32, i32, p, sz, p, i32, p, p]
    lib.das_lse_combine.restype = ctypes.c_int
    lib.das_merge_attn_states.argtypes = [p, p, p, p, p, p, i64, i32, i32, p]
    lib.das_merge_attn_states.restype = ctypes.c_int
    lib.das_strerror.argtypes = [ctypes.c_int]
    lib.das_strerror.restype = ctypes.c_char_p
    return lib


def das_strerror(status: int) -> str:
    return load_library().das_strerror(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != DAS_OK:
        raise DasError(status, where)


def das_plan(B: int, Hkv: int, G: int, Smax: int, D: int, num_splits: int = 0,
             num_cus: int = 0) -> Tuple[int, int]:
    """(number of splits, rows per split) the library will use."""
    ns, chunk = ctypes.c_int32(), ctypes.c_int32()
    _check(load_library().das_plan(B, Hkv, G, Smax, D, num_splits, num_cus,
                                   ctypes.byref(ns), ctypes.byref(chunk)), "das_plan")
    return ns.value, chunk.value


def das_plan_kv(kv_dtype: int, B: int, Hkv: int, G: int, Smax: int, D: int, num_splits: int = 0,
                num_cus: int = 0) -> Tuple[int, int]:
    """(number of splits, rows per split) of the one-call entry point for a
    K/V cache of kv_dtype (DAS_BF16, DAS_E4M3 or DAS_INT4)."""
    ns, chunk = ctypes.c_int32(), ctypes.c_int32()
    _check(load_library().das_plan_kv(kv_dtype, B, Hkv, G, Smax, D, num_splits, num_cus,
                                      ctypes.byref(ns), ctypes.byref(chunk)), "das_plan_kv")
    return ns.value, chunk.value


def das_decode_workspace_bytes(B: int, Hq: int, Hkv: int, Smax: int, D: int,
                               num_splits: int = 0, num_cus: int = 0) -> int:
    n = load_library().das_decode_workspace_bytes(B, Hq, Hkv, Smax, D, num_splits, num_cus)
    if n == ctypes.c_size_t(-1).value:
        raise DasError(DAS_EINVAL, "das_decode_workspace_bytes")
    return int(n)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Context in which the tensors a call allocates itself (workspace, out,
    lse) are created: on the stream the kernels run on, so that their
    zero-fill is ordered before the launch and the caching allocator reuses
    their memory only behind work on that stream."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _decode_shapes(q, k_cache, v_cache, seq_lens, kv_format: int = DAS_BF16):
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seq_lens", seq_lens)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    kv_dtypes = {DAS_BF16: (torch.bfloat16,), DAS_E4M3: (torch.uint8, torch.float8_e4m3fn),
                 DAS_INT4: (torch.uint8,)}[kv_format]
    if q.dtype != torch.bfloat16 or k_cache.dtype not in kv_dtypes or v_cache.dtype not in kv_dtypes:
        raise ValueError("q must be bfloat16; k_cache and v_cache bfloat16, E4M3 codes "
                         "(uint8 or float8_e4m3fn) for the fp8 entry points, or packed INT4 "
                         "codes (uint8) for the int4 entry points")
    if seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32")
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B,Hq,D]; k_cache, v_cache must be [B,Hkv,Smax,D] "
                         "([B,Hkv,Smax,D/2] bytes for INT4)")
    B, Hq, D = q.shape
    _, Hkv, Smax, _ = k_cache.shape
    row = D // 2 if kv_format == DAS_INT4 else D
    if k_cache.shape[0] != B or k_cache.shape[3] != row or seq_lens.shape != (B,):
        raise ValueError("shape mismatch between q, caches and seq_lens")
    return B, Hq, Hkv, Smax, D


def _outputs(q, B, Hq, D, out, lse_out, out_dtype, with_lse):
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    if out.dtype not in (torch.float32, torch.bfloat16) or out.shape != (B, Hq, D) \
            or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous float32 or bfloat16 [B,Hq,D] tensor on q's device")
    if lse_out is None and with_lse:
        lse_out = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse_out is not None and (lse_out.dtype != torch.float32 or lse_out.shape != (B, Hq)
                                or not lse_out.is_contiguous() or lse_out.device != q.device):
        raise ValueError("lse_out must be a contiguous float32 [B,Hq] tensor on q's device")
    return out, lse_out


def _workspace(q, B, Hq, Hkv, Smax, D, num_splits, workspace):
    need = das_decode_workspace_bytes(B, Hq, Hkv, Smax, D, num_splits)
    if workspace is None:
        # zero-filled: the workspace starts with the library's arrival counters
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
    return workspace, workspace.numel() * workspace.element_size()


def _run_decode(fn_name, q, k_cache, v_cache, seq_lens, scale, out, lse_out, out_dtype,
                num_splits, workspace, stream, with_lse):
    B, Hq, Hkv, Smax, D = _decode_shapes(q, k_cache, v_cache, seq_lens)
    with _on(stream):
        out, lse_out = _outputs(q, B, Hq, D, out, lse_out, out_dtype, with_lse)
        workspace, ws_bytes = _workspace(q, B, Hq, Hkv, Smax, D, num_splits, workspace)
    dtype_code = DAS_BF16 if out.dtype == torch.bfloat16 else DAS_F32
    fn = getattr(load_library(), fn_name)
    _check(fn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), B, Hq, Hkv, Smax, D,
              float(scale), _ptr(out), dtype_code, _ptr(lse_out), int(num_splits),
              _ptr(workspace), ws_bytes, _stream(stream)), fn_name)
    return out, lse_out, workspace


def _scales(k_scale, v_scale, shape):
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        if not (t.is_cuda and t.is_contiguous()) or t.dtype != torch.float32 \
                or tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must be a contiguous float32 {list(shape)} device tensor")


# the entry points with a quantised cache and the cache format of each
_SCALED = {"das_decode_attention_fp8": DAS_E4M3, "das_split_kv_decode_fp8": DAS_E4M3,
           "das_decode_attention_int4": DAS_INT4, "das_split_kv_decode_int4": DAS_INT4}


def _scale_shape(kv_format, B, Hkv, Smax):
    """E4M3: one scale per kv-head; INT4: one per cached row."""
    return (Hkv,) if kv_format == DAS_E4M3 else (B, Hkv, Smax)


def _run_decode_fp8(fn_name, q, k_cache, v_cache, k_scale, v_scale, seq_lens, scale, out,
                    lse_out, out_dtype, num_splits, workspace, stream, with_lse):
    fmt = _SCALED[fn_name]
    B, Hq, Hkv, Smax, D = _decode_shapes(q, k_cache, v_cache, seq_lens, fmt)
    _scales(k_scale, v_scale, _scale_shape(fmt, B, Hkv, Smax))
    with _on(stream):
        out, lse_out = _outputs(q, B, Hq, D, out, lse_out, out_dtype, with_lse)
        workspace, ws_bytes = _workspace(q, B, Hq, Hkv, Smax, D, num_splits, workspace)
    dtype_code = DAS_BF16 if out.dtype == torch.bfloat16 else DAS_F32
    fn = getattr(load_library(), fn_name)
    _check(fn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(seq_lens),
              B, Hq, Hkv, Smax, D, float(scale), _ptr(out), dtype_code, _ptr(lse_out),
              int(num_splits), _ptr(workspace), ws_bytes, _stream(stream)), fn_name)
    return out, lse_out, workspace


class PreparedCall:
    """One C-ABI call with its argument list marshalled once.

    For launch loops (benchmarks, serving steps) where the same tensors are
    used over and over: calling it re-issues the C call with the stored
    pointers and sizes, skipping the Python-side shape checks.  It keeps the
    tensors it points to alive."""

    def __init__(self, name: str, args: tuple, keep: tuple, lib: Optional[ctypes.CDLL] = None):
        self._fn = getattr(lib if lib is not None else load_library(), name)
        self._name = name
        self._args = args
        self._keep = keep

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != DAS_OK:
            raise DasError(rc, self._name)

    def on_library(self, lib: ctypes.CDLL) -> "PreparedCall":
        """The same call (same pointers and sizes) into another build of the
        library, e.g. one from open_library."""
        return PreparedCall(self._name, self._args, self._keep, lib)


def prepare_decode(fn_name: str, q, k_cache, v_cache, seq_lens, scale: float,
                   out: torch.Tensor, lse_out: Optional[torch.Tensor], num_splits: int,
                   workspace: torch.Tensor, stream=None, k_scale=None,
                   v_scale=None) -> PreparedCall:
    """Prepared das_decode_attention / das_split_kv_decode call, or their _fp8
    and _int4 forms (then with k_scale and v_scale); the same checks run once."""
    fmt = _SCALED.get(fn_name, DAS_BF16)
    fp8 = fmt != DAS_BF16
    if not fp8 and fn_name not in ("das_decode_attention", "das_split_kv_decode"):
        raise ValueError(fn_name)
    B, Hq, Hkv, Smax, D = _decode_shapes(q, k_cache, v_cache, seq_lens, fmt)
    if fp8:
        _scales(k_scale, v_scale, _scale_shape(fmt, B, Hkv, Smax))
    out, lse_out = _outputs(q, B, Hq, D, out, lse_out, out.dtype, lse_out is not None)
    ws_bytes = workspace.numel() * workspace.element_size()
    if ws_bytes < das_decode_workspace_bytes(B, Hq, Hkv, Smax, D, num_splits):
        raise DasError(DAS_EWORKSPACE, fn_name)
    code = DAS_BF16 if out.dtype == torch.bfloat16 else DAS_F32
    scales = (_ptr(k_scale), _ptr(v_scale)) if fp8 else ()
    args = (_ptr(q), _ptr(k_cache), _ptr(v_cache)) + scales + (
        _ptr(seq_lens), B, Hq, Hkv, Smax, D, ctypes.c_float(scale), _ptr(out), code,
        _ptr(lse_out), int(num_splits), _ptr(workspace), ws_bytes, _stream(stream))
    return PreparedCall(fn_name, args, (q, k_cache, v_cache, seq_lens, out, lse_out, workspace,
                                        k_scale, v_scale))


def prepare_lse_combine(seq_lens, Hq: int, Hkv: int, Smax: int, D: int, workspace, out,
                        lse_out=None, num_splits: int = 0, stream=None) -> PreparedCall:
    """Prepared das_lse_combine call."""
    B = seq_lens.shape[0]
    code = DAS_BF16 if out.dtype == torch.bfloat16 else DAS_F32
    args = (_ptr(seq_lens), B, Hq, Hkv, Smax, D, int(num_splits), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _ptr(out), code, _ptr(lse_out),
            _stream(stream))
    return PreparedCall("das_lse_combine", args, (seq_lens, workspace, out, lse_out))


def das_decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         seq_lens: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
                         lse_out: Optional[torch.Tensor] = None,
                         out_dtype: torch.dtype = torch.float32, num_splits: int = 0,
                         workspace: Optional[torch.Tensor] = None, stream=None,
                         with_lse: bool = True):
    """Decode attention; returns (out [B,Hq,D], lse [B,Hq] or None)."""
    out, lse_out, _ = _run_decode("das_decode_attention", q, k_cache, v_cache, seq_lens, scale,
                                  out, lse_out, out_dtype, num_splits, workspace, stream, with_lse)
    return out, lse_out


def das_decode_attention_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                 seq_lens: torch.Tensor, scale: float, out: torch.Tensor,
                                 lse_out: Optional[torch.Tensor] = None, num_splits: int = 0,
                                 stream=None):
    """das_decode_attention with the library's static workspace: the caller
    passes its outputs (nothing is allocated on this path); returns (out, lse)."""
    B, Hq, Hkv, Smax, D = _decode_shapes(q, k_cache, v_cache, seq_lens)
    out, lse_out = _outputs(q, B, Hq, D, out, lse_out, out.dtype, False)
    code = DAS_BF16 if out.dtype == torch.bfloat16 else DAS_F32
    _check(load_library().das_decode_attention_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), B, Hq, Hkv, Smax, D, float(scale),
        _ptr(out), code, _ptr(lse_out), int(num_splits), _stream(stream)),
        "das_decode_attention_noalloc")
    return out, lse_out


def das_split_kv_decode(q, k_cache, v_cache, seq_lens, scale, out=None, lse_out=None,
                        out_dtype=torch.float32, num_splits=0, workspace=None, stream=None,
                        with_lse=True):
    """Phase 1 only; returns (out, lse, workspace).  Finish with das_lse_combine."""
    return _run_decode("das_split_kv_decode", q, k_cache, v_cache, seq_lens, scale, out, lse_out,
                       out_dtype, num_splits, workspace, stream, with_lse)


def das_decode_attention_fp8(q, k_cache, v_cache, k_scale, v_scale, seq_lens, scale, out=None,
                             lse_out=None, out_dtype=torch.float32, num_splits=0, workspace=None,
                             stream=None, with_lse=True):
    """Decode attention over an E4M3 K/V cache (codes as uint8 or float8_e4m3fn,
    fp32 scales [Hkv] for K and V); returns (out, lse)."""
    out, lse_out, _ = _run_decode_fp8("das_decode_attention_fp8", q, k_cache, v_cache, k_scale,
                                      v_scale, seq_lens, scale, out, lse_out, out_dtype,
                                      num_splits, workspace, stream, with_lse)
    return out, lse_out


def das_split_kv_decode_fp8(q, k_cache, v_cache, k_scale, v_scale, seq_lens, scale, out=None,
                            lse_out=None, out_dtype=torch.float32, num_splits=0, workspace=None,
                            stream=None, with_lse=True):
    """Phase 1 alone over an E4M3 K/V cache; returns (out, lse, workspace)."""
    return _run_decode_fp8("das_split_kv_decode_fp8", q, k_cache, v_cache, k_scale, v_scale,
                           seq_lens, scale, out, lse_out, out_dtype, num_splits, workspace,
                           stream, with_lse)


def das_decode_attention_int4(q, k_cache, v_cache, k_scale, v_scale, seq_lens, scale, out=None,
                              lse_out=None, out_dtype=torch.float32, num_splits=0,
                              workspace=None, stream=None, with_lse=True):
    """Decode attention over a 4-bit integer K/V cache (packed two's-complement
    codes uint8 [B,Hkv,Smax,D/2], element 2i in the low nibble; fp32 row scales
    [B,Hkv,Smax] for K and V); returns (out, lse)."""
    out, lse_out, _ = _run_decode_fp8("das_decode_attention_int4", q, k_cache, v_cache, k_scale,
                                      v_scale, seq_lens, scale, out, lse_out, out_dtype,
                                      num_splits, workspace, stream, with_lse)
    return out, lse_out


def das_split_kv_decode_int4(q, k_cache, v_cache, k_scale, v_scale, seq_lens, scale, out=None,
                             lse_out=None, out_dtype=torch.float32, num_splits=0, workspace=None,
                             stream=None, with_lse=True):
    """Phase 1 alone over an INT4 K/V cache; returns (out, lse, workspace)."""
    return _run_decode_fp8("das_split_kv_decode_int4", q, k_cache, v_cache, k_scale, v_scale,
                           seq_lens, scale, out, lse_out, out_dtype, num_splits, workspace,
                           stream, with_lse)


def _paged_args(q, k_pool, v_pool, block_table, seq_lens, scale, page_size, layout, k_scale,
                v_scale, out, lse_out, out_dtype, num_splits, workspace, stream, with_lse,
                kv_dtype=None):
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool),
                    ("block_table", block_table), ("seq_lens", seq_lens)):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    if q.dtype != torch.bfloat16 or q.dim() != 3:
        raise ValueError("q must be bfloat16 [B,Hq,D]")
    if kv_dtype is None:   # bf16 or E4M3 from the pool's dtype; INT4 must be named
        if k_pool.dtype == torch.bfloat16:
            kv_dtype = DAS_BF16
        elif k_pool.dtype in (torch.uint8, torch.float8_e4m3fn):
            kv_dtype = DAS_E4M3
        else:
            raise ValueError("page pools must be bfloat16, or E4M3 codes (uint8 / float8_e4m3fn)")
    want = {DAS_BF16: (torch.bfloat16,), DAS_E4M3: (torch.uint8, torch.float8_e4m3fn),
            DAS_INT4: (torch.uint8,)}.get(kv_dtype)
    if want is None or k_pool.dtype not in want:
        raise ValueError("page pool dtype does not match kv_dtype")
    if v_pool.dtype != k_pool.dtype or v_pool.shape != k_pool.shape or k_pool.dim() != 4:
        raise ValueError("k_pool and v_pool must share one 4-d shape and dtype")
    B, Hq, D = q.shape
    if layout == DAS_PAGED_HND:
        num_pages, Hkv, P, Dk = k_pool.shape
    elif layout == DAS_PAGED_NHD:
        num_pages, P, Hkv, Dk = k_pool.shape
    else:
        raise ValueError("layout must be DAS_PAGED_HND or DAS_PAGED_NHD")
    if P != page_size or Dk != (D // 2 if kv_dtype == DAS_INT4 else D):
        raise ValueError("pool shape disagrees with page_size or D")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_blocks]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    if kv_dtype == DAS_E4M3:
        _scales(k_scale, v_scale, (Hkv,))
    elif kv_dtype == DAS_INT4:   # row-scale pools laid out like the code pools
        _scales(k_scale, v_scale, k_pool.shape[:3])
    max_blocks = block_table.shape[1]
    with _on(stream):
        out, lse_out = _outputs(q, B, Hq, D, out, lse_out, out_dtype, with_lse)
        workspace, ws_bytes = _workspace(q, B, Hq, Hkv, max_blocks * P, D, num_splits, workspace)
    code = DAS_BF16 if out.dtype == torch.bfloat16 else DAS_F32
    args = (_ptr(q), _ptr(k_pool), _ptr(v_pool), kv_dtype, _ptr(k_scale), _ptr(v_scale),
            _ptr(block_table), max_blocks, P, num_pages, layout, _ptr(seq_lens), B, Hq, Hkv, D,
            ctypes.c_float(scale), _ptr(out), code, _ptr(lse_out), int(num_splits),
            _ptr(workspace), ws_bytes, _stream(stream))
    keep = (q, k_pool, v_pool, block_table, seq_lens, out, lse_out, workspace, k_scale, v_scale)
    return args, keep, out, lse_out


def das_decode_attention_paged(q, k_pool, v_pool, block_table, seq_lens, scale, page_size,
                               layout=0, k_scale=None, v_scale=None, out=None, lse_out=None,
                               out_dtype=torch.float32, num_splits=0, workspace=None, stream=None,
                               with_lse=True, kv_dtype=None):
    """Decode attention over a paged cache (bf16, E4M3 or -- with
    kv_dtype=DAS_INT4 and row-scale pools shaped like the code pools minus D --
    INT4 page pools; int32 block table [B, max_blocks]); returns (out, lse)."""
    args, _, out, lse_out = _paged_args(q, k_pool, v_pool, block_table, seq_lens, scale,
                                        page_size, layout, k_scale, v_scale, out, lse_out,
                                        out_dtype, num_splits, workspace, stream, with_lse,
                                        kv_dtype)
    _check(load_library().das_decode_attention_paged(*args), "das_decode_attention_paged")
    return out, lse_out


def prepare_decode_paged(q, k_pool, v_pool, block_table, seq_lens, scale, page_size, layout,
                         out, lse_out, num_splits, workspace, stream=None, k_scale=None,
                         v_scale=None, kv_dtype=None) -> "PreparedCall":
    """Prepared das_decode_attention_paged call (same checks once)."""
    args, keep, _, _ = _paged_args(q, k_pool, v_pool, block_table, seq_lens, scale, page_size,
                                   layout, k_scale, v_scale, out, lse_out, out.dtype, num_splits,
                                   workspace, stream, lse_out is not None, kv_dtype)
    return PreparedCall("das_decode_attention_paged", args, keep)


def das_lse_combine(seq_lens: torch.Tensor, Hq: int, Hkv: int, Smax: int, D: int,
                    workspace: torch.Tensor, out: torch.Tensor,
                    lse_out: Optional[torch.Tensor] = None, num_splits: int = 0, stream=None):
    """Phase 2 only: merge the partials in ``workspace`` into ``out`` / ``lse_out``."""
    B = seq_lens.shape[0]
    dtype_code = DAS_BF16 if out.dtype == torch.bfloat16 else DAS_F32
    _check(load_library().das_lse_combine(
        _ptr(seq_lens), B, Hq, Hkv, Smax, D, int(num_splits), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), dtype_code, _ptr(lse_out),
        _stream(stream)), "das_lse_combine")
    return out, lse_out


def das_merge_attn_states(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: torch.Tensor,
                          lse_b: torch.Tensor, o_out: Optional[torch.Tensor] = None,
                          lse_out: Optional[torch.Tensor] = None, stream=None):
    """LSE merge of two attention states; o_* are [..., D], lse_* are [...]."""
    if o_a.shape != o_b.shape or lse_a.shape != lse_b.shape or o_a.shape[:-1] != lse_a.shape:
        raise ValueError("merge: shape mismatch")
    if o_a.dtype != o_b.dtype or o_a.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("o_a and o_b must share dtype float32 or bfloat16")
    if lse_a.dtype != torch.float32 or lse_b.dtype != torch.float32:
        raise ValueError("lse must be float32")
    # the kernel writes rows * D elements of o_a's dtype and rows floats
    if o_out is not None and (o_out.shape != o_a.shape or o_out.dtype != o_a.dtype
                              or not o_out.is_contiguous()):
        raise ValueError("o_out must be a contiguous tensor of o_a's shape and dtype")
    if lse_out is not None and (lse_out.shape != lse_a.shape or lse_out.dtype != torch.float32
                                or not lse_out.is_contiguous()):
        raise ValueError("lse_out must be a contiguous float32 tensor of lse_a's shape")
    for t in (o_a, o_b, lse_a, lse_b) + tuple(t for t in (o_out, lse_out) if t is not None):
        if not (t.is_cuda and t.is_contiguous()) or t.device != o_a.device:
            raise ValueError("merge inputs and outputs must be contiguous tensors on one device")
    with _on(stream):
        if o_out is None:
            o_out = torch.empty_like(o_a)
        if lse_out is None:
            lse_out = torch.empty_like(lse_a)
    D = o_a.shape[-1]
    rows = lse_a.numel()
    code = DAS_BF16 if o_a.dtype == torch.bfloat16 else DAS_F32
    _check(load_library().das_merge_attn_states(
        _ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o_out), _ptr(lse_out), rows, D, code,
        _stream(stream)), "das_merge_attn_states")
    return o_out, lse_out
