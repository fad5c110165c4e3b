"""fp64 CPU oracle for single-query softmax attention and the LSE merge.

TEST INFRASTRUCTURE ONLY: this package is imported by ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` and by
nothing else.  The HIP library never imports, links or calls it, and it
imports nothing from the HIP library.  Inputs come from the shared seeded
generator (``workloads``), which holds no attention arithmetic.

Pieces:

* ``attention``  -- the plain definition in C (fp64, OpenMP over independent
  (batch, head) rows): ``softmax(scale * q.K^T) V`` and its natural-log LSE.
  Sources: FlashDecoding++ post (TechKnowGenie), §1 (decode step) and §5
  (unsplit ground truth as matmul, softmax, matmul).
* ``split_attention`` -- the two-phase split form in the order of §3 of the
  same post (per-chunk max/sum/unnormalised output, then global max,
  correction factors, global sum, division).  Used only to pin that the
  split is exact.
* ``attention_fp8`` / ``e4m3_decode`` -- the same definition over an 8-bit
  floating-point K/V cache (FlashDecoding++ post, §4: quantised K/V turned
  back into wider floats inside the kernel), read as OCP E4M3 codes with one
  fp32 scale per kv-head for K and one for V.
* ``attention_int4`` / ``int4_decode`` -- the same definition over a 4-bit
  integer K/V cache (same post, §4, which names INT4 beside FP8), read as
  two's-complement codes, two per byte (element 2i in the low nibble), with
  one fp32 scale per cached row (batch row, kv-head, token) for K and for V.
* ``gather_paged`` / ``gather_paged_int4`` / ``attention_paged`` -- a paged K/V cache (FlashDecoding++
  post, §6: engines keep K/V in blocks allocated anywhere in a pool, listed
  per sequence by a block table, and map each block onto a slice of a
  chunk).  Row j of sequence b is row j mod P of block
  ``block_table[b][j // P]``; the gather writes that out, and attention over
  the paged cache is the definition above over the gathered rows.
* ``merge`` -- the LSE / online-softmax merge of two attention states that
  the SGLang Diffusion "Parallelism Overview" page relies on for ring hops and
  tail parts ("What happens to the shapes", "Constraints").
* ``abs_attention`` / ``abs_attention_fp8`` / ``abs_attention_int4`` /
  ``abs_attention_paged`` -- the same definitions with every V element
  replaced by its absolute value, out = sum_j w_j |v_j| / Z: the magnitude of
  the terms an output averages.  Rounding inside a kernel moves an output by
  an amount relative to this magnitude, not to the output itself, which can
  cancel to near zero; the bf16-output tolerance is stated in terms of it.
* ``round_to_bf16`` -- fp64 to bfloat16, round-to-nearest-even, directly from
  fp64 (no fp32 step), for the bf16-output tolerance.
* ``attention_fsum_textbook`` -- pure-Python brute force with ``math.fsum``
  and the textbook softmax (no max shift), for tiny inputs.

Every function here is pinned by ``tests/test_oracle.py`` against closed
forms, invariants, brute force and the pages' own equivalence check.
"""
from __future__ import annotations

import ctypes
import math
import os
import struct
import subprocess
from typing import Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "das_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libdas_oracle.so")
_lib = None


def build(verbose: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the C oracle with gcc (host only, no GPU code)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(out + ".tmp", out)
    return out


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def _check_inputs(q, k, v, seq_lens):
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    if q.ndim != 3 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,Hq,D]; k, v must be [B,Hkv,Smax,D]")
    B, Hq, D = q.shape
    if k.shape[0] != B or k.shape[3] != D or seq_lens.shape != (B,):
        raise ValueError("shape mismatch between q, k/v and seq_lens")
    Hkv = k.shape[1]
    if Hkv == 0 or Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return q, k, v, seq_lens


class OracleLib:
    """ctypes view of one build of ``das_oracle.c``."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        p = ctypes.c_void_p
        i32 = ctypes.c_int32
        for name in ("das_oracle_attention", "das_oracle_abs_attention"):
            getattr(lib, name).argtypes = [p, p, p, p, i32, i32, i32, i32, i32,
                                           ctypes.c_double, p, p]
            getattr(lib, name).restype = None
        lib.das_oracle_split_attention.argtypes = [p, p, p, p, i32, i32, i32, i32, i32,
                                                   ctypes.c_double, i32, p, p]
        lib.das_oracle_split_attention.restype = None
        lib.das_oracle_merge.argtypes = [p, p, p, p, ctypes.c_int64, i32, p, p]
        lib.das_oracle_merge.restype = None
        lib.das_oracle_e4m3_decode.argtypes = [p, ctypes.c_int64, p]
        lib.das_oracle_e4m3_decode.restype = None
        for name in ("das_oracle_attention_fp8", "das_oracle_abs_attention_fp8",
                     "das_oracle_attention_int4", "das_oracle_abs_attention_int4"):
            getattr(lib, name).argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32,
                                           ctypes.c_double, p, p]
            getattr(lib, name).restype = None
        lib.das_oracle_int4_decode.argtypes = [p, ctypes.c_int64, p]
        lib.das_oracle_int4_decode.restype = None
        lib.das_oracle_max_threads.argtypes = []
        lib.das_oracle_max_threads.restype = ctypes.c_int
        lib.das_oracle_set_threads.argtypes = [ctypes.c_int]
        lib.das_oracle_set_threads.restype = None
        self.lib = lib
        self.path = path

    def max_threads(self) -> int:
        return int(self.lib.das_oracle_max_threads())

    def set_threads(self, n: int) -> None:
        self.lib.das_oracle_set_threads(int(n))

    def attention(self, q, k, v, seq_lens, scale: float,
                  _fn: str = "das_oracle_attention") -> Tuple[np.ndarray, np.ndarray]:
        """Unsplit fp64 attention.  Inputs are bf16 bit arrays (uint16)."""
        q, k, v, seq_lens = _check_inputs(q, k, v, seq_lens)
        B, Hq, D = q.shape
        Hkv, smax = k.shape[1], k.shape[2]
        out = np.empty((B, Hq, D), dtype=np.float64)
        lse = np.empty((B, Hq), dtype=np.float64)
        getattr(self.lib, _fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(seq_lens), B, Hq, Hkv,
                               smax, D, float(scale), _ptr(out), _ptr(lse))
        return out, lse

    def abs_attention(self, q, k, v, seq_lens, scale: float) -> np.ndarray:
        """sum_j w_j |v_j| / Z per output element (fp64), the softmax weights
        w_j / Z of ``attention``; 0 for an empty row set."""
        return self.attention(q, k, v, seq_lens, scale, _fn="das_oracle_abs_attention")[0]

    def split_attention(self, q, k, v, seq_lens, scale: float,
                        chunk: int) -> Tuple[np.ndarray, np.ndarray]:
        """Two-phase split form with fixed chunks of ``chunk`` rows over [0, Smax)."""
        if chunk < 1:
            raise ValueError("chunk must be >= 1")
        q, k, v, seq_lens = _check_inputs(q, k, v, seq_lens)
        B, Hq, D = q.shape
        Hkv, smax = k.shape[1], k.shape[2]
        out = np.empty((B, Hq, D), dtype=np.float64)
        lse = np.empty((B, Hq), dtype=np.float64)
        self.lib.das_oracle_split_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(seq_lens), B, Hq,
                                            Hkv, smax, D, float(scale), int(chunk), _ptr(out),
                                            _ptr(lse))
        return out, lse

    def e4m3_decode(self, codes) -> np.ndarray:
        """Values of OCP E4M3 codes (uint8), as float64; NaN for the NaN codes."""
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        out = np.empty(codes.shape, dtype=np.float64)
        self.lib.das_oracle_e4m3_decode(_ptr(codes), codes.size, _ptr(out))
        return out

    def attention_fp8(self, q, k, v, k_scale, v_scale, seq_lens, scale: float,
                      _fn: str = "das_oracle_attention_fp8") -> Tuple[np.ndarray, np.ndarray]:
        """Unsplit fp64 attention over an E4M3 K/V cache: q bf16 bits (uint16),
        k/v E4M3 codes (uint8), k_scale/v_scale fp32 per kv-head."""
        q = np.ascontiguousarray(q, dtype=np.uint16)
        k = np.ascontiguousarray(k, dtype=np.uint8)
        v = np.ascontiguousarray(v, dtype=np.uint8)
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        k_scale = np.ascontiguousarray(k_scale, dtype=np.float32)
        v_scale = np.ascontiguousarray(v_scale, dtype=np.float32)
        if q.ndim != 3 or k.ndim != 4 or k.shape != v.shape:
            raise ValueError("q must be [B,Hq,D]; k and v [B,Hkv,Smax,D] of the same shape")
        B, Hq, D = q.shape
        Hkv, smax = k.shape[1], k.shape[2]
        if k.shape[0] != B or k.shape[3] != D or Hq % Hkv or seq_lens.shape != (B,):
            raise ValueError("inconsistent shapes")
        if k_scale.shape != (Hkv,) or v_scale.shape != (Hkv,):
            raise ValueError("k_scale and v_scale must be [Hkv]")
        out = np.empty((B, Hq, D), dtype=np.float64)
        lse = np.empty((B, Hq), dtype=np.float64)
        getattr(self.lib, _fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale),
                               _ptr(seq_lens), B, Hq, Hkv, smax, D, float(scale),
                               _ptr(out), _ptr(lse))
        return out, lse

    def abs_attention_fp8(self, q, k, v, k_scale, v_scale, seq_lens, scale: float) -> np.ndarray:
        """sum_j w_j |v_j| / Z over an E4M3 cache (the magnitude form of
        ``attention_fp8``)."""
        return self.attention_fp8(q, k, v, k_scale, v_scale, seq_lens, scale,
                                  _fn="das_oracle_abs_attention_fp8")[0]

    def int4_decode(self, packed) -> np.ndarray:
        """Values of packed two's-complement INT4 codes (uint8 [..., n/2] ->
        float64 [..., n]): element 2i is the low nibble of byte i."""
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.float64)
        self.lib.das_oracle_int4_decode(_ptr(packed), out.size, _ptr(out))
        return out

    def attention_int4(self, q, k, v, k_scale, v_scale, seq_lens, scale: float,
                       _fn: str = "das_oracle_attention_int4") -> Tuple[np.ndarray, np.ndarray]:
        """Unsplit fp64 attention over an INT4 K/V cache: q bf16 bits (uint16),
        k/v packed INT4 codes (uint8 [B,Hkv,Smax,D/2]), k_scale/v_scale fp32 per
        cached row [B,Hkv,Smax]."""
        q = np.ascontiguousarray(q, dtype=np.uint16)
        k = np.ascontiguousarray(k, dtype=np.uint8)
        v = np.ascontiguousarray(v, dtype=np.uint8)
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        k_scale = np.ascontiguousarray(k_scale, dtype=np.float32)
        v_scale = np.ascontiguousarray(v_scale, dtype=np.float32)
        if q.ndim != 3 or k.ndim != 4 or k.shape != v.shape:
            raise ValueError("q must be [B,Hq,D]; k and v [B,Hkv,Smax,D/2] of the same shape")
        B, Hq, D = q.shape
        Hkv, smax = k.shape[1], k.shape[2]
        if k.shape[0] != B or 2 * k.shape[3] != D or Hq % Hkv or seq_lens.shape != (B,):
            raise ValueError("inconsistent shapes")
        if k_scale.shape != (B, Hkv, smax) or v_scale.shape != (B, Hkv, smax):
            raise ValueError("k_scale and v_scale must be [B,Hkv,Smax]")
        out = np.empty((B, Hq, D), dtype=np.float64)
        lse = np.empty((B, Hq), dtype=np.float64)
        getattr(self.lib, _fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale),
                               _ptr(seq_lens), B, Hq, Hkv, smax, D, float(scale), _ptr(out),
                               _ptr(lse))
        return out, lse

    def abs_attention_int4(self, q, k, v, k_scale, v_scale, seq_lens, scale: float) -> np.ndarray:
        """sum_j w_j |v_j| / Z over an INT4 cache (the magnitude form of
        ``attention_int4``)."""
        return self.attention_int4(q, k, v, k_scale, v_scale, seq_lens, scale,
                                   _fn="das_oracle_abs_attention_int4")[0]

    def merge(self, o_a, lse_a, o_b, lse_b) -> Tuple[np.ndarray, np.ndarray]:
        """LSE merge of two states; o_* are [..., D], lse_* are [...]."""
        o_a = np.ascontiguousarray(o_a, dtype=np.float64)
        o_b = np.ascontiguousarray(o_b, dtype=np.float64)
        lse_a = np.ascontiguousarray(lse_a, dtype=np.float64)
        lse_b = np.ascontiguousarray(lse_b, dtype=np.float64)
        if o_a.shape != o_b.shape or lse_a.shape != lse_b.shape or o_a.shape[:-1] != lse_a.shape:
            raise ValueError("merge: shape mismatch")
        D = o_a.shape[-1]
        rows = int(np.prod(lse_a.shape, dtype=np.int64))
        o = np.empty_like(o_a)
        lse = np.empty_like(lse_a)
        self.lib.das_oracle_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), rows, D,
                                  _ptr(o), _ptr(lse))
        return o, lse


def default() -> OracleLib:
    """The oracle built from ``das_oracle.c`` (compiled on first use if missing or stale)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = OracleLib(_LIB_PATH)
    return _lib


def attention(q, k, v, seq_lens, scale: float):
    return default().attention(q, k, v, seq_lens, scale)


def split_attention(q, k, v, seq_lens, scale: float, chunk: int):
    return default().split_attention(q, k, v, seq_lens, scale, chunk)


def merge(o_a, lse_a, o_b, lse_b):
    return default().merge(o_a, lse_a, o_b, lse_b)


PAGED_HND = 0   # pool [num_pages][Hkv][P][D]
PAGED_NHD = 1   # pool [num_pages][P][Hkv][D]


def gather_paged(pool, block_table, seq_lens, page_size: int, layout: int, smax: int,
                 fill) -> np.ndarray:
    """Contiguous [B][Hkv][smax][D] copy of a paged cache: row j < seq_lens[b]
    of kv-head g is row j % P of page block_table[b][j // P] (head g of it);
    rows at or past seq_lens[b] hold ``fill``."""
    pool = np.asarray(pool)
    block_table = np.asarray(block_table)
    if layout == PAGED_HND:
        _, Hkv, P, D = pool.shape
    elif layout == PAGED_NHD:
        _, P, Hkv, D = pool.shape
    else:
        raise ValueError("layout must be PAGED_HND or PAGED_NHD")
    if P != page_size:
        raise ValueError("pool page size differs from page_size")
    B = len(seq_lens)
    out = np.full((B, Hkv, smax, D), fill, dtype=pool.dtype)
    for b in range(B):
        for j in range(int(seq_lens[b])):
            page = int(block_table[b][j // P])
            r = j % P
            if layout == PAGED_HND:
                out[b, :, j, :] = pool[page, :, r, :]
            else:
                out[b, :, j, :] = pool[page, r, :, :]
    return out


def attention_paged(q, k_pool, v_pool, block_table, seq_lens, page_size: int, layout: int,
                    scale: float, lib=None):
    """fp64 attention over a paged bf16 cache: the definition over the gathered rows."""
    smax = int(np.asarray(block_table).shape[1]) * page_size
    k = gather_paged(k_pool, block_table, seq_lens, page_size, layout, smax, 0x7FC0)
    v = gather_paged(v_pool, block_table, seq_lens, page_size, layout, smax, 0x7FC0)
    return (lib or default()).attention(q, k, v, seq_lens, scale)


def gather_paged_int4(paged):
    """Contiguous INT4 codes and row scales of a paged INT4 cache (a
    workloads.PagedInputs with scale pools): codes [B][Hkv][smax][D/2] (0x88
    past each sequence) and scales [B][Hkv][smax] (NaN past each sequence),
    gathered like ``gather_paged``."""
    smax = int(np.asarray(paged.block_table).shape[1]) * paged.page_size
    sl = paged.base.seq_lens
    args = (paged.block_table, sl, paged.page_size, paged.layout, smax)
    k = gather_paged(paged.k_pool, *args, 0x88)
    v = gather_paged(paged.v_pool, *args, 0x88)
    ks = gather_paged(paged.k_scale_pool[..., None], *args, np.float32(np.nan))[..., 0]
    vs = gather_paged(paged.v_scale_pool[..., None], *args, np.float32(np.nan))[..., 0]
    return k, v, ks, vs


def abs_attention_paged(q, k_pool, v_pool, block_table, seq_lens, page_size: int, layout: int,
                        scale: float, lib=None):
    """sum_j w_j |v_j| / Z over a paged bf16 cache (the gathered rows)."""
    smax = int(np.asarray(block_table).shape[1]) * page_size
    k = gather_paged(k_pool, block_table, seq_lens, page_size, layout, smax, 0x7FC0)
    v = gather_paged(v_pool, block_table, seq_lens, page_size, layout, smax, 0x7FC0)
    return (lib or default()).abs_attention(q, k, v, seq_lens, scale)


def abs_attention(q, k, v, seq_lens, scale: float):
    return default().abs_attention(q, k, v, seq_lens, scale)


def abs_attention_fp8(q, k, v, k_scale, v_scale, seq_lens, scale: float):
    return default().abs_attention_fp8(q, k, v, k_scale, v_scale, seq_lens, scale)


def abs_attention_int4(q, k, v, k_scale, v_scale, seq_lens, scale: float):
    return default().abs_attention_int4(q, k, v, k_scale, v_scale, seq_lens, scale)


def e4m3_decode(codes):
    return default().e4m3_decode(codes)


def int4_decode(packed):
    return default().int4_decode(packed)


def attention_int4(q, k, v, k_scale, v_scale, seq_lens, scale: float):
    return default().attention_int4(q, k, v, k_scale, v_scale, seq_lens, scale)


def attention_fp8(q, k, v, k_scale, v_scale, seq_lens, scale: float):
    return default().attention_fp8(q, k, v, k_scale, v_scale, seq_lens, scale)


def max_threads() -> int:
    return default().max_threads()


def set_threads(n: int) -> None:
    default().set_threads(n)


# ---------------------------------------------------------------------------
# fp64 -> bfloat16, round to nearest, ties to even, straight from fp64.
# bfloat16 keeps 8 significant bits and fp32's exponent range: normal numbers
# down to 2^-126, subnormals spaced 2^-133, largest finite (2 - 2^-7) * 2^127.
# ---------------------------------------------------------------------------
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_to_bf16(x) -> np.ndarray:
    """Return the bfloat16 value nearest to each fp64 value (ties to even), as fp64."""
    x = np.asarray(x, dtype=np.float64)
    mant, expo = np.frexp(x)                    # x = mant * 2**expo, 0.5 <= |mant| < 1
    quantum_exp = np.maximum(expo - 8, -133)     # 8 significant bits; subnormal floor
    scaled = np.ldexp(x, -quantum_exp)
    r = np.ldexp(np.rint(scaled), quantum_exp)   # np.rint rounds half to even
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def bf16_bits_of(values) -> np.ndarray:
    """Bit patterns of values that are already exactly representable in bfloat16."""
    f = np.asarray(values, dtype=np.float64).astype(np.float32)
    bits = f.view(np.uint32)
    if np.any(bits & np.uint32(0xFFFF)):
        raise ValueError("value not representable in bfloat16")
    return (bits >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# Pure-Python brute force (tiny inputs only).
# ---------------------------------------------------------------------------
def bf16_to_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def attention_fsum_textbook(q_row: Sequence[float], k_rows: Sequence[Sequence[float]],
                            v_rows: Sequence[Sequence[float]], scale: float):
    """Textbook softmax attention for one query row, without the max shift.

    weights_j = exp(s_j) / sum_i exp(s_i);  out = sum_j weights_j v_j;
    lse = ln sum_j exp(s_j).  Every sum is a correctly rounded ``math.fsum``.
    Valid only while exp(s_j) stays finite.
    """
    s = [scale * math.fsum(a * b for a, b in zip(q_row, k)) for k in k_rows]
    e = [math.exp(x) for x in s]
    Z = math.fsum(e)
    D = len(v_rows[0]) if v_rows else len(q_row)
    out = [math.fsum(e[j] * v_rows[j][d] for j in range(len(e))) / Z for d in range(D)]
    return out, math.log(Z)
