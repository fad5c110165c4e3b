"""Seeded synthetic inputs for single-query split-KV decode attention.

This module only draws and packs inputs. It holds none of the attention
arithmetic, so that both the fp64 oracle (``oracle/``) and the HIP library
(``decode_attention_split_amd``) can be fed the same bits without sharing any
code with each other.

Recipe (one config = one seed, ``seed = 42 + config index``):

* ``numpy.random.Generator(PCG64(seed))``.
* From the main stream, in this order: ``seq_lens`` (only when lengths are
  random), then q as one float32 ``standard_normal`` draw in (batch, head, d)
  order.
* K and V of batch row ``b``, kv-head ``h`` come from their own stream,
  ``PCG64(seed).jumped(1 + (t*B + b)*Hkv + h)`` with ``t = 0`` for K and
  ``t = 1`` for V: one float32 ``standard_normal`` draw over the valid rows
  in (row, d) order.  Independent streams let large caches be filled on
  several host threads.
* Every draw is rounded to bfloat16 with round-to-nearest-even.  Optional
  exact power-of-two multipliers (the peaked-softmax stress config scales K
  by 4) are applied after rounding.
* K/V rows past ``seq_lens[b]`` are filled with a bfloat16 quiet NaN
  (0x7FC0) so that any kernel reading them contaminates its result.
* ``scale = 1/sqrt(D)`` rounded to float32 (the library takes a float).

Paged caches (``make_paged_inputs``): the contiguous draw above (bf16, E4M3
or INT4), then every sequence's rows are cut into pages of P rows and the
pages are placed in a pool in an order given by
``PCG64(seed + 7919).permutation``; the pool also holds a few spare pages
(all NaN, or INT4 code byte 0x88) that no table points to, and the
block-table entries past a sequence's last page point to a spare page.  An
INT4 cache's row scales are scattered the same way into scale pools.

8-bit (E4M3) K/V caches (``make_fp8_inputs``): q as above; per kv-head
scales ``k_scale[g] = k_mult * (4 + g) / 64`` and ``v_scale[g] = (3 + g) / 64``
(float32); the codes of K (``t = 2``) and V (``t = 3``) of batch row ``b``,
kv-head ``h`` come from stream ``PCG64(seed).jumped(1 + (t*B + b)*Hkv + h)``:
one float32 ``standard_normal`` draw over the valid rows, times ``k_mult``
for K, divided by the head's scale, clamped to +-448 and rounded to the
nearest E4M3 code (ties to even; torch's float8_e4m3fn conversion).  Rows past
``seq_lens[b]`` hold the E4M3 NaN code 0x7F.

The five named configs are the decode shapes the FlashDecoding++ post
(techknowgenie, "FlashDecoding++: 시퀀스 차원 KV 분할 병렬화 ...") argues
about in §1-§2: single-query decode, GQA with 8 KV heads, long context, a
batched variable-length mix and a ragged peaked-softmax stress case.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional, Sequence

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    smax: int
    seq_lens: Optional[Sequence[int]] = None   # fixed lengths; None = random or all smax
    random_lens: Optional[tuple] = None         # (low, high) inclusive, drawn first
    k_mult: float = 1.0                         # exact power of two applied to K after rounding
    description: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.D)))


CONFIGS = [
    Config("mha_b1_h8_d64_l1024", B=1, Hq=8, Hkv=8, D=64, smax=1024,
           description="MHA decode, B=1, Hq=Hkv=8, D=64, L=1024"),
    Config("gqa_b1_h32x8_d128_l32768", B=1, Hq=32, Hkv=8, D=128, smax=32768,
           description="Llama-3-8B-shaped GQA decode, B=1, Hq=32, Hkv=8, D=128, L=32768"),
    Config("gqa_b1_h32x8_d128_l131072", B=1, Hq=32, Hkv=8, D=128, smax=131072,
           description="long-context GQA decode, B=1, Hq=32, Hkv=8, D=128, L=131072"),
    Config("gqa_b64_h32x8_d128_varlen16k", B=64, Hq=32, Hkv=8, D=128, smax=16384,
           random_lens=(512, 16384),
           description="batched varlen GQA decode, B=64, L~U[512,16384], Smax=16384"),
    Config("gqa8_b8_h64x8_d128_ragged", B=8, Hq=64, Hkv=8, D=128, smax=100003,
           seq_lens=(1, 17, 255, 4095, 4097, 16383, 65537, 100003), k_mult=4.0,
           description="ragged group-8 GQA stress, B=8, Hq=64, Hkv=8, K x4 (peaked softmax)"),
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 bit patterns, nearest-even (finite inputs)."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    u += t
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _scale_bits(bits: np.ndarray, mult: float) -> np.ndarray:
    if mult == 1.0:
        return bits
    m, e = math.frexp(mult)
    if m != 0.5:
        raise ValueError("k_mult must be a power of two so that scaling stays exact")
    return f32_to_bf16_bits(bf16_bits_to_f32(bits) * np.float32(mult))


@dataclasses.dataclass
class Inputs:
    config: Config
    seed: int
    q: np.ndarray          # uint16 [B, Hq, D]
    k: np.ndarray          # uint16 [B, Hkv, Smax, D]
    v: np.ndarray          # uint16 [B, Hkv, Smax, D]
    seq_lens: np.ndarray   # int32 [B]
    scale: float

    @property
    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes: every valid row of K and V read once per kv-head."""
        c = self.config
        return int(self.seq_lens.astype(np.int64).sum()) * c.Hkv * c.D * 2 * 2


def draw_seq_lens(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    if cfg.random_lens is not None:
        lo, hi = cfg.random_lens
        return rng.integers(lo, hi, size=cfg.B, endpoint=True).astype(np.int32)
    if cfg.seq_lens is not None:
        return np.asarray(cfg.seq_lens, dtype=np.int32)
    return np.full(cfg.B, cfg.smax, dtype=np.int32)


def _fill_rows(seed: int, tensor: int, B: int, H: int, smax: int, D: int,
               lens: np.ndarray, mult: float = 1.0) -> np.ndarray:
    """K (tensor 0) or V (tensor 1): seeded valid rows, NaN-poisoned beyond them."""
    out = np.full((B, H, smax, D), BF16_QNAN, dtype=np.uint16)

    def one(task: int) -> None:
        b, h = divmod(task, H)
        L = int(lens[b])
        if L == 0:
            return
        rng = np.random.Generator(np.random.PCG64(seed).jumped(1 + (tensor * B + b) * H + h))
        bits = f32_to_bf16_bits(rng.standard_normal(L * D, dtype=np.float32))
        out[b, h, :L, :] = _scale_bits(bits, mult).reshape(L, D)

    tasks = range(B * H)
    workers = min(B * H, max(1, os.cpu_count() or 1), 16)
    if workers <= 1 or B * H * int(lens.max(initial=0)) * D < (1 << 22):
        for t in tasks:
            one(t)
    else:
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, tasks))
    return out


def make_inputs(cfg: Config, seed: int, smax: Optional[int] = None,
                seq_lens: Optional[Sequence[int]] = None) -> Inputs:
    """Draw one seeded input set for ``cfg``.

    ``smax`` / ``seq_lens`` override the config's cache length and lengths
    (used for small parity cases and edge lengths); an explicit ``seq_lens``
    replaces the length draw.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int32)
    else:
        lens = draw_seq_lens(cfg, rng)
    B = len(lens)
    S = int(smax if smax is not None else max(cfg.smax, int(lens.max(initial=0))))
    if lens.size and (lens.min() < 0 or lens.max() > S):
        raise ValueError("seq_lens must lie in [0, Smax]")
    q = f32_to_bf16_bits(rng.standard_normal(B * cfg.Hq * cfg.D, dtype=np.float32))
    q = q.reshape(B, cfg.Hq, cfg.D)
    k = _fill_rows(seed, 0, B, cfg.Hkv, S, cfg.D, lens, cfg.k_mult)
    v = _fill_rows(seed, 1, B, cfg.Hkv, S, cfg.D, lens)
    return Inputs(cfg, seed, q, k, v, lens, cfg.scale)


def make_inputs_bulk(cfg: Config, seed: int, seq_lens: Sequence[int],
                     smax: Optional[int] = None) -> Inputs:
    """Like ``make_inputs`` for very large batches of short sequences: q, then
    all valid rows of K (in (b, head, row, dim) order), then all of V, each
    drawn in one call from one ``Generator(PCG64(seed))`` (``make_inputs``
    draws every (b, head) from its own jumped stream, whose set-up dominates
    when there are hundreds of thousands of them).  A different draw from
    ``make_inputs`` with the same seed; rows past each sequence are NaN."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.asarray(seq_lens, dtype=np.int32)
    B = len(lens)
    S = int(smax if smax is not None else max(cfg.smax, int(lens.max(initial=0))))
    if lens.size and (lens.min() < 0 or lens.max() > S):
        raise ValueError("seq_lens must lie in [0, Smax]")
    q = f32_to_bf16_bits(rng.standard_normal(B * cfg.Hq * cfg.D, dtype=np.float32))
    q = q.reshape(B, cfg.Hq, cfg.D)
    # flat row index of every valid row, (b, head) blocks of S rows in order
    per = np.repeat(lens.astype(np.int64), cfg.Hkv)                    # rows per (b, head)
    n = int(per.sum())
    first = np.repeat(np.arange(B * cfg.Hkv, dtype=np.int64) * S, per)
    within = np.arange(n, dtype=np.int64) - np.repeat(np.cumsum(per) - per, per)
    rows = first + within
    out = []
    for mult in (cfg.k_mult, 1.0):
        t = np.full((B * cfg.Hkv * S, cfg.D), BF16_QNAN, dtype=np.uint16)
        bits = f32_to_bf16_bits(rng.standard_normal(n * cfg.D, dtype=np.float32))
        t[rows] = _scale_bits(bits, mult).reshape(n, cfg.D)
        out.append(t.reshape(B, cfg.Hkv, S, cfg.D))
    return Inputs(cfg, seed, q, out[0], out[1], lens, cfg.scale)


def config_inputs(index: int) -> Inputs:
    """The named config ``index`` at its full size, seed 42 + index."""
    return make_inputs(CONFIGS[index], 42 + index)


def custom_config(B: int, Hq: int, Hkv: int, D: int, smax: int, name: str = "custom",
                  k_mult: float = 1.0) -> Config:
    return Config(name, B=B, Hq=Hq, Hkv=Hkv, D=D, smax=smax, k_mult=k_mult)


E4M3_NAN = np.uint8(0x7F)


def fp8_scales(cfg: Config):
    """Per kv-head float32 scales (k_scale, v_scale) of the 8-bit caches."""
    g = np.arange(cfg.Hkv, dtype=np.float64)
    k_scale = (cfg.k_mult * (4.0 + g) / 64.0).astype(np.float32)
    v_scale = ((3.0 + g) / 64.0).astype(np.float32)
    return k_scale, v_scale


def _fill_fp8_rows(seed: int, tensor: int, B: int, H: int, smax: int, D: int,
                   lens: np.ndarray, head_scale: np.ndarray, mult: float = 1.0) -> np.ndarray:
    """E4M3 codes of K (tensor 2) or V (tensor 3), NaN code beyond the valid rows."""
    import torch

    out = np.full((B, H, smax, D), E4M3_NAN, dtype=np.uint8)

    def one(task: int) -> None:
        b, h = divmod(task, H)
        L = int(lens[b])
        if L == 0:
            return
        rng = np.random.Generator(np.random.PCG64(seed).jumped(1 + (tensor * B + b) * H + h))
        x = rng.standard_normal(L * D, dtype=np.float32)
        if mult != 1.0:
            x *= np.float32(mult)
        x /= head_scale[h]
        np.clip(x, -448.0, 448.0, out=x)
        codes = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        out[b, h, :L, :] = codes.reshape(L, D)

    tasks = range(B * H)
    workers = min(B * H, max(1, os.cpu_count() or 1), 16)
    if workers <= 1 or B * H * int(lens.max(initial=0)) * D < (1 << 22):
        for t in tasks:
            one(t)
    else:
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, tasks))
    return out


@dataclasses.dataclass
class Fp8Inputs:
    config: Config
    seed: int
    q: np.ndarray          # uint16 [B, Hq, D] bf16 bits
    k: np.ndarray          # uint8 [B, Hkv, Smax, D] E4M3 codes
    v: np.ndarray          # uint8 [B, Hkv, Smax, D] E4M3 codes
    k_scale: np.ndarray    # float32 [Hkv]
    v_scale: np.ndarray    # float32 [Hkv]
    seq_lens: np.ndarray   # int32 [B]
    scale: float

    @property
    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes: every valid row of K and V read once (1 byte per element)."""
        c = self.config
        return int(self.seq_lens.astype(np.int64).sum()) * c.Hkv * c.D * 2


def make_fp8_inputs(cfg: Config, seed: int, smax: Optional[int] = None,
                    seq_lens: Optional[Sequence[int]] = None) -> Fp8Inputs:
    """One seeded input set for ``cfg`` with an 8-bit (E4M3) K/V cache."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int32)
    else:
        lens = draw_seq_lens(cfg, rng)
    B = len(lens)
    S = int(smax if smax is not None else max(cfg.smax, int(lens.max(initial=0))))
    if lens.size and (lens.min() < 0 or lens.max() > S):
        raise ValueError("seq_lens must lie in [0, Smax]")
    q = f32_to_bf16_bits(rng.standard_normal(B * cfg.Hq * cfg.D, dtype=np.float32))
    q = q.reshape(B, cfg.Hq, cfg.D)
    k_scale, v_scale = fp8_scales(cfg)
    k = _fill_fp8_rows(seed, 2, B, cfg.Hkv, S, cfg.D, lens, k_scale, cfg.k_mult)
    v = _fill_fp8_rows(seed, 3, B, cfg.Hkv, S, cfg.D, lens, v_scale)
    return Fp8Inputs(cfg, seed, q, k, v, k_scale, v_scale, lens, cfg.scale)


def config_fp8_inputs(index: int) -> Fp8Inputs:
    """The named config ``index`` at its full size with an E4M3 cache, seed 42 + index."""
    return make_fp8_inputs(CONFIGS[index], 42 + index)


def _fill_int4_rows(seed: int, tensor: int, B: int, H: int, smax: int, D: int,
                    lens: np.ndarray, mult: float = 1.0):
    """Packed INT4 codes and per-row fp32 scales of K (tensor 2) or V (tensor 3).

    Each valid row of standard normals (times ``mult``) gets the scale
    max|x| / 7.5 and the codes rint(x / scale) clipped to [-8, 7], so every code
    value occurs; two's-complement nibbles, element 2i in the low nibble.  Rows
    past the valid ones hold code byte 0x88 and a NaN scale."""
    codes = np.full((B, H, smax, D // 2), 0x88, dtype=np.uint8)
    scales = np.full((B, H, smax), np.nan, dtype=np.float32)

    def one(task: int) -> None:
        b, h = divmod(task, H)
        L = int(lens[b])
        if L == 0:
            return
        rng = np.random.Generator(np.random.PCG64(seed).jumped(1 + (tensor * B + b) * H + h))
        x = rng.standard_normal(L * D, dtype=np.float32).reshape(L, D)
        if mult != 1.0:
            x *= np.float32(mult)
        s = (np.max(np.abs(x), axis=1) / np.float32(7.5)).astype(np.float32)
        s[s == 0] = np.float32(1.0)
        n = np.clip(np.rint(x / s[:, None]), -8, 7).astype(np.int8).view(np.uint8) & np.uint8(15)
        codes[b, h, :L, :] = n[:, 0::2] | (n[:, 1::2] << np.uint8(4))
        scales[b, h, :L] = s

    tasks = range(B * H)
    workers = min(B * H, max(1, os.cpu_count() or 1), 16)
    if workers <= 1 or B * H * int(lens.max(initial=0)) * D < (1 << 22):
        for t in tasks:
            one(t)
    else:
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, tasks))
    return codes, scales


@dataclasses.dataclass
class Int4Inputs:
    config: Config
    seed: int
    q: np.ndarray          # uint16 [B, Hq, D] bf16 bits
    k: np.ndarray          # uint8 [B, Hkv, Smax, D/2] packed INT4 codes
    v: np.ndarray          # uint8 [B, Hkv, Smax, D/2] packed INT4 codes
    k_scale: np.ndarray    # float32 [B, Hkv, Smax]
    v_scale: np.ndarray    # float32 [B, Hkv, Smax]
    seq_lens: np.ndarray   # int32 [B]
    scale: float

    @property
    def kv_bytes(self) -> int:
        """Algorithmic bytes: every valid row of K and V read once, D/2 bytes of
        codes plus its 4-byte scale."""
        c = self.config
        return int(self.seq_lens.astype(np.int64).sum()) * c.Hkv * (c.D // 2 + 4) * 2


def make_int4_inputs(cfg: Config, seed: int, smax: Optional[int] = None,
                     seq_lens: Optional[Sequence[int]] = None) -> Int4Inputs:
    """One seeded input set for ``cfg`` with a 4-bit integer K/V cache (same
    draw order and streams as the bf16 inputs: seq_lens, q, then K, then V)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int32)
    else:
        lens = draw_seq_lens(cfg, rng)
    B = len(lens)
    S = int(smax if smax is not None else max(cfg.smax, int(lens.max(initial=0))))
    if lens.size and (lens.min() < 0 or lens.max() > S):
        raise ValueError("seq_lens must lie in [0, Smax]")
    if cfg.D % 2:
        raise ValueError("INT4 rows need an even D")
    q = f32_to_bf16_bits(rng.standard_normal(B * cfg.Hq * cfg.D, dtype=np.float32))
    q = q.reshape(B, cfg.Hq, cfg.D)
    k, ks = _fill_int4_rows(seed, 2, B, cfg.Hkv, S, cfg.D, lens, cfg.k_mult)
    v, vs = _fill_int4_rows(seed, 3, B, cfg.Hkv, S, cfg.D, lens)
    return Int4Inputs(cfg, seed, q, k, v, ks, vs, lens, cfg.scale)


def config_int4_inputs(index: int) -> Int4Inputs:
    """The seeded INT4 inputs of workload ``index`` (seed 42 + index)."""
    return make_int4_inputs(CONFIGS[index], 42 + index)


PAGED_HND = 0   # pool [num_pages][Hkv][P][D]
PAGED_NHD = 1   # pool [num_pages][P][Hkv][D]


def scatter_to_pages(k: np.ndarray, v: np.ndarray, seq_lens: np.ndarray, page_size: int,
                     layout: int, seed: int, fill, spare_pages: int = 3):
    """Cut every sequence's valid rows of k and v ([B][Hkv][Smax][D]) into
    pages of page_size rows and place the pages in a pool in the order
    ``PCG64(seed + 7919).permutation``; spare pages (all ``fill``) close the
    pool and fill the block-table entries past each sequence's last page.
    Returns (k_pool, v_pool, block_table)."""
    B, Hkv, S, D = k.shape
    P = int(page_size)
    max_blocks = (S + P - 1) // P
    used = [(int(L) + P - 1) // P for L in seq_lens]
    n_used = int(sum(used))
    num_pages = n_used + spare_pages
    order = np.random.Generator(np.random.PCG64(seed + 7919)).permutation(num_pages)
    spare = [int(p) for p in order[n_used:]] or [0]
    table = np.empty((B, max_blocks), dtype=np.int32)
    shape = (num_pages, Hkv, P, D) if layout == PAGED_HND else (num_pages, P, Hkv, D)
    k_pool = np.full(shape, fill, dtype=k.dtype)
    v_pool = np.full(shape, fill, dtype=v.dtype)
    nxt = 0
    for b in range(B):
        L = int(seq_lens[b])
        for i in range(max_blocks):
            if i < used[b]:
                page = int(order[nxt])
                nxt += 1
                j0, j1 = i * P, min(L, (i + 1) * P)
                for src, pool in ((k, k_pool), (v, v_pool)):
                    rows = src[b, :, j0:j1, :]                     # [Hkv][n][D]
                    if layout == PAGED_HND:
                        pool[page, :, : j1 - j0, :] = rows
                    else:
                        pool[page, : j1 - j0, :, :] = rows.transpose(1, 0, 2)
                table[b, i] = page
            else:
                table[b, i] = spare[i % len(spare)]
    return k_pool, v_pool, table


@dataclasses.dataclass
class PagedInputs:
    base: object              # Inputs, Fp8Inputs or Int4Inputs: the same rows, contiguous
    page_size: int
    layout: int
    k_pool: np.ndarray        # [num_pages][Hkv][P][D] (HND) or [num_pages][P][Hkv][D] (NHD)
    v_pool: np.ndarray        # (INT4: D/2 bytes of codes per row)
    block_table: np.ndarray   # int32 [B][max_blocks]
    k_scale_pool: Optional[np.ndarray] = None   # INT4: float32 [num_pages][Hkv][P] (HND)
    v_scale_pool: Optional[np.ndarray] = None   # or [num_pages][P][Hkv] (NHD)

    @property
    def kv_bytes(self) -> int:
        return self.base.kv_bytes


def make_paged_inputs(cfg: Config, seed: int, page_size: int, layout: int = PAGED_HND,
                      smax: Optional[int] = None, seq_lens: Optional[Sequence[int]] = None,
                      spare_pages: int = 3, fp8: bool = False, int4: bool = False,
                      base=None) -> PagedInputs:
    """``make_inputs`` (or ``make_fp8_inputs`` / ``make_int4_inputs``; same
    seed, same rows), scattered into a page pool.  An INT4 cache's row scales
    go into scale pools laid out like the code pools (same pages, same
    table); spare rows hold code byte 0x88 and a NaN scale.  ``base``: inputs
    of that format already drawn with this seed (``cfg``, ``smax`` and
    ``seq_lens`` are then not used to draw them again)."""
    if fp8 and int4:
        raise ValueError("one cache format at a time")
    if int4:
        base = base if base is not None else make_int4_inputs(cfg, seed, smax=smax,
                                                              seq_lens=seq_lens)
        fill = np.uint8(0x88)
    elif fp8:
        base = base if base is not None else make_fp8_inputs(cfg, seed, smax=smax,
                                                             seq_lens=seq_lens)
        fill = E4M3_NAN
    else:
        base = base if base is not None else make_inputs(cfg, seed, smax=smax,
                                                         seq_lens=seq_lens)
        fill = BF16_QNAN
    if base.k.dtype != (np.uint8 if (fp8 or int4) else np.uint16):
        raise ValueError("base inputs are not of the requested cache format")
    k_pool, v_pool, table = scatter_to_pages(base.k, base.v, base.seq_lens, page_size, layout,
                                             seed, fill, spare_pages)
    ks_pool = vs_pool = None
    if int4:
        ks_pool, vs_pool, table_s = scatter_to_pages(
            base.k_scale[..., None], base.v_scale[..., None], base.seq_lens, page_size, layout,
            seed, np.float32(np.nan), spare_pages)
        assert np.array_equal(table, table_s)
        ks_pool, vs_pool = ks_pool[..., 0].copy(), vs_pool[..., 0].copy()
    return PagedInputs(base, int(page_size), layout, k_pool, v_pool, table, ks_pool, vs_pool)
