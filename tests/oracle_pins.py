"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes one build of the oracle (``oracle.OracleLib``)
and raises ``AssertionError`` when that build disagrees with a closed form, an
invariant of softmax attention or the LSE merge, a pure-Python brute force, a
library routine, or the equivalence check printed in the FlashDecoding++ post
(TechKnowGenie, §5).  ``tests/test_oracle.py`` runs them on the real oracle;
``tests/test_oracle_mutants.py`` runs them on copies of the oracle with planted
mistakes and requires every mistake to be caught.
"""
from __future__ import annotations

import functools
import json
import math
import os
import re
from fractions import Fraction

import numpy as np

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bits(values) -> np.ndarray:
    return oracle.bf16_bits_of(np.asarray(values, dtype=np.float64))


def _f(bits) -> np.ndarray:
    return workloads.bf16_bits_to_f32(bits).astype(np.float64)


def _small(seed, B=2, Hq=4, Hkv=2, D=16, smax=24, lens=(24, 13), k_mult=1.0):
    cfg = workloads.custom_config(B, Hq, Hkv, D, smax, k_mult=k_mult)
    return workloads.make_inputs(cfg, seed, smax=smax, seq_lens=lens)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max |diff| {err:.3e} > {tol:.1e}"


def expr(s: str):
    """Closed-form expression from the golden files: integer, a/b, or log(n)."""
    s = str(s).strip()
    if re.fullmatch(r"-?\d+(/\d+)?", s):
        return float(Fraction(s))
    m = re.fullmatch(r"log\((\d+)\)", s)
    if m:
        return math.log(int(m.group(1)))
    raise ValueError(f"unknown expression {s!r}")


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def pin_zero_query_gives_mean(lib):
    """q = 0: every logit is 0, out = mean of the valid V rows, lse = ln L exactly."""
    x = _small(11, lens=(24, 13))
    q0 = np.zeros_like(x.q)
    out, lse = lib.attention(q0, x.k, x.v, x.seq_lens, x.scale)
    for b, L in enumerate(x.seq_lens):
        for h in range(x.q.shape[1]):
            g = h // (x.q.shape[1] // x.k.shape[1])
            rows = _f(x.v[b, g, :L])
            mean = [math.fsum(rows[:, d]) / L for d in range(rows.shape[1])]
            _close(out[b, h], mean, 1e-14, "q=0 mean")
            assert lse[b, h] == math.log(L), "q=0: lse must be exactly ln L"


def pin_zero_scale_gives_mean(lib):
    """scale = 0 with a nonzero q: same closed form as q = 0."""
    x = _small(12, lens=(7, 24))
    out, lse = lib.attention(x.q, x.k, x.v, x.seq_lens, 0.0)
    for b, L in enumerate(x.seq_lens):
        rows = _f(x.v[b, 0, :L])
        _close(out[b, 0], rows.sum(axis=0) / L, 1e-14, "scale=0 mean")
        assert lse[b, 0] == math.log(L)


def pin_single_row(lib):
    """L = 1: out is that V row exactly; lse is the logit scale * q.k_0."""
    x = _small(13, lens=(1, 1))
    out, lse = lib.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    G = x.q.shape[1] // x.k.shape[1]
    for b in range(2):
        for h in range(x.q.shape[1]):
            g = h // G
            assert np.array_equal(out[b, h], _f(x.v[b, g, 0])), "L=1: out must equal the V row"
            s = x.scale * math.fsum(_f(x.q[b, h]) * _f(x.k[b, g, 0]))
            assert abs(lse[b, h] - s) <= 1e-15 * max(1.0, abs(s)), "L=1: lse must be the logit"


def pin_worked_examples(lib):
    """Hand-derived closed forms stored in tests/golden/worked_examples.json."""
    with open(os.path.join(GOLDEN, "worked_examples.json")) as fh:
        doc = json.load(fh)
    for ex in doc["examples"]:
        Hq, Hkv, D = ex["Hq"], ex["Hkv"], ex["D"]
        L = len(ex["k"][0])
        q = _bits(ex["q"]).reshape(1, Hq, D)
        k = _bits(ex["k"]).reshape(1, Hkv, L, D)
        v = _bits(ex["v"]).reshape(1, Hkv, L, D)
        out, lse = lib.attention(q, k, v, np.array([L], np.int32), expr(ex["scale"]))
        want_out = np.array([[expr(e) for e in row] for row in ex["out"]])
        want_lse = np.array([expr(e) for e in ex["lse"]])
        _close(out[0], want_out, 1e-14, ex["name"] + " out")
        _close(lse[0], want_lse, 1e-14, ex["name"] + " lse")


def pin_one_hot_values_give_probabilities(lib):
    """V rows = unit vectors: out[:L] is the probability vector itself.

    Compared with the textbook softmax (no max shift, math.fsum) and with
    torch's fp64 softmax / logsumexp (the unsplit ground truth of §5)."""
    import torch

    D, L = 16, 11
    x = _small(14, B=1, Hq=2, Hkv=1, D=D, smax=L, lens=(L,))
    v = np.zeros_like(x.v)
    for j in range(L):
        v[0, 0, j, j] = _bits([1.0])[0]
    out, lse = lib.attention(x.q, x.k, v, x.seq_lens, x.scale)
    for h in range(2):
        qf, kf = _f(x.q[0, h]), _f(x.k[0, 0, :L])
        ref, ref_lse = oracle.attention_fsum_textbook(list(qf), kf.tolist(), np.eye(L, D).tolist(),
                                                      x.scale)
        _close(out[0, h], ref, 1e-15, "one-hot V vs textbook softmax")
        assert np.all(out[0, h, L:] == 0.0)
        s = torch.tensor(kf @ qf * x.scale, dtype=torch.float64)
        _close(out[0, h, :L], torch.softmax(s, 0).numpy(), 1e-15, "one-hot V vs torch softmax")
        assert abs(lse[0, h] - torch.logsumexp(s, 0).item()) <= 1e-14
        assert abs(lse[0, h] - ref_lse) <= 1e-14


def pin_two_rows_huge_logits(lib):
    """Two rows with logits near 1000, where exp overflows fp64 without the max shift.

    Closed form: out = sigma(a-b) v0 + sigma(b-a) v1, lse = max(a,b) + log1p(exp(-|a-b|))."""
    q = _bits([[[1, 0, 0, 0]]])
    k = _bits([[[[1, 0, 0, 0], [1.0078125, 0, 0, 0]]]])
    v = _bits([[[[1, -2, 0.5, 3], [-1, 4, 0.25, -3]]]])
    scale = 1000.0
    a, b = scale * 1.0, scale * 1.0078125
    out, lse = lib.attention(q, k, v, np.array([2], np.int32), scale)
    assert np.all(np.isfinite(out)) and math.isfinite(lse[0, 0])
    sa = 1.0 / (1.0 + math.exp(b - a))
    sb = 1.0 / (1.0 + math.exp(a - b))
    want = sa * _f(v[0, 0, 0]) + sb * _f(v[0, 0, 1])
    _close(out[0, 0], want, 1e-15, "two-row closed form")
    assert abs(lse[0, 0] - (max(a, b) + math.log1p(math.exp(-abs(a - b))))) <= 1e-12


def pin_identical_keys_give_mean(lib):
    """All K rows equal: equal weights, out = mean V, lse = s + ln L."""
    x = _small(15, B=1, Hq=2, Hkv=1, D=8, smax=9, lens=(9,))
    k = np.broadcast_to(x.k[:, :, :1, :], x.k.shape).copy()
    out, lse = lib.attention(x.q, k, x.v, x.seq_lens, x.scale)
    rows = _f(x.v[0, 0])
    for h in range(2):
        _close(out[0, h], rows.mean(axis=0), 1e-15, "identical keys mean")
        s = x.scale * math.fsum(_f(x.q[0, h]) * _f(k[0, 0, 0]))
        assert abs(lse[0, h] - (s + math.log(9))) <= 1e-14


def pin_gqa_head_mapping(lib):
    """kv-head g holds constant V = 2^g: query head h must return 2^(h // G) exactly."""
    for Hq, Hkv in ((8, 2), (8, 8), (8, 1), (6, 3), (32, 2)):
        x = _small(16, B=2, Hq=Hq, Hkv=Hkv, D=4, smax=10, lens=(10, 6))
        v = np.zeros_like(x.v)
        for g in range(Hkv):
            v[:, g] = _bits([2.0 ** g])[0]
        out, _ = lib.attention(x.q, x.k, v, x.seq_lens, x.scale)
        G = Hq // Hkv
        for h in range(Hq):
            assert np.all(out[:, h] == 2.0 ** (h // G)), f"head {h} of Hq={Hq}, Hkv={Hkv}"


def pin_empty_and_poisoned_rows(lib):
    """L = 0 gives (0, -inf); NaN rows past L never leak; L > Smax is clamped to Smax."""
    x = _small(17, lens=(0, 5))
    assert np.isnan(_f(x.k[1, 0, 5])).all()
    out, lse = lib.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    assert np.all(out[0] == 0.0) and np.all(lse[0] == -np.inf)
    assert np.all(np.isfinite(out[1])) and np.all(np.isfinite(lse[1]))
    y = _small(18, lens=(24, 24))
    full = lib.attention(y.q, y.k, y.v, y.seq_lens, y.scale)
    over = lib.attention(y.q, y.k, y.v, np.array([30, 99], np.int32), y.scale)
    assert np.array_equal(full[0], over[0]) and np.array_equal(full[1], over[1])


def pin_bruteforce_tiny(lib):
    """C oracle vs the pure-Python textbook formula with math.fsum on tiny inputs."""
    for D, lens in ((4, (40, 3)), (64, (17, 1))):
        x = _small(19 + D, B=2, Hq=4, Hkv=2, D=D, smax=40, lens=lens)
        out, lse = lib.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
        for b, L in enumerate(lens):
            for h in range(4):
                g = h // 2
                ref, ref_lse = oracle.attention_fsum_textbook(
                    _f(x.q[b, h]).tolist(), _f(x.k[b, g, :L]).tolist(), _f(x.v[b, g, :L]).tolist(),
                    x.scale)
                _close(out[b, h], ref, 1e-13, f"brute force D={D} b={b} h={h}")
                assert abs(lse[b, h] - ref_lse) <= 1e-13


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def pin_row_permutation_invariance(lib):
    """Permuting the valid K/V rows (same permutation on both) changes nothing."""
    x = _small(20, lens=(24, 19))
    rng = np.random.default_rng(0)
    k, v = x.k.copy(), x.v.copy()
    for b, L in enumerate(x.seq_lens):
        perm = rng.permutation(L)
        k[b, :, :L] = x.k[b, :, perm].transpose(1, 0, 2)
        v[b, :, :L] = x.v[b, :, perm].transpose(1, 0, 2)
    a = lib.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    p = lib.attention(x.q, k, v, x.seq_lens, x.scale)
    _close(a[0], p[0], 1e-14, "permuted rows out")
    _close(a[1], p[1], 1e-13, "permuted rows lse")


def pin_linear_in_v(lib):
    """out(2V) = 2 out(V) exactly, and out(Va + Vb) = out(Va) + out(Vb)."""
    x = _small(21, lens=(24, 10))
    o1, _ = lib.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    v2 = _bits(np.nan_to_num(_f(x.v)) * 2.0)
    o2, _ = lib.attention(x.q, x.k, v2, x.seq_lens, x.scale)
    assert np.array_equal(o2, 2.0 * o1), "doubling V must double out exactly"
    rng = np.random.default_rng(1)
    va = rng.integers(-8, 9, size=x.v.shape).astype(np.float64)
    vb = rng.integers(-8, 9, size=x.v.shape).astype(np.float64)
    oa, _ = lib.attention(x.q, x.k, _bits(va), x.seq_lens, x.scale)
    ob, _ = lib.attention(x.q, x.k, _bits(vb), x.seq_lens, x.scale)
    oab, _ = lib.attention(x.q, x.k, _bits(va + vb), x.seq_lens, x.scale)
    _close(oab, oa + ob, 1e-13, "linearity in V")


def pin_split_equals_unsplit(lib):
    """The two-phase split is exact for every chunking, empty trailing chunks included."""
    x = _small(22, B=3, Hq=8, Hkv=2, D=16, smax=40, lens=(40, 23, 1), k_mult=4.0)
    full = lib.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    for chunk in (1, 2, 3, 5, 16, 39, 40, 47):
        sp = lib.split_attention(x.q, x.k, x.v, x.seq_lens, x.scale, chunk)
        _close(sp[0], full[0], 1e-13, f"split chunk={chunk} out")
        _close(sp[1], full[1], 1e-13, f"split chunk={chunk} lse")


@functools.lru_cache(maxsize=1)
def _fd_check_inputs():
    with open(os.path.join(GOLDEN, "fd_equivalence_check.json")) as fh:
        fix = json.load(fh)["what_the_page_fixes"]
    cfg = workloads.custom_config(fix["batch"], fix["heads"], fix["heads"], fix["head_dim"],
                                  fix["seq_len"])
    return fix, workloads.make_inputs(cfg, fix["seed"])


def pin_fd_equivalence_check(lib):
    """The page's own check (§5): B=1, H=32, D=128, S=8192, chunk 512, |split - unsplit| < 1e-5."""
    fix, x = _fd_check_inputs()
    full = lib.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    sp = lib.split_attention(x.q, x.k, x.v, x.seq_lens, x.scale, fix["chunk"])
    err = float(np.max(np.abs(full[0] - sp[0])))
    assert err < fix["max_abs_deviation_bound"], "the page's bound"
    assert err < 1e-13, f"fp64 split deviates by {err:.3e}"
    _close(sp[1], full[1], 1e-12, "fd check lse")


def pin_merge_algebra(lib):
    """Merge: commutative (bitwise), associative, -inf is the identity, merge(s, s) = (o, lse + ln 2)."""
    rng = np.random.default_rng(2)
    R, D = 7, 5
    o = [rng.standard_normal((R, D)) for _ in range(3)]
    s = [rng.standard_normal(R) * 20 for _ in range(3)]
    ab = lib.merge(o[0], s[0], o[1], s[1])
    ba = lib.merge(o[1], s[1], o[0], s[0])
    assert np.array_equal(ab[0], ba[0]) and np.array_equal(ab[1], ba[1]), "commutativity"
    left = lib.merge(ab[0], ab[1], o[2], s[2])
    bc = lib.merge(o[1], s[1], o[2], s[2])
    right = lib.merge(o[0], s[0], bc[0], bc[1])
    _close(left[0], right[0], 1e-13, "associativity out")
    _close(left[1], right[1], 1e-13, "associativity lse")
    ident = lib.merge(o[0], s[0], np.zeros((R, D)), np.full(R, -np.inf))
    _close(ident[0], o[0], 0.0, "identity out")
    _close(ident[1], s[0], 0.0, "identity lse")
    twice = lib.merge(o[0], s[0], o[0], s[0])
    _close(twice[0], o[0], 1e-13, "self-merge out")
    _close(twice[1], s[0] + math.log(2.0), 1e-14, "self-merge lse")
    empty = lib.merge(o[0], np.full(R, -np.inf), o[1], np.full(R, -np.inf))
    assert np.all(empty[0] == 0.0) and np.all(empty[1] == -np.inf)
    # weights: a dominant side wins; closed form of the two-state merge
    w = lib.merge(np.ones((1, 1)), np.array([0.0]), np.zeros((1, 1)), np.array([math.log(3.0)]))
    _close(w[0], [[0.25]], 1e-16, "merge weights 1:3")
    _close(w[1], [math.log(4.0)], 1e-15, "merge lse ln(1+3)")


def pin_merge_of_halves_equals_whole(lib):
    """Attention over rows [0, m) merged with attention over [m, L) equals attention over [0, L)."""
    x = _small(23, B=2, Hq=4, Hkv=2, D=16, smax=30, lens=(30, 21), k_mult=4.0)
    whole = lib.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    for m in (1, 9, 20):
        first = lib.attention(x.q, x.k, x.v, np.minimum(x.seq_lens, m).astype(np.int32), x.scale)
        k2 = np.full_like(x.k, workloads.BF16_QNAN)
        v2 = np.full_like(x.v, workloads.BF16_QNAN)
        k2[:, :, :30 - m] = x.k[:, :, m:]
        v2[:, :, :30 - m] = x.v[:, :, m:]
        second = lib.attention(x.q, k2, v2, np.maximum(x.seq_lens - m, 0).astype(np.int32),
                               x.scale)
        merged = lib.merge(first[0], first[1], second[0], second[1])
        _close(merged[0], whole[0], 1e-13, f"halves at {m}: out")
        _close(merged[1], whole[1], 1e-13, f"halves at {m}: lse")


# cheap pins first, the page-sized equivalence check last
# ---- 8-bit (E4M3) K/V cache: FlashDecoding++ post §4 ----

def _small_fp8(seed, B=2, Hq=4, Hkv=2, D=16, smax=24, lens=(24, 13), k_mult=1.0):
    cfg = workloads.custom_config(B, Hq, Hkv, D, smax, k_mult=k_mult)
    return workloads.make_fp8_inputs(cfg, seed, smax=smax, seq_lens=lens)


def pin_e4m3_decode_matches_torch(lib):
    """All 256 codes decode as torch's own float8_e4m3fn does (an independent implementation)."""
    import torch

    codes = np.arange(256, dtype=np.uint8)
    mine = lib.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref)), "NaN codes differ"
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok]), "E4M3 values differ from torch"
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok])), "signs of zero differ"


def pin_e4m3_special_values(lib):
    """Values the E4M3 format fixes: zeros, smallest subnormal and normal, one,
    the largest finite value 448, the NaN codes, and ordering of the codes."""
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0, 0xFE: -448.0,
             0xB8: -1.0}
    codes = np.array(sorted(table), dtype=np.uint8)
    got = lib.e4m3_decode(codes)
    for c, g in zip(codes, got):
        assert g == table[int(c)], f"code 0x{int(c):02X} -> {g}, want {table[int(c)]}"
    all_vals = lib.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.isnan(all_vals[0x7F]) and np.isnan(all_vals[0xFF]), "0x7F / 0xFF must be NaN"
    assert int(np.isnan(all_vals).sum()) == 2, "exactly two NaN codes, no infinities"
    assert all_vals[0x80] == 0.0 and np.signbit(all_vals[0x80]), "0x80 is -0"
    pos = all_vals[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must increase"
    assert np.array_equal(all_vals[0x80:0xFF], -pos), "sign bit negates"


def pin_fp8_attention_equals_bf16_definition(lib):
    """With these scales every k_scale*e4m3(code) is exact in bfloat16, so the
    8-bit path must agree bitwise with the (pinned) bf16 definition fed the
    dequantised values."""
    x = _small_fp8(21, Hq=8, Hkv=2, D=32, smax=40, lens=(40, 17))
    for mult in (1.0, 4.0):
        if mult != 1.0:
            x = _small_fp8(22, Hq=8, Hkv=2, D=32, smax=40, lens=(40, 17), k_mult=mult)
        kd = lib.e4m3_decode(x.k) * x.k_scale[None, :, None, None].astype(np.float64)
        vd = lib.e4m3_decode(x.v) * x.v_scale[None, :, None, None].astype(np.float64)
        kb, vb = _bits(np.nan_to_num(kd)), _bits(np.nan_to_num(vd))
        assert np.array_equal(_f(kb), np.nan_to_num(kd)) and np.array_equal(_f(vb), np.nan_to_num(vd)), \
            "dequantised values must be exact in bf16 for this pin"
        o8, l8 = lib.attention_fp8(x.q, x.k, x.v, x.k_scale, x.v_scale, x.seq_lens, x.scale)
        ob, lb = lib.attention(x.q, kb, vb, x.seq_lens, x.scale)
        assert np.array_equal(o8, ob) and np.array_equal(l8, lb), f"fp8 vs bf16 definition (k x{mult})"


def pin_fp8_scale_folding(lib):
    """Doubling k_scale is doubling the softmax scale; doubling v_scale doubles
    the output and leaves the LSE alone (all exact scalings by 2)."""
    x = _small_fp8(23)
    o, l = lib.attention_fp8(x.q, x.k, x.v, x.k_scale, x.v_scale, x.seq_lens, x.scale)
    o2, l2 = lib.attention_fp8(x.q, x.k, x.v, x.k_scale * 2, x.v_scale, x.seq_lens, x.scale)
    o3, l3 = lib.attention_fp8(x.q, x.k, x.v, x.k_scale, x.v_scale, x.seq_lens, x.scale * 2)
    assert np.array_equal(o2, o3) and np.array_equal(l2, l3), "k_scale and scale must fold"
    o4, l4 = lib.attention_fp8(x.q, x.k, x.v, x.k_scale, x.v_scale * 2, x.seq_lens, x.scale)
    assert np.array_equal(o4, 2 * o) and np.array_equal(l4, l), "v_scale must scale the output only"
    assert not np.allclose(o2, o), "k_scale must matter"


def pin_fp8_bruteforce_tiny(lib):
    """Non-dyadic per-head scales against a pure-Python textbook softmax with
    math.fsum, the codes decoded by torch."""
    import torch

    x = _small_fp8(24, B=1, Hq=4, Hkv=2, D=8, smax=6, lens=(6,))
    ks = np.array([0.1, 0.3], dtype=np.float32)
    vs = np.array([0.7, 0.05], dtype=np.float32)
    o, l = lib.attention_fp8(x.q, x.k, x.v, ks, vs, x.seq_lens, x.scale)
    dec = lambda c: torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).double().numpy()
    kf, vf, qf = dec(x.k), dec(x.v), _f(x.q)
    for h in range(4):
        g = h // 2
        k_rows = [[float(ks[g]) * kf[0, g, j, d] for d in range(8)] for j in range(6)]
        v_rows = [[float(vs[g]) * vf[0, g, j, d] for d in range(8)] for j in range(6)]
        ro, rl = oracle.attention_fsum_textbook(list(qf[0, h]), k_rows, v_rows, x.scale)
        assert np.allclose(o[0, h], ro, rtol=1e-12, atol=1e-14), f"head {h}"
        assert abs(l[0, h] - rl) <= 1e-12 * max(1.0, abs(rl)), f"lse head {h}"


# ---- 4-bit integer K/V cache: FlashDecoding++ post §4 (INT4 beside FP8) ----

def _small_int4(seed, B=2, Hq=4, Hkv=2, D=16, smax=24, lens=(24, 13), k_mult=1.0):
    cfg = workloads.custom_config(B, Hq, Hkv, D, smax, k_mult=k_mult)
    return workloads.make_int4_inputs(cfg, seed, smax=smax, seq_lens=lens)


def _int4_by_shifts(packed):
    """Sign extension by arithmetic shifts of int8 (an independent route):
    element 2i from the low nibble of byte i, 2i + 1 from the high nibble."""
    b = np.ascontiguousarray(packed, dtype=np.uint8)
    lo = ((b << np.uint8(4)).view(np.int8) >> 4).astype(np.float64)
    hi = (b.view(np.int8) >> 4).astype(np.float64)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.float64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def pin_int4_decode_matches_sign_extension(lib):
    """All 256 bytes decode as int8 arithmetic shifts sign-extend them."""
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    assert np.array_equal(lib.int4_decode(codes), _int4_by_shifts(codes))


def pin_int4_decode_layout(lib):
    """Bytes whose two elements the format fixes: low nibble first, two's complement."""
    table = {0x00: (0, 0), 0x01: (1, 0), 0x10: (0, 1), 0x07: (7, 0), 0x08: (-8, 0),
             0x0F: (-1, 0), 0x70: (0, 7), 0x80: (0, -8), 0xF0: (0, -1), 0x9A: (-6, -7),
             0x7F: (-1, 7), 0xF7: (7, -1)}
    codes = np.array([list(table)], dtype=np.uint8)
    got = lib.int4_decode(codes).reshape(-1, 2)
    for c, g in zip(table, got):
        assert tuple(g) == table[c], f"byte 0x{c:02X} -> {tuple(g)}, want {table[c]}"


def pin_int4_attention_equals_bf16_definition(lib):
    """With power-of-two row scales every scale*int4 value is exact in bfloat16,
    so the 4-bit path must agree bitwise with the (pinned) bf16 definition fed
    the dequantised values; the scales vary by row, head and batch row."""
    x = _small_int4(31, Hq=8, Hkv=2, D=32, smax=40, lens=(40, 17))
    B, Hkv, S = x.k_scale.shape
    j = np.arange(S)[None, None, :]
    ks = np.ldexp(1.0, -(1 + (j + np.arange(Hkv)[None, :, None] + 2 * np.arange(B)[:, None, None]) % 4))
    vs = np.ldexp(1.0, -((3 * j + np.arange(Hkv)[None, :, None] + np.arange(B)[:, None, None]) % 5))
    ks, vs = ks.astype(np.float32), vs.astype(np.float32)
    kd = lib.int4_decode(x.k) * ks[..., None]
    vd = lib.int4_decode(x.v) * vs[..., None]
    kb, vb = _bits(kd), _bits(vd)
    assert np.array_equal(_f(kb), kd) and np.array_equal(_f(vb), vd), "dequantised values must be exact in bf16"
    o4, l4 = lib.attention_int4(x.q, x.k, x.v, ks, vs, x.seq_lens, x.scale)
    ob, lb = lib.attention(x.q, kb, vb, x.seq_lens, x.scale)
    assert np.array_equal(o4, ob) and np.array_equal(l4, lb), "int4 vs bf16 definition"


def pin_int4_scale_folding(lib):
    """Doubling every K scale is doubling the softmax scale; doubling every V
    scale doubles the output and leaves the LSE alone (exact scalings by 2)."""
    x = _small_int4(33)
    o, l = lib.attention_int4(x.q, x.k, x.v, x.k_scale, x.v_scale, x.seq_lens, x.scale)
    o2, l2 = lib.attention_int4(x.q, x.k, x.v, x.k_scale * 2, x.v_scale, x.seq_lens, x.scale)
    o3, l3 = lib.attention_int4(x.q, x.k, x.v, x.k_scale, x.v_scale, x.seq_lens, x.scale * 2)
    assert np.array_equal(o2, o3) and np.array_equal(l2, l3), "k_scale and scale must fold"
    o4, l4 = lib.attention_int4(x.q, x.k, x.v, x.k_scale, x.v_scale * 2, x.seq_lens, x.scale)
    assert np.array_equal(o4, 2 * o) and np.array_equal(l4, l), "v_scale must scale the output only"
    assert not np.allclose(o2, o), "k_scale must matter"


def pin_int4_bruteforce_tiny(lib):
    """The generator's own non-dyadic per-row scales against a pure-Python
    textbook softmax with math.fsum, the codes decoded by int8 shifts."""
    x = _small_int4(34, B=2, Hq=4, Hkv=2, D=8, smax=7, lens=(7, 4))
    o, l = lib.attention_int4(x.q, x.k, x.v, x.k_scale, x.v_scale, x.seq_lens, x.scale)
    kf, vf, qf = _int4_by_shifts(x.k), _int4_by_shifts(x.v), _f(x.q)
    for b in range(2):
        L = int(x.seq_lens[b])
        for h in range(4):
            g = h // 2
            k_rows = [[float(x.k_scale[b, g, j]) * kf[b, g, j, d] for d in range(8)] for j in range(L)]
            v_rows = [[float(x.v_scale[b, g, j]) * vf[b, g, j, d] for d in range(8)] for j in range(L)]
            ro, rl = oracle.attention_fsum_textbook(list(qf[b, h]), k_rows, v_rows, x.scale)
            assert np.allclose(o[b, h], ro, rtol=1e-12, atol=1e-14), f"row {b} head {h}"
            assert abs(l[b, h] - rl) <= 1e-12 * max(1.0, abs(rl)), f"lse row {b} head {h}"


# ---- paged K/V cache: FlashDecoding++ post §6 ----

def pin_paged_gather_inverts_the_generators_scatter(lib):
    """The generator scatters rows into a shuffled page pool with its own code;
    the oracle's gather must give back exactly the contiguous rows (and the
    fill value beyond each sequence), for both pool layouts and several page
    sizes, with spare pages in the pool and in the table."""
    cfg = workloads.custom_config(4, 8, 2, 16, 200)
    for P in (32, 64):
        for layout in (oracle.PAGED_HND, oracle.PAGED_NHD):
            x = workloads.make_paged_inputs(cfg, 31 + P + layout, P, layout, seq_lens=(200, 1, 64, 0))
            smax = x.block_table.shape[1] * P
            for pool, ref in ((x.k_pool, x.base.k), (x.v_pool, x.base.v)):
                got = oracle.gather_paged(pool, x.block_table, x.base.seq_lens, P, layout, smax, 7)
                for b, L in enumerate(x.base.seq_lens):
                    assert np.array_equal(got[b, :, :L], ref[b, :, :L]), f"P={P} layout={layout} b={b}"
                    assert np.all(got[b, :, L:] == 7), "rows past the sequence must be the fill"


def pin_paged_identity_table_is_a_reshape(lib):
    """With block_table[b][i] = b * max_blocks + i, an HND pool is the
    contiguous cache reshaped, and an NHD pool that with rows and heads
    swapped (numpy reshape / transpose)."""
    rng = np.random.default_rng(5)
    B, Hkv, P, nb, D = 2, 3, 32, 4, 8
    cache = rng.integers(0, 1 << 16, size=(B, Hkv, nb * P, D), dtype=np.uint16)
    table = np.arange(B * nb, dtype=np.int32).reshape(B, nb)
    lens = np.array([nb * P, nb * P], dtype=np.int32)
    hnd = cache.reshape(B, Hkv, nb, P, D).transpose(0, 2, 1, 3, 4).reshape(B * nb, Hkv, P, D)
    nhd = hnd.transpose(0, 2, 1, 3)
    assert np.array_equal(oracle.gather_paged(hnd, table, lens, P, oracle.PAGED_HND, nb * P, 0), cache)
    assert np.array_equal(oracle.gather_paged(nhd, table, lens, P, oracle.PAGED_NHD, nb * P, 0), cache)


def pin_paged_attention_equals_contiguous(lib):
    """Attention over the paged cache is bitwise the (pinned) contiguous
    definition over the same rows."""
    cfg = workloads.custom_config(3, 8, 2, 32, 150)
    x = workloads.make_paged_inputs(cfg, 41, 32, oracle.PAGED_NHD, seq_lens=(150, 33, 0))
    o, l = oracle.attention_paged(x.base.q, x.k_pool, x.v_pool, x.block_table, x.base.seq_lens,
                                  32, oracle.PAGED_NHD, x.base.scale, lib=lib)
    ro, rl = lib.attention(x.base.q, x.base.k, x.base.v, x.base.seq_lens, x.base.scale)
    assert np.array_equal(o, ro) and np.array_equal(l, rl)


def pin_paged_int4_gather_inverts_the_generators_scatter(lib):
    """INT4 page pools and their row-scale pools: the gather returns exactly
    the contiguous codes and scales the generator drew (both layouts), 0x88
    and NaN past each sequence, and attention over them is bitwise the
    contiguous INT4 definition."""
    cfg = workloads.custom_config(3, 8, 2, 32, 150)
    for layout in (oracle.PAGED_HND, oracle.PAGED_NHD):
        x = workloads.make_paged_inputs(cfg, 43 + layout, 32, layout, seq_lens=(150, 33, 0),
                                        int4=True)
        k, v, ks, vs = oracle.gather_paged_int4(x)
        b = x.base
        for i, L in enumerate(b.seq_lens):
            assert np.array_equal(k[i, :, :L], b.k[i, :, :L]) and np.array_equal(v[i, :, :L], b.v[i, :, :L])
            assert np.array_equal(ks[i, :, :L], b.k_scale[i, :, :L])
            assert np.array_equal(vs[i, :, :L], b.v_scale[i, :, :L])
            assert np.all(k[i, :, L:] == 0x88) and np.all(np.isnan(vs[i, :, L:]))
        o, l = lib.attention_int4(b.q, k, v, ks, vs, b.seq_lens, b.scale)
        ro, rl = lib.attention_int4(b.q, b.k, b.v, b.k_scale, b.v_scale, b.seq_lens, b.scale)
        assert np.array_equal(o, ro) and np.array_equal(l, rl)


# ---- magnitude form: sum_j w_j |v_j| / Z (the scale of the bf16-output bound) ----

def pin_abs_zero_query_gives_mean_magnitude(lib):
    """q = 0: every weight is 1/L, so the magnitude form is the exact mean of
    |v| over the valid rows, for bf16, E4M3 and INT4 caches (with V scales of
    both signs for the last two)."""
    x = _small(51, lens=(24, 13))
    q0 = np.zeros_like(x.q)
    m = lib.abs_attention(q0, x.k, x.v, x.seq_lens, x.scale)
    # negative V scales on some heads / rows: the magnitude is |scale * value|
    xf = _small_fp8(52)
    xf.v_scale[1::2] *= -1
    mf = lib.abs_attention_fp8(np.zeros_like(xf.q), xf.k, xf.v, xf.k_scale, xf.v_scale,
                               xf.seq_lens, xf.scale)
    xi = _small_int4(53)
    xi.v_scale[:, :, ::2] *= -1
    mi = lib.abs_attention_int4(np.zeros_like(xi.q), xi.k, xi.v, xi.k_scale, xi.v_scale,
                                xi.seq_lens, xi.scale)
    import torch
    dec8 = torch.from_numpy(np.ascontiguousarray(xf.v)).view(torch.float8_e4m3fn).double().numpy()
    dec4 = _int4_by_shifts(xi.v)
    G = x.q.shape[1] // x.k.shape[1]
    for b in range(2):
        for h in range(x.q.shape[1]):
            g = h // G
            L = int(x.seq_lens[b])
            rows = np.abs(_f(x.v[b, g, :L]))
            _close(m[b, h], [math.fsum(rows[:, d]) / L for d in range(rows.shape[1])], 1e-14,
                   "bf16 q=0 mean |v|")
            L = int(xf.seq_lens[b])
            rows = np.abs(float(xf.v_scale[g]) * dec8[b, g, :L])
            _close(mf[b, h], [math.fsum(rows[:, d]) / L for d in range(rows.shape[1])], 1e-14,
                   "E4M3 q=0 mean |v|")
            L = int(xi.seq_lens[b])
            rows = np.abs(xi.v_scale[b, g, :L, None].astype(np.float64) * dec4[b, g, :L])
            _close(mi[b, h], [math.fsum(rows[:, d]) / L for d in range(rows.shape[1])], 1e-14,
                   "INT4 q=0 mean |v|")


def pin_abs_one_signed_values_equal_the_output(lib):
    """When every V element has one sign the magnitude form is |out|: bitwise
    out itself for non-negative V and -out for non-positive V (bf16 sign bits
    cleared or set; E4M3 sign bits cleared; INT4 nibbles limited to 0..7)."""
    x = _small(54, lens=(24, 9))
    pos = x.v & np.uint16(0x7FFF)
    neg = x.v | np.uint16(0x8000)
    o, _ = lib.attention(x.q, x.k, pos, x.seq_lens, x.scale)
    assert np.array_equal(lib.abs_attention(x.q, x.k, pos, x.seq_lens, x.scale), o)
    o, _ = lib.attention(x.q, x.k, neg, x.seq_lens, x.scale)
    assert np.array_equal(lib.abs_attention(x.q, x.k, neg, x.seq_lens, x.scale), -o)
    xf = _small_fp8(55)
    vf = xf.v & np.uint8(0x7F)
    o, _ = lib.attention_fp8(xf.q, xf.k, vf, xf.k_scale, xf.v_scale, xf.seq_lens, xf.scale)
    assert np.array_equal(lib.abs_attention_fp8(xf.q, xf.k, vf, xf.k_scale, xf.v_scale,
                                                xf.seq_lens, xf.scale), o)
    xi = _small_int4(56)
    vi = xi.v & np.uint8(0x77)
    o, _ = lib.attention_int4(xi.q, xi.k, vi, xi.k_scale, xi.v_scale, xi.seq_lens, xi.scale)
    assert np.array_equal(lib.abs_attention_int4(xi.q, xi.k, vi, xi.k_scale, xi.v_scale,
                                                 xi.seq_lens, xi.scale), o)


def pin_abs_bruteforce_tiny(lib):
    """The magnitude form against a pure-Python textbook sum with math.fsum:
    sum_j exp(s_j) |v_j| / sum_j exp(s_j)."""
    x = _small(57, B=2, Hq=4, Hkv=2, D=8, smax=20, lens=(20, 5))
    m = lib.abs_attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    for b, L in enumerate(x.seq_lens):
        for h in range(4):
            g = h // 2
            qv, ks, vs = _f(x.q[b, h]), _f(x.k[b, g, :L]), _f(x.v[b, g, :L])
            e = [math.exp(x.scale * math.fsum(qv * ks[j])) for j in range(L)]
            Z = math.fsum(e)
            want = [math.fsum(e[j] * abs(vs[j, d]) for j in range(L)) / Z for d in range(8)]
            _close(m[b, h], want, 1e-13, f"magnitude brute force b={b} h={h}")


def pin_abs_bounds_the_output(lib):
    """Triangle inequality: |out| <= magnitude everywhere, strictly somewhere
    for random V of both signs; an empty sequence gives 0."""
    x = _small(58, lens=(24, 0))
    o, _ = lib.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    m = lib.abs_attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    assert np.all(np.abs(o) <= m * (1 + 1e-15)), "|out| must not exceed the magnitude"
    assert np.any(np.abs(o[0]) < 0.5 * m[0]), "random signs must cancel somewhere"
    assert np.all(m[1] == 0.0), "an empty sequence has magnitude 0"


ALL_PINS = sorted((v for k, v in globals().items() if k.startswith("pin_") and callable(v)),
                  key=lambda f: (f is pin_fd_equivalence_check, f.__name__))


def run_all(lib_path: str) -> int:
    """Run every pin against one build; print the first failure.  Exit code 1 if any fails."""
    lib = oracle.OracleLib(lib_path)
    for pin in ALL_PINS:
        try:
            pin(lib)
        except AssertionError as e:
            print(f"CAUGHT {pin.__name__}: {e}", flush=True)
            return 1
    print("ALL PINS PASS", flush=True)
    return 0


if __name__ == "__main__":
    import sys

    sys.exit(run_all(sys.argv[1]))
