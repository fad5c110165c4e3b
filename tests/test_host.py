"""Host-side logic of the C ABI, on the CPU: exported symbols, argument
checks (nothing is launched when a check fails) and the split plan."""
import ctypes
import math
import os
import subprocess

import pytest

import decode_attention_split_amd as das

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "das.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(das.LIB_PATH):
        from decode_attention_split_amd import build
        build.build()
    return das.load_library()


def _header_functions():
    import re
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(das_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol(lib):
    declared = _header_functions()
    assert set(declared) == set(das.EXPORTED)
    nm = subprocess.run(["nm", "-D", "--defined-only", das.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = {line.split()[-1] for line in nm.splitlines() if " T " in line}
    for name in declared:
        assert name in exported, f"{name} declared in das.h but not exported"
        getattr(lib, name)


def test_debug_build_exports_the_same_symbols(lib):
    """libdas_debug.so (the LDS-poisoning debug build, made by the same
    build step) loads and exports every declared entry point too."""
    declared = _header_functions()
    dbg = das.open_library(das.DEBUG_LIB_PATH)
    nm = subprocess.run(["nm", "-D", "--defined-only", das.DEBUG_LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = {line.split()[-1] for line in nm.splitlines() if " T " in line}
    for name in declared:
        assert name in exported, f"{name} not exported by the debug build"
        getattr(dbg, name)
    assert das.load_library() is lib   # opening another build leaves the loaded one in place


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4):
        assert das.das_strerror(code)
    assert "unknown" in das.das_strerror(7)


def plan(B, Hkv, G, Smax, D, ns=0, cus=256):
    return das.das_plan(B, Hkv, G, Smax, D, ns, cus)


@pytest.mark.parametrize("B,Hkv,G,Smax,D", [
    (1, 8, 8, 1024, 64), (1, 8, 4, 32768, 128), (1, 8, 4, 131072, 128),
    (64, 8, 4, 16384, 128), (8, 8, 8, 100003, 128), (3, 2, 1, 1, 64), (1, 1, 2, 5000000, 128)])
def test_auto_plan_covers_the_sequence(B, Hkv, G, Smax, D):
    ns, chunk = plan(B, Hkv, G, Smax, D)
    assert chunk % das.DAS_CHUNK_QUANTUM == 0
    assert 1 <= ns <= das.DAS_MAX_SPLITS
    assert (ns - 1) * chunk < Smax <= ns * chunk       # every row in exactly one split
    if ns > 1:                                          # partial traffic floor
        assert chunk >= (512 if G == 8 else 256)


def test_auto_plan_fills_the_chip_for_long_single_sequences():
    ns, chunk = plan(1, 8, 4, 32768, 128)
    assert 8 * ns >= 3 * 256 // 4                       # about three workgroups per four CUs
    ns2, _ = plan(1, 8, 4, 131072, 128)
    assert 8 * ns2 >= 3 * 256 // 4


def test_forced_splits():
    for n in (1, 2, 3, 7, 64, 300):
        ns, chunk = plan(1, 8, 4, 32768, 128, ns=n)
        assert ns <= n and chunk % das.DAS_CHUNK_QUANTUM == 0
        assert (ns - 1) * chunk < 32768 <= ns * chunk
        assert chunk == math.ceil(math.ceil(32768 / n) / 128) * 128
    assert plan(1, 8, 4, 32768, 128, ns=1) == (1, 32768)


@pytest.mark.parametrize("args,status", [
    ((1, 8, 3, 1024, 128), das.DAS_ENOTSUP),      # G = 3
    ((1, 8, 4, 1024, 96), das.DAS_ENOTSUP),       # D = 96
    ((0, 8, 4, 1024, 128), das.DAS_EINVAL),
    ((1, 0, 4, 1024, 128), das.DAS_EINVAL),
    ((1, 8, 4, 0, 128), das.DAS_EINVAL),
    ((70000, 8, 4, 1024, 128), das.DAS_EINVAL),
])
def test_plan_rejects(args, status):
    with pytest.raises(das.DasError) as e:
        das.das_plan(*args, 0, 256)
    assert e.value.status == status


def test_plan_rejects_too_many_splits():
    with pytest.raises(das.DasError):
        das.das_plan(1, 8, 4, 1 << 20, 128, das.DAS_MAX_SPLITS + 1, 256)


def test_workspace_bytes(lib):
    B, Hq, Hkv, Smax, D = 64, 32, 8, 16384, 128
    ns, chunk = plan(B, Hkv, Hq // Hkv, Smax, D)
    n = das.das_decode_workspace_bytes(B, Hq, Hkv, Smax, D, 0, 256)
    o_end = das.DAS_WORKSPACE_COUNTER_BYTES + B * Hq * ns * D * 4
    assert n == ((o_end + 255) // 256) * 256 + B * Hq * ns * 2 * 4
    assert das.das_decode_workspace_bytes(1, 8, 8, 1024, 64, 1, 256) == 0   # one split: none
    with pytest.raises(das.DasError):
        das.das_decode_workspace_bytes(1, 6, 4, 1024, 64, 0, 256)           # Hq % Hkv


def test_plan_kv_int4_fills_every_cu_and_the_workspace_covers_it():
    # bf16 and E4M3 share das_plan's plan; INT4 aims for one workgroup per CU
    for shape in ((1, 8, 4, 32768, 128), (1, 8, 4, 131072, 128), (64, 8, 4, 16384, 128),
                  (8, 8, 8, 100003, 128), (1, 8, 1, 1024, 64)):
        base = plan(*shape)
        assert das.das_plan_kv(das.DAS_BF16, *shape, 0, 256) == base
        assert das.das_plan_kv(das.DAS_E4M3, *shape, 0, 256) == base
    assert das.das_plan_kv(das.DAS_INT4, 1, 8, 4, 32768, 128, 0, 256) == (32, 1024)
    assert das.das_plan_kv(das.DAS_INT4, 1, 8, 4, 131072, 128, 0, 256) == (32, 4096)
    # a batch that already fills the chip keeps its plan
    assert das.das_plan_kv(das.DAS_INT4, 64, 8, 4, 16384, 128, 0, 256) == plan(64, 8, 4, 16384, 128)
    # forced splits: the same plan for every format
    assert das.das_plan_kv(das.DAS_INT4, 1, 8, 4, 32768, 128, 7, 256) == \
        das.das_plan(1, 8, 4, 32768, 128, 7, 256)
    for Hq, Hkv, S, D in ((32, 8, 32768, 128), (32, 8, 131072, 128), (8, 8, 1024, 64)):
        need = das.das_decode_workspace_bytes(1, Hq, Hkv, S, D, 0, 256)
        for code in (das.DAS_BF16, das.DAS_INT4):
            ns, _ = das.das_plan_kv(code, 1, Hkv, Hq // Hkv, S, D, 0, 256)
            assert ns <= 1 or need >= das.DAS_WORKSPACE_COUNTER_BYTES + Hq * ns * (D + 2) * 4
    with pytest.raises(das.DasError):
        das.das_plan_kv(das.DAS_F32, 1, 8, 4, 1024, 128, 0, 256)


def _call_decode(lib, **kw):
    a = dict(q=16, k=16, v=16, sl=16, B=1, Hq=8, Hkv=2, Smax=1024, D=128, scale=0.1, out=16,
             dt=0, lse=0, ns=4, ws=16, wsb=1 << 30, st=None)
    a.update(kw)
    P = lambda x: ctypes.c_void_p(x) if x else None
    return lib.das_decode_attention(P(a["q"]), P(a["k"]), P(a["v"]), P(a["sl"]), a["B"], a["Hq"],
                                    a["Hkv"], a["Smax"], a["D"], a["scale"], P(a["out"]), a["dt"],
                                    P(a["lse"]), a["ns"], P(a["ws"]), a["wsb"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), das.DAS_EINVAL), (dict(k=0), das.DAS_EINVAL), (dict(v=0), das.DAS_EINVAL),
    (dict(sl=0), das.DAS_EINVAL), (dict(out=0), das.DAS_EINVAL),
    (dict(Hq=6, Hkv=4), das.DAS_EINVAL), (dict(Hq=6, Hkv=2), das.DAS_ENOTSUP),
    (dict(D=80), das.DAS_ENOTSUP), (dict(dt=5), das.DAS_EINVAL), (dict(B=0), das.DAS_EINVAL),
    (dict(Smax=0), das.DAS_EINVAL), (dict(ns=-1), das.DAS_EINVAL),
    (dict(scale=float("nan")), das.DAS_EINVAL), (dict(q=24), das.DAS_EINVAL),
    (dict(ws=0), das.DAS_EWORKSPACE), (dict(wsb=100), das.DAS_EWORKSPACE),
    (dict(ns=das.DAS_MAX_SPLITS + 1), das.DAS_EINVAL),
    (dict(Smax=(1 << 23)), das.DAS_ENOTSUP),        # 32-bit row offsets per sequence
])
def test_decode_argument_checks(lib, kw, status):
    # All pointers are fake: a failed check must return before any launch.
    assert _call_decode(lib, **kw) == status


def _call_decode_fp8(lib, **kw):
    a = dict(q=16, k=16, v=16, ks=16, vs=16, sl=16, B=1, Hq=8, Hkv=2, Smax=1024, D=128, scale=0.1,
             out=16, dt=0, lse=0, ns=4, ws=16, wsb=1 << 30, st=None)
    a.update(kw)
    P = lambda x: ctypes.c_void_p(x) if x else None
    return lib.das_decode_attention_fp8(P(a["q"]), P(a["k"]), P(a["v"]), P(a["ks"]), P(a["vs"]),
                                        P(a["sl"]), a["B"], a["Hq"], a["Hkv"], a["Smax"], a["D"],
                                        a["scale"], P(a["out"]), a["dt"], P(a["lse"]), a["ns"],
                                        P(a["ws"]), a["wsb"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(ks=0), das.DAS_EINVAL), (dict(vs=0), das.DAS_EINVAL),
    (dict(q=0), das.DAS_EINVAL), (dict(k=0), das.DAS_EINVAL), (dict(v=8), das.DAS_EINVAL),
    (dict(Hq=6, Hkv=2), das.DAS_ENOTSUP), (dict(D=80), das.DAS_ENOTSUP),
    (dict(ws=0), das.DAS_EWORKSPACE),
    (dict(Smax=(1 << 24)), das.DAS_ENOTSUP),        # 32-bit row offsets: (Smax+256)*D >= 2^31
])
def test_decode_fp8_argument_checks(lib, kw, status):
    # All pointers are fake: a failed check must return before any launch.
    assert _call_decode_fp8(lib, **kw) == status
    if "ks" not in kw and "vs" not in kw:   # the same checks as the bf16 entry point
        assert _call_decode(lib, **kw) == status


def test_fp8_row_bound_is_twice_the_bf16_one(lib):
    # (Smax + 256) * D * bytes per element < 2^31: 1-byte codes allow twice the
    # rows.  Both calls fail a check (no launch): the bf16 one on the row
    # bound, the fp8 one only later, on the missing workspace.
    smax = 1 << 23
    assert _call_decode(lib, Smax=smax, ws=0) == das.DAS_ENOTSUP
    assert _call_decode_fp8(lib, Smax=smax, ws=0) == das.DAS_EWORKSPACE


def _call_decode_int4(lib, **kw):
    a = dict(q=16, k=16, v=16, ks=16, vs=16, sl=16, B=1, Hq=8, Hkv=2, Smax=1024, D=128, scale=0.1,
             out=16, dt=0, lse=0, ns=4, ws=16, wsb=1 << 30, st=None)
    a.update(kw)
    P = lambda x: ctypes.c_void_p(x) if x else None
    return lib.das_decode_attention_int4(P(a["q"]), P(a["k"]), P(a["v"]), P(a["ks"]), P(a["vs"]),
                                         P(a["sl"]), a["B"], a["Hq"], a["Hkv"], a["Smax"], a["D"],
                                         a["scale"], P(a["out"]), a["dt"], P(a["lse"]), a["ns"],
                                         P(a["ws"]), a["wsb"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(ks=0), das.DAS_EINVAL), (dict(vs=0), das.DAS_EINVAL),
    (dict(ks=18), das.DAS_EINVAL), (dict(vs=17), das.DAS_EINVAL),      # scales 4-byte aligned
    (dict(q=0), das.DAS_EINVAL), (dict(k=0), das.DAS_EINVAL), (dict(v=8), das.DAS_EINVAL),
    (dict(Hq=6, Hkv=2), das.DAS_ENOTSUP), (dict(D=80), das.DAS_ENOTSUP),
    (dict(ws=0), das.DAS_EWORKSPACE),
    (dict(Smax=(1 << 25)), das.DAS_ENOTSUP),        # 32-bit row offsets: (Smax+256)*D/2 >= 2^31
])
def test_decode_int4_argument_checks(lib, kw, status):
    # All pointers are fake: a failed check must return before any launch.
    assert _call_decode_int4(lib, **kw) == status


def test_int4_row_bound_is_four_times_the_bf16_one(lib):
    # D/2-byte rows allow four times the bf16 rows before the 32-bit offsets
    # run out; the int4 call then fails only on the missing workspace.
    smax = 1 << 24
    assert _call_decode_fp8(lib, Smax=smax, ws=0) == das.DAS_ENOTSUP
    assert _call_decode_int4(lib, Smax=smax, ws=0) == das.DAS_EWORKSPACE


@pytest.mark.parametrize("kw,status", [
    (dict(ks=0), das.DAS_EINVAL), (dict(vs=0), das.DAS_EINVAL),       # INT4 needs scale pools
    (dict(ks=18), das.DAS_EINVAL), (dict(vs=2), das.DAS_EINVAL),      # misaligned scale pools
    (dict(ws=0), das.DAS_EWORKSPACE),                                 # checks pass up to here
])
def test_paged_int4_argument_checks(lib, kw, status):
    """A paged INT4 cache takes row-scale pools: missing or misaligned ones
    are refused before anything is launched (fake pointers)."""
    a = dict(kvt=das.DAS_INT4, ks=16, vs=16)
    a.update(kw)
    assert _call_paged(lib, **a) == status


def test_merge_argument_checks(lib):
    P = ctypes.c_void_p
    f = lib.das_merge_attn_states
    assert f(P(16), P(16), P(16), P(16), P(16), P(16), -1, 128, 0, None) == das.DAS_EINVAL
    assert f(P(16), P(16), P(16), P(16), P(16), P(16), 4, 96, 0, None) == das.DAS_ENOTSUP
    assert f(P(16), P(16), P(16), P(16), P(16), P(16), 4, 128, 9, None) == das.DAS_EINVAL
    assert f(None, P(16), P(16), P(16), P(16), P(16), 4, 128, 0, None) == das.DAS_EINVAL
    assert f(P(8), P(16), P(16), P(16), P(16), P(16), 4, 128, 0, None) == das.DAS_EINVAL
    assert f(None, None, None, None, None, None, 0, 128, 0, None) == das.DAS_OK  # empty


@pytest.mark.parametrize("bad", ["o_short", "o_dtype", "o_strided", "lse_short", "lse_dtype"])
def test_merge_binding_rejects_mismatched_outputs(bad):
    """Caller-supplied merge outputs must have the inputs' shape and dtype (the
    kernel writes rows * D elements of o_a's dtype and rows floats): a smaller
    or differently typed buffer is refused before anything is launched."""
    import torch

    o = torch.zeros(6, 128)
    lse = torch.zeros(6)
    outs = {"o_short": (torch.zeros(5, 128), None),
            "o_dtype": (torch.zeros(6, 128, dtype=torch.bfloat16), None),
            "o_strided": (torch.zeros(128, 6).t(), None),
            "lse_short": (None, torch.zeros(5)),
            "lse_dtype": (None, torch.zeros(6, dtype=torch.float64))}[bad]
    with pytest.raises(ValueError, match="o_out|lse_out"):
        das.das_merge_attn_states(o, lse, o.clone(), lse.clone(), o_out=outs[0], lse_out=outs[1])


def test_binding_constants_match_the_header():
    import re
    text = open(os.path.join(ROOT, "include", "das.h")).read()
    found = dict(re.findall(r"\b(DAS_[A-Z0-9_]+)\s*=\s*(-?\d+)", text))
    found.update({k: v for k, v in re.findall(r"#define\s+(DAS_[A-Z0-9_]+)\s+(\d+)\b", text)})
    assert found, "no constants parsed"
    for name, value in found.items():
        assert hasattr(das, name), f"binding lacks {name}"
        assert getattr(das, name) == int(value), f"{name}: binding {getattr(das, name)} != header {value}"


def _call_paged(lib, **kw):
    a = dict(q=16, k=16, v=16, kvt=das.DAS_BF16, ks=0, vs=0, bt=16, mb=64, P=64, npg=100,
             lay=das.DAS_PAGED_HND, sl=16, B=1, Hq=8, Hkv=2, D=128, scale=0.1, out=16, dt=0,
             lse=0, ns=4, ws=16, wsb=1 << 30, st=None)
    a.update(kw)
    P = lambda x: ctypes.c_void_p(x) if x else None
    return lib.das_decode_attention_paged(
        P(a["q"]), P(a["k"]), P(a["v"]), a["kvt"], P(a["ks"]), P(a["vs"]), P(a["bt"]), a["mb"],
        a["P"], a["npg"], a["lay"], P(a["sl"]), a["B"], a["Hq"], a["Hkv"], a["D"], a["scale"],
        P(a["out"]), a["dt"], P(a["lse"]), a["ns"], P(a["ws"]), a["wsb"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(bt=0), das.DAS_EINVAL), (dict(bt=18), das.DAS_EINVAL),        # null / misaligned table
    (dict(kvt=das.DAS_F32), das.DAS_EINVAL), (dict(kvt=7), das.DAS_EINVAL),
    (dict(kvt=das.DAS_E4M3), das.DAS_EINVAL),                             # E4M3 without scales
    (dict(lay=2), das.DAS_EINVAL), (dict(mb=0), das.DAS_EINVAL), (dict(npg=0), das.DAS_EINVAL),
    (dict(P=16), das.DAS_ENOTSUP), (dict(P=48), das.DAS_ENOTSUP), (dict(P=1 << 17), das.DAS_ENOTSUP),
    (dict(q=0), das.DAS_EINVAL), (dict(k=8), das.DAS_EINVAL), (dict(D=80), das.DAS_ENOTSUP),
    (dict(ws=0), das.DAS_EWORKSPACE), (dict(wsb=100), das.DAS_EWORKSPACE),
    (dict(mb=1 << 26, P=64), das.DAS_EINVAL),                            # max_blocks * P >= 2^31
    (dict(P=65536, Hq=128, Hkv=128, lay=das.DAS_PAGED_NHD), das.DAS_ENOTSUP),  # page >= 2^31 bytes
])
def test_paged_argument_checks(lib, kw, status):
    # All pointers are fake: a failed check must return before any launch.
    assert _call_paged(lib, **kw) == status


def test_group_of_16_plans_for_every_cache_format():
    # G = 16 (e.g. Hq = 128, Hkv = 8): every cache format plans with chunks of
    # at least 1024 rows; bf16 and E4M3 share the plan, INT4 aims for every CU
    ns, chunk = plan(1, 8, 16, 32768, 128)
    assert chunk >= 1024 and (ns - 1) * chunk < 32768 <= ns * chunk
    assert das.das_plan_kv(das.DAS_E4M3, 1, 8, 16, 32768, 128, 0, 256) == (ns, chunk)
    ns4, chunk4 = das.das_plan_kv(das.DAS_INT4, 1, 8, 16, 32768, 128, 0, 256)
    assert chunk4 >= 1024 and (ns4 - 1) * chunk4 < 32768 <= ns4 * chunk4 and ns4 >= ns
    with pytest.raises(das.DasError) as e:
        das.das_plan(1, 8, 32, 32768, 128, 0, 256)          # G = 32
    assert e.value.status == das.DAS_ENOTSUP
