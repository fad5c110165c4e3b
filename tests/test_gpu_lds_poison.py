"""The debug build (libdas_debug.so, compiled with DAS_DEBUG_LDS_POISON=1):
every wave's LDS tile region starts as 0xFF bytes (NaN as bf16, E4M3 and
fp32) and is filled with them again after each tile the wave has finished
reading, and the per-wave statistics slots start as NaN.  A read of LDS that
is not ordered after the write it needs (a missing wait for a load that
writes LDS directly, a missing barrier before the cross-wave merge) then
returns NaN instead of plausible stale values.

Over every kernel variant (bf16, E4M3 and INT4 caches, contiguous and paged,
G = 1 ... 16, D = 64 and 128, one split, fused merge and the separate merge
kernel), the debug build must give finite results bit-for-bit equal to the
regular build's, which the other GPU tests check against the fp64 oracle.
Each case runs twice on the debug build (the second time over LDS left by the
first)."""
import numpy as np
import pytest
import torch

import decode_attention_split_amd as das
import workloads
from gpu_helpers import dev, note, to_dev

pytestmark = pytest.mark.gpu

HND, NHD = workloads.PAGED_HND, workloads.PAGED_NHD


@pytest.fixture(scope="module")
def debug_lib():
    return das.open_library(das.DEBUG_LIB_PATH)


def _decode_call(kind, x):
    """(prepare(out, lse, ws, splits) -> PreparedCall, B, Hq, D, workspace
    bytes(splits)) for a contiguous cache of `kind`."""
    d = dev()
    if kind == "bf16":
        q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
        ks = vs = None
        name = "das_decode_attention"
    else:
        q = to_dev(x.q)
        k, v = torch.from_numpy(x.k).to(d), torch.from_numpy(x.v).to(d)
        ks, vs = torch.from_numpy(x.k_scale).to(d), torch.from_numpy(x.v_scale).to(d)
        name = "das_decode_attention_fp8" if kind == "fp8" else "das_decode_attention_int4"
    sl = torch.from_numpy(x.seq_lens).to(d)
    B, Hq, D = x.q.shape
    Hkv, Smax = x.k.shape[1], x.k.shape[2]

    def prepare(out, lse, ws, splits):
        return das.prepare_decode(name, q, k, v, sl, x.scale, out, lse, splits, ws,
                                  k_scale=ks, v_scale=vs)

    return prepare, B, Hq, D, lambda ns: das.das_decode_workspace_bytes(B, Hq, Hkv, Smax, D, ns)


def _paged_call(x):
    d = dev()
    if x.k_pool.dtype == np.uint16:
        kp, vp = to_dev(x.k_pool), to_dev(x.v_pool)
        ks = vs = None
        kv = das.DAS_BF16
    else:
        kp, vp = torch.from_numpy(x.k_pool).to(d), torch.from_numpy(x.v_pool).to(d)
        ks, vs = torch.from_numpy(x.k_scale_pool).to(d), torch.from_numpy(x.v_scale_pool).to(d)
        kv = das.DAS_INT4
    q = to_dev(x.base.q)
    bt = torch.from_numpy(x.block_table).to(d)
    sl = torch.from_numpy(x.base.seq_lens).to(d)
    B, Hq, D = x.base.q.shape
    Hkv = x.base.k.shape[1]
    smax = x.block_table.shape[1] * x.page_size

    def prepare(out, lse, ws, splits):
        return das.prepare_decode_paged(q, kp, vp, bt, sl, x.base.scale, x.page_size, x.layout,
                                        out, lse, splits, ws, k_scale=ks, v_scale=vs,
                                        kv_dtype=kv)

    return prepare, B, Hq, D, lambda ns: das.das_decode_workspace_bytes(B, Hq, Hkv, smax, D, ns)


def _compare(what, prepare, B, Hq, D, ws_bytes, splits, debug_lib, out_dtype=torch.float32):
    d = dev()
    results = []
    for lib in (None, debug_lib, debug_lib):
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=d)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=d)
        ws = torch.zeros(max(ws_bytes(splits), 16), dtype=torch.uint8, device=d)
        call = prepare(out, lse, ws, splits)
        (call if lib is None else call.on_library(lib))()
        results.append((out, lse))
    torch.cuda.synchronize()
    (ro, rl), *dbg = results
    for i, (o, l) in enumerate(dbg):
        assert not torch.isnan(o.float()).any(), f"{what}: NaN output from the debug build (run {i})"
        assert not torch.isnan(l).any(), f"{what}: NaN LSE from the debug build (run {i})"
        assert torch.equal(o, ro), f"{what}: debug build output differs (run {i})"
        assert torch.equal(l, rl), f"{what}: debug build LSE differs (run {i})"
    note(f"  {what}: debug build bit-for-bit equal, finite")


CONTIGUOUS = [
    # kind, (B, Hq, Hkv, D, Smax), seq_lens, forced splits (0 = automatic)
    ("bf16", (2, 8, 8, 64, 700), (700, 1), 0),
    ("bf16", (2, 8, 4, 128, 900), (900, 333), 5),
    ("bf16", (3, 16, 4, 128, 2000), (2000, 0, 1500), 0),
    ("bf16", (1, 16, 2, 64, 600), (600,), 1),
    ("bf16", (2, 32, 4, 128, 1300), (1300, 95), 0),
    ("bf16", (2, 32, 2, 128, 1500), (1500, 31), 3),
    ("fp8", (2, 8, 8, 128, 800), (800, 77), 0),
    ("fp8", (2, 16, 4, 64, 1000), (1000, 513), 0),
    ("fp8", (1, 32, 2, 128, 900), (900,), 2),
    ("int4", (2, 8, 4, 128, 1000), (1000, 3), 0),
    ("int4", (2, 16, 4, 64, 1200), (1200, 640), 0),
    ("int4", (1, 32, 2, 128, 1100), (1100,), 4),
    ("int4", (2, 8, 8, 64, 500), (500, 250), 1),
]


@pytest.mark.parametrize("kind,shape,lens,splits", CONTIGUOUS,
                         ids=[f"{c[0]}-G{c[1][1] // c[1][2]}-D{c[1][3]}-ns{c[3]}"
                              for c in CONTIGUOUS])
def test_debug_build_matches_regular_build(kind, shape, lens, splits, debug_lib):
    B, Hq, Hkv, D, smax = shape
    cfg = workloads.custom_config(B, Hq, Hkv, D, smax, k_mult=2.0)
    seed = 9000 + 7 * D + Hq // Hkv + splits
    make = {"bf16": workloads.make_inputs, "fp8": workloads.make_fp8_inputs,
            "int4": workloads.make_int4_inputs}[kind]
    x = make(cfg, seed, seq_lens=lens)
    note(f"case lds-poison {kind} shape={shape} lens={lens} splits={splits}")
    prepare, B, Hq, D, ws = _decode_call(kind, x)
    _compare(f"{kind} {shape} ns={splits}", prepare, B, Hq, D, ws, splits, debug_lib)
    if kind == "bf16":
        _compare(f"{kind} {shape} ns={splits} bf16 out", prepare, B, Hq, D, ws, splits,
                 debug_lib, torch.bfloat16)


def test_debug_build_on_the_separate_merge_kernel(debug_lib):
    """A grid of more than 4 split workgroups per CU: phase 2 runs as its own
    kernel (B = 64 varlen decode, lengths as the named varlen config draws
    them but at most 2,048 rows)."""
    cfg = workloads.custom_config(64, 32, 8, 128, 2048)
    rng = np.random.Generator(np.random.PCG64(9100))
    lens = rng.integers(64, 2048, size=64, endpoint=True)
    x = workloads.make_inputs(cfg, 9101, seq_lens=lens)
    note("case lds-poison bf16 B=64 varlen, separate merge kernel")
    prepare, B, Hq, D, ws = _decode_call("bf16", x)
    ns, _ = das.das_plan(B, 8, 4, 2048, 128, 0)
    assert 64 * 8 * ns > 4 * torch.cuda.get_device_properties(0).multi_processor_count
    _compare("bf16 B=64 varlen", prepare, B, Hq, D, ws, 0, debug_lib)


@pytest.mark.parametrize("kind,P,layout,G", [("bf16", 32, HND, 4), ("bf16", 64, NHD, 1),
                                             ("int4", 64, HND, 8), ("int4", 32, NHD, 2)],
                         ids=["bf16-P32-HND-G4", "bf16-P64-NHD-G1", "int4-P64-HND-G8",
                              "int4-P32-NHD-G2"])
def test_debug_build_matches_regular_build_paged(kind, P, layout, G, debug_lib):
    cfg = workloads.custom_config(3, 2 * G, 2, 128, 1000, k_mult=2.0)
    x = workloads.make_paged_inputs(cfg, 9200 + P + G, P, layout, seq_lens=(1000, 777, 33),
                                    int4=kind == "int4")
    note(f"case lds-poison paged {kind} P={P} layout={layout} G={G}")
    prepare, B, Hq, D, ws = _paged_call(x)
    for splits in (0, 3):
        _compare(f"paged {kind} P={P} G={G} ns={splits}", prepare, B, Hq, D, ws, splits,
                 debug_lib)
