"""Paged K/V cache (FlashDecoding++ post, §6): das_decode_attention_paged vs the
fp64 oracle over the gathered rows, element by element, on seeded inputs
scattered into shuffled page pools with spare NaN pages (bf16, E4M3 and INT4
pools; INT4 with row-scale pools laid out like the code pools).  Same tolerances as
the contiguous cache (fp32 output max|err| <= 5e-4, LSE max|err| <= 1e-4)."""
import numpy as np
import pytest
import torch

import decode_attention_split_amd as das
import oracle
import workloads
from gpu_helpers import check_bf16, check_f32, dev, note, run, to_dev, upload

pytestmark = pytest.mark.gpu

HND, NHD = workloads.PAGED_HND, workloads.PAGED_NHD


def upload_paged(x: workloads.PagedInputs):
    d = dev()
    if x.k_pool.dtype == np.uint16:
        kp, vp = to_dev(x.k_pool), to_dev(x.v_pool)
        ks = vs = None
    elif x.k_scale_pool is not None:      # INT4: row-scale pools
        kp, vp = torch.from_numpy(x.k_pool).to(d), torch.from_numpy(x.v_pool).to(d)
        ks, vs = torch.from_numpy(x.k_scale_pool).to(d), torch.from_numpy(x.v_scale_pool).to(d)
    else:
        kp, vp = torch.from_numpy(x.k_pool).to(d), torch.from_numpy(x.v_pool).to(d)
        ks, vs = torch.from_numpy(x.base.k_scale).to(d), torch.from_numpy(x.base.v_scale).to(d)
    return (to_dev(x.base.q), kp, vp, torch.from_numpy(x.block_table).to(d),
            torch.from_numpy(x.base.seq_lens).to(d), ks, vs)


def run_paged(x, num_splits=0, out_dtype=torch.float32, tensors=None):
    q, kp, vp, bt, sl, ks, vs = tensors if tensors is not None else upload_paged(x)
    out, lse = das.das_decode_attention_paged(
        q, kp, vp, bt, sl, x.base.scale, x.page_size, x.layout, k_scale=ks, v_scale=vs,
        out_dtype=out_dtype, num_splits=num_splits,
        kv_dtype=das.DAS_INT4 if x.k_scale_pool is not None else None)
    torch.cuda.synchronize()
    return out, lse


def ref_paged(x):
    if x.k_scale_pool is not None:
        k, v, ks, vs = oracle.gather_paged_int4(x)
        return oracle.attention_int4(x.base.q, k, v, ks, vs, x.base.seq_lens, x.base.scale)
    if x.k_pool.dtype == np.uint16:
        return oracle.attention_paged(x.base.q, x.k_pool, x.v_pool, x.block_table,
                                      x.base.seq_lens, x.page_size, x.layout, x.base.scale)
    smax = x.block_table.shape[1] * x.page_size
    k = oracle.gather_paged(x.k_pool, x.block_table, x.base.seq_lens, x.page_size, x.layout, smax, 0x7F)
    v = oracle.gather_paged(x.v_pool, x.block_table, x.base.seq_lens, x.page_size, x.layout, smax, 0x7F)
    return oracle.attention_fp8(x.base.q, k, v, x.base.k_scale, x.base.v_scale, x.base.seq_lens,
                                x.base.scale)


@pytest.mark.parametrize("layout", [HND, NHD], ids=["HND", "NHD"])
@pytest.mark.parametrize("D,G", [(D, G) for D in (64, 128) for G in (1, 2, 4, 8, 16)],
                         ids=lambda v: str(v))
def test_paged_small_shapes(D, G, layout):
    """Every (D, G), both pool layouts, two page sizes, several split counts."""
    cfg = workloads.custom_config(3, 2 * G, 2, D, 1000, k_mult=2.0)
    for P in (32, 256):
        x = workloads.make_paged_inputs(cfg, 8000 + 10 * D + G + P, P, layout, seq_lens=(1000, 777, 33))
        ref = ref_paged(x)
        t = upload_paged(x)
        for ns in (0, 1, 3, 7):
            note(f"case paged D={D} G={G} P={P} layout={layout} num_splits={ns}")
            out, lse = run_paged(x, ns, tensors=t)
            check_f32(out, lse, *ref, f"paged D={D} G={G} P={P} L{layout} ns={ns}")


@pytest.mark.parametrize("layout", [HND, NHD], ids=["HND", "NHD"])
@pytest.mark.parametrize("G,fmt", [(4, "bf16"), (1, "bf16"), (2, "int4"), (8, "int4")],
                         ids=["G4-bf16", "G1-bf16", "G2-int4", "G8-int4"])
def test_paged_long_splits_read_the_table_in_rounds(G, fmt, layout):
    """A wave keeps the block-table entries of its pages in one register,
    64 at a time: with 32-row pages and one split over 20,000 rows a wave
    passes 79 pages, so the entries are loaded in two rounds (two splits: 40
    pages, one round)."""
    cfg = workloads.custom_config(2, 2 * G, 2, 128, 20000, k_mult=2.0)
    x = workloads.make_paged_inputs(cfg, 8300 + G + layout, 32, layout, seq_lens=(20000, 16700),
                                    int4=fmt == "int4")
    ref = ref_paged(x)
    t = upload_paged(x)
    for ns in (1, 2):
        note(f"case paged long split G={G} {fmt} layout={layout} num_splits={ns}")
        out, lse = run_paged(x, ns, tensors=t)
        check_f32(out, lse, *ref, f"paged long G={G} {fmt} L{layout} ns={ns}")


@pytest.mark.parametrize("layout", [HND, NHD], ids=["HND", "NHD"])
def test_paged_single_split_equals_contiguous_bitwise(layout):
    """With one split, the paged call streams the same rows in the same order
    as the contiguous call: bitwise the same result."""
    cfg = workloads.custom_config(2, 32, 8, 128, 3000)
    x = workloads.make_paged_inputs(cfg, 8100 + layout, 64, layout, seq_lens=(3000, 1234))
    out_p, lse_p = run_paged(x, 1)
    out_c, lse_c = run(x.base, 1)
    assert torch.equal(out_p, out_c) and torch.equal(lse_p, lse_c)


@pytest.mark.parametrize("P", [32, 64, 128])
def test_paged_edge_lengths(P):
    """Partial last pages, a page boundary either side, L = 0 and L = 1."""
    lens = (0, 1, P - 1, P, P + 1, 2 * P - 1, 2 * P, 2 * P + 1, 5 * P + 3)
    cfg = workloads.custom_config(len(lens), 8, 2, 128, 5 * P + 3)
    x = workloads.make_paged_inputs(cfg, 8200 + P, P, NHD, seq_lens=lens)
    ref = ref_paged(x)
    t = upload_paged(x)
    for ns in (0, 1, 2, 5):
        note(f"case paged edge lengths P={P} num_splits={ns}")
        out, lse = run_paged(x, ns, tensors=t)
        check_f32(out, lse, *ref, f"paged edge P={P} ns={ns}")
        assert torch.all(out[0] == 0) and torch.all(lse[0] == -float("inf"))


@pytest.mark.parametrize("layout", [HND, NHD], ids=["HND", "NHD"])
def test_paged_fp8(layout):
    """E4M3 page pools with per-kv-head scales."""
    cfg = workloads.custom_config(3, 32, 8, 128, 2500)
    x = workloads.make_paged_inputs(cfg, 8300 + layout, 64, layout, seq_lens=(2500, 999, 64),
                                    fp8=True)
    ref = ref_paged(x)
    t = upload_paged(x)
    for ns in (0, 1, 4):
        note(f"case paged fp8 layout={layout} num_splits={ns}")
        out, lse = run_paged(x, ns, tensors=t)
        check_f32(out, lse, *ref, f"paged fp8 L{layout} ns={ns}")


@pytest.mark.parametrize("layout", [HND, NHD], ids=["HND", "NHD"])
@pytest.mark.parametrize("D,G", [(D, G) for D in (64, 128) for G in (1, 2, 4, 8, 16)],
                         ids=lambda v: str(v))
def test_paged_int4(D, G, layout):
    """INT4 page pools with row-scale pools laid out like them: every (D, G),
    both layouts, two page sizes, several split counts."""
    cfg = workloads.custom_config(3, 2 * G, 2, D, 1000, k_mult=2.0)
    for P in (32, 256):
        x = workloads.make_paged_inputs(cfg, 8600 + 10 * D + G + P, P, layout,
                                        seq_lens=(1000, 777, 33), int4=True)
        ref = ref_paged(x)
        t = upload_paged(x)
        for ns in (0, 1, 3, 7):
            note(f"case paged int4 D={D} G={G} P={P} layout={layout} num_splits={ns}")
            out, lse = run_paged(x, ns, tensors=t)
            check_f32(out, lse, *ref, f"paged int4 D={D} G={G} P={P} L{layout} ns={ns}")


@pytest.mark.parametrize("P", [32, 128])
def test_paged_int4_edge_lengths(P):
    """INT4 pools: partial last pages, a page boundary either side, L = 0, 1."""
    lens = (0, 1, P - 1, P, P + 1, 2 * P - 1, 2 * P, 2 * P + 1, 5 * P + 3)
    cfg = workloads.custom_config(len(lens), 8, 2, 128, 5 * P + 3)
    x = workloads.make_paged_inputs(cfg, 8700 + P, P, NHD, seq_lens=lens, int4=True)
    ref = ref_paged(x)
    t = upload_paged(x)
    for ns in (0, 1, 2, 5):
        note(f"case paged int4 edge lengths P={P} num_splits={ns}")
        out, lse = run_paged(x, ns, tensors=t)
        check_f32(out, lse, *ref, f"paged int4 edge P={P} ns={ns}")
        assert torch.all(out[0] == 0) and torch.all(lse[0] == -float("inf"))


@pytest.mark.parametrize("idx,P,layout", [(1, 64, HND), (3, 256, NHD)],
                         ids=["gqa_32k_P64_HND", "varlen_b64_P256_NHD"])
def test_paged_int4_named_config_full_size(idx, P, layout):
    """Named configs at full size in INT4 page pools, automatic plan, against
    the oracle over every output."""
    cfg = workloads.CONFIGS[idx]
    note(f"case paged int4 full config {cfg.name} P={P}: generating inputs")
    x = workloads.make_paged_inputs(cfg, 42 + idx, P, layout, int4=True)
    t = upload_paged(x)
    note(f"case paged int4 full config {cfg.name}: auto splits")
    out, lse = run_paged(x, 0, tensors=t)
    note(f"case paged int4 full config {cfg.name}: oracle on all {len(x.base.seq_lens)} rows")
    b = x.base
    ref_o, ref_l = oracle.attention_int4(b.q, b.k, b.v, b.k_scale, b.v_scale, b.seq_lens, b.scale)
    check_f32(out, lse, ref_o, ref_l, f"paged int4 {cfg.name}")
    del t
    torch.cuda.empty_cache()


def test_paged_table_entries_outside_the_pool_are_contained():
    """A table entry outside [0, num_pages) is clamped on the device: the call
    completes and every sequence whose entries are valid is still exact."""
    cfg = workloads.custom_config(3, 8, 2, 128, 640)
    x = workloads.make_paged_inputs(cfg, 8400, 64, HND, seq_lens=(640, 640, 300))
    ref_o, ref_l = ref_paged(x)
    bad = x.block_table.copy()
    bad[1, 3] = 1 << 30          # inside sequence 1's rows: clamped to the last page
    bad[1, 4] = -7               # likewise, clamped to page 0
    bad[2, 9] = 1 << 30          # past sequence 2's rows: never read
    q, kp, vp, _, sl, ks, vs = upload_paged(x)
    bt = torch.from_numpy(bad).to(dev())
    out, lse = run_paged(x, 0, tensors=(q, kp, vp, bt, sl, ks, vs))
    ok = [0, 2]
    check_f32(out[ok], lse[ok], ref_o[ok], ref_l[ok], "sequences with valid entries")


@pytest.mark.parametrize("idx,P,layout", [(1, 64, HND), (2, 256, HND), (3, 256, NHD),
                                          (4, 128, NHD)],
                         ids=["gqa_32k_P64_HND", "gqa_128k_P256_HND", "varlen_b64_P256_NHD",
                              "ragged_b8_P128_NHD"])
def test_paged_named_config_full_size(idx, P, layout):
    """Named configs at full size in a paged pool, automatic plan, against the
    oracle over every output (the definition over the rows the generator
    scattered into the pool), with fp32 and bf16 outputs."""
    cfg = workloads.CONFIGS[idx]
    note(f"case paged full config {cfg.name} P={P}: generating inputs")
    x = workloads.make_paged_inputs(cfg, 42 + idx, P, layout)
    t = upload_paged(x)
    note(f"case paged full config {cfg.name}: auto splits")
    out, lse = run_paged(x, 0, tensors=t)
    note(f"case paged full config {cfg.name}: oracle on all {len(x.base.seq_lens)} batch rows")
    ref_o, ref_l = oracle.attention(x.base.q, x.base.k, x.base.v, x.base.seq_lens, x.base.scale)
    check_f32(out, lse, ref_o, ref_l, f"paged {cfg.name}")
    note(f"case paged full config {cfg.name}: bf16 output")
    outb, lseb = run_paged(x, 0, out_dtype=torch.bfloat16, tensors=t)
    mag = oracle.abs_attention(x.base.q, x.base.k, x.base.v, x.base.seq_lens, x.base.scale)
    check_bf16(outb, ref_o, mag, f"paged {cfg.name} bf16")
    assert torch.equal(lseb, lse), "lse differs between output modes"
    del t
    torch.cuda.empty_cache()
