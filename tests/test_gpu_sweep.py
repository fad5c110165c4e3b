"""A seeded random sweep of the whole supported space against the fp64
oracle: head dims, group sizes, kv-head counts, batch sizes, cache lengths
(log-uniform up to 20000 rows), sequence lengths (empty, tile and page
edges, full), forced and automatic split counts, softmax scales, fp32 and
bf16 outputs, and every cache format (bf16, E4M3, INT4, and bf16, E4M3 and
INT4 page pools in both layouts).  Each case is drawn from its own seed, so a failing
case is named by that seed.

Every case runs with fp32 output against the oracle (max|err| <= 5e-4 on
the output, <= 1e-4 on LSE); a third of them run again with bf16 output,
which must be the fp32 result rounded once to nearest even, bit for bit, and
within 1 bf16 ulp of the rounded oracle where |oracle| >= 2^-5 * m, and within
2^-14 * m + half an ulp everywhere (m = sum_j w_j |v_j| / Z per element, the
oracle's magnitude form)."""
import numpy as np
import pytest
import torch

import decode_attention_split_amd as das
import oracle
import workloads
from gpu_helpers import check_bf16, check_f32, dev, note, to_dev

pytestmark = pytest.mark.gpu

GROUPS = 16           # test functions
CASES_PER_GROUP = 32  # cases per test function
FORMATS = ("bf16", "fp8", "int4", "paged", "paged_fp8", "paged_int4")


def draw_case(seed: int) -> dict:
    rng = np.random.Generator(np.random.PCG64(seed))
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.integers(1, 5))
    B = int(rng.integers(1, 9))
    fmt = FORMATS[int(rng.integers(0, len(FORMATS)))]
    smax = int(np.exp(rng.uniform(0.0, np.log(20000.0))))   # log-uniform, 1 .. 20000
    page = int(rng.choice([32, 64, 128, 256])) if fmt.startswith("paged") else 0
    # lengths: uniform, plus edge values around 32-row tiles and pages
    lens = rng.integers(0, smax + 1, size=B)
    for i in range(B):
        r = rng.random()
        if r < 0.15:
            lens[i] = 0
        elif r < 0.3:
            lens[i] = smax
        elif r < 0.5:
            q = int(rng.choice([32, page or 32, 128]))
            lens[i] = min(smax, max(0, q * int(rng.integers(0, smax // q + 1)) + int(rng.integers(-1, 2))))
    r = rng.random()
    ns = 0 if r < 0.4 else (1 if r < 0.55 else int(rng.integers(2, 49)))
    return dict(seed=seed, D=D, G=G, Hkv=Hkv, B=B, fmt=fmt, smax=smax, page=page,
                layout=int(rng.integers(0, 2)), lens=tuple(int(v) for v in lens), ns=ns,
                scale=float(rng.uniform(0.3, 1.5)) / float(np.sqrt(D)),
                bf16_out=bool(rng.random() < 0.3), k_mult=float(rng.choice([1.0, 2.0, 4.0])))


def run_case(c: dict, out_dtype, want_mag: bool = False):
    cfg = workloads.custom_config(c["B"], c["G"] * c["Hkv"], c["Hkv"], c["D"], c["smax"],
                                  k_mult=c["k_mult"])
    d = dev()
    fmt, ns, lens = c["fmt"], c["ns"], c["lens"]
    if fmt == "bf16":
        x = workloads.make_inputs(cfg, c["seed"], seq_lens=lens)
        x.scale = c["scale"]
        ref = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
        mag = (lambda: oracle.abs_attention(x.q, x.k, x.v, x.seq_lens, x.scale))
        out, lse = das.das_decode_attention(to_dev(x.q), to_dev(x.k), to_dev(x.v),
                                            torch.from_numpy(x.seq_lens).to(d), x.scale,
                                            out_dtype=out_dtype, num_splits=ns)
    elif fmt == "fp8":
        x = workloads.make_fp8_inputs(cfg, c["seed"], seq_lens=lens)
        x.scale = c["scale"]
        ref = oracle.attention_fp8(x.q, x.k, x.v, x.k_scale, x.v_scale, x.seq_lens, x.scale)
        mag = (lambda: oracle.abs_attention_fp8(x.q, x.k, x.v, x.k_scale, x.v_scale, x.seq_lens,
                                                x.scale))
        out, lse = das.das_decode_attention_fp8(
            to_dev(x.q), torch.from_numpy(x.k).to(d), torch.from_numpy(x.v).to(d),
            torch.from_numpy(x.k_scale).to(d), torch.from_numpy(x.v_scale).to(d),
            torch.from_numpy(x.seq_lens).to(d), x.scale, out_dtype=out_dtype, num_splits=ns)
    elif fmt == "int4":
        x = workloads.make_int4_inputs(cfg, c["seed"], seq_lens=lens)
        x.scale = c["scale"]
        ref = oracle.attention_int4(x.q, x.k, x.v, x.k_scale, x.v_scale, x.seq_lens, x.scale)
        # the INT4 kernels sum codes offset by 8: their rounding is relative
        # to sum_j w_j |s_j| (|n_j| + 8) (see test_gpu_int4.mag_int4)
        mag = (lambda: oracle.abs_attention_int4(x.q, x.k, x.v, x.k_scale, x.v_scale,
                                                 x.seq_lens, x.scale)
               + 8.0 * oracle.abs_attention_int4(x.q, x.k, np.full_like(x.v, 0x11), x.k_scale,
                                                 x.v_scale, x.seq_lens, x.scale))
        out, lse = das.das_decode_attention_int4(
            to_dev(x.q), torch.from_numpy(x.k).to(d), torch.from_numpy(x.v).to(d),
            torch.from_numpy(x.k_scale).to(d), torch.from_numpy(x.v_scale).to(d),
            torch.from_numpy(x.seq_lens).to(d), x.scale, out_dtype=out_dtype, num_splits=ns)
    elif fmt == "paged_int4":
        x = workloads.make_paged_inputs(cfg, c["seed"], c["page"], c["layout"], seq_lens=lens,
                                        int4=True)
        x.base.scale = c["scale"]
        k, v, ks, vs = oracle.gather_paged_int4(x)
        b = x.base
        ref = oracle.attention_int4(b.q, k, v, ks, vs, b.seq_lens, b.scale)
        mag = (lambda: oracle.abs_attention_int4(b.q, k, v, ks, vs, b.seq_lens, b.scale)
               + 8.0 * oracle.abs_attention_int4(b.q, k, np.full_like(v, 0x11), ks, vs,
                                                 b.seq_lens, b.scale))
        out, lse = das.das_decode_attention_paged(
            to_dev(b.q), torch.from_numpy(x.k_pool).to(d), torch.from_numpy(x.v_pool).to(d),
            torch.from_numpy(x.block_table).to(d), torch.from_numpy(b.seq_lens).to(d), b.scale,
            x.page_size, x.layout, k_scale=torch.from_numpy(x.k_scale_pool).to(d),
            v_scale=torch.from_numpy(x.v_scale_pool).to(d), out_dtype=out_dtype,
            num_splits=ns, kv_dtype=das.DAS_INT4)
    else:
        fp8 = fmt == "paged_fp8"
        x = workloads.make_paged_inputs(cfg, c["seed"], c["page"], c["layout"], seq_lens=lens,
                                        fp8=fp8)
        x.base.scale = c["scale"]
        smax = x.block_table.shape[1] * x.page_size
        if fp8:
            k = oracle.gather_paged(x.k_pool, x.block_table, x.base.seq_lens, x.page_size,
                                    x.layout, smax, 0x7F)
            v = oracle.gather_paged(x.v_pool, x.block_table, x.base.seq_lens, x.page_size,
                                    x.layout, smax, 0x7F)
            ref = oracle.attention_fp8(x.base.q, k, v, x.base.k_scale, x.base.v_scale,
                                       x.base.seq_lens, x.base.scale)
            mag = (lambda: oracle.abs_attention_fp8(x.base.q, k, v, x.base.k_scale,
                                                    x.base.v_scale, x.base.seq_lens, x.base.scale))
            kp, vp = torch.from_numpy(x.k_pool).to(d), torch.from_numpy(x.v_pool).to(d)
            ks, vs = torch.from_numpy(x.base.k_scale).to(d), torch.from_numpy(x.base.v_scale).to(d)
        else:
            ref = oracle.attention_paged(x.base.q, x.k_pool, x.v_pool, x.block_table,
                                         x.base.seq_lens, x.page_size, x.layout, x.base.scale)
            mag = (lambda: oracle.abs_attention_paged(x.base.q, x.k_pool, x.v_pool,
                                                      x.block_table, x.base.seq_lens,
                                                      x.page_size, x.layout, x.base.scale))
            kp, vp, ks, vs = to_dev(x.k_pool), to_dev(x.v_pool), None, None
        out, lse = das.das_decode_attention_paged(
            to_dev(x.base.q), kp, vp, torch.from_numpy(x.block_table).to(d),
            torch.from_numpy(x.base.seq_lens).to(d), x.base.scale, x.page_size, x.layout,
            k_scale=ks, v_scale=vs, out_dtype=out_dtype, num_splits=ns)
    torch.cuda.synchronize()
    return out, lse, ref, (mag() if want_mag else None)


@pytest.mark.parametrize("group", range(GROUPS))
def test_random_sweep(group):
    for i in range(CASES_PER_GROUP):
        c = draw_case(90000 + group * CASES_PER_GROUP + i)
        desc = (f"sweep seed={c['seed']} {c['fmt']} D={c['D']} G={c['G']} Hkv={c['Hkv']} "
                f"B={c['B']} Smax={c['smax']} lens={c['lens']} ns={c['ns']} page={c['page']} "
                f"layout={c['layout']} bf16_out={c['bf16_out']}")
        note(desc)
        out, lse, (ref_o, ref_l), _ = run_case(c, torch.float32)
        check_f32(out, lse, ref_o, ref_l, desc)
        if c["bf16_out"]:
            outb, lseb, _, mag = run_case(c, torch.bfloat16, want_mag=True)
            # the bf16 output is the fp32 result rounded once, to nearest even
            assert torch.equal(outb, out.to(torch.bfloat16)), f"{desc}: bf16 != rne(fp32 output)"
            assert torch.equal(lseb, lse), f"{desc}: lse differs between output modes"
            check_bf16(outb, ref_o, mag, desc)
