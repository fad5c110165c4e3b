"""4-bit integer K/V cache (FlashDecoding++ post, §4, which names INT4 beside
FP8): the HIP path vs the fp64 oracle, element by element, on seeded inputs.
Codes are two's-complement nibbles (element 2i in the low nibble), one fp32
scale per cached row for K and one for V.  Same tolerances as the bf16 cache:
fp32 output max|err| <= 5e-4, LSE max|err| <= 1e-4; bf16 output within 1 bf16
ulp of the rounded oracle where |oracle| >= 2^-5 * m, and within 2^-14 * m +
half an ulp everywhere (m = sum_j w_j |v_j| / Z, the oracle's magnitude form).  Rows past
seq_lens hold code byte 0x88 and a NaN scale in every cache, so a read past a
sequence shows up as a wrong or non-finite result."""
import numpy as np
import pytest
import torch

import decode_attention_split_amd as das
import oracle
import workloads
from gpu_helpers import check_bf16, check_f32, dev, note, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [(D, G) for D in (64, 128) for G in (1, 2, 4, 8, 16)]


def upload_int4(x: workloads.Int4Inputs):
    d = dev()
    return (to_dev(x.q), torch.from_numpy(x.k).to(d), torch.from_numpy(x.v).to(d),
            torch.from_numpy(x.k_scale).to(d), torch.from_numpy(x.v_scale).to(d),
            torch.from_numpy(x.seq_lens).to(d))


def run_int4(x, num_splits=0, out_dtype=torch.float32, tensors=None):
    q, k, v, ks, vs, sl = tensors if tensors is not None else upload_int4(x)
    out, lse = das.das_decode_attention_int4(q, k, v, ks, vs, sl, x.scale, out_dtype=out_dtype,
                                             num_splits=num_splits)
    torch.cuda.synchronize()
    return out, lse


def mag_int4(x):
    """The magnitude the INT4 kernels' rounding is relative to.  They sum the
    codes offset by 8 (u = n + 8) and take 8 * sum_j p_j s_j off afterwards,
    so the terms they add are s_j (n_j + 8): per element
    sum_j w_j |s_j| (|n_j| + 8) = m + 8 * m1, with m the oracle's magnitude form
    and m1 the same with every code 1 (sum_j w_j |s_j|)."""
    m = oracle.abs_attention_int4(x.q, x.k, x.v, x.k_scale, x.v_scale, x.seq_lens, x.scale)
    ones = np.full_like(x.v, 0x11)
    m1 = oracle.abs_attention_int4(x.q, x.k, ones, x.k_scale, x.v_scale, x.seq_lens, x.scale)
    return m + 8.0 * m1


def ref_int4(x, rows=None):
    if rows is None:
        return oracle.attention_int4(x.q, x.k, x.v, x.k_scale, x.v_scale, x.seq_lens, x.scale)
    return oracle.attention_int4(x.q[rows], x.k[rows], x.v[rows], x.k_scale[rows],
                                 x.v_scale[rows], x.seq_lens[rows], x.scale)


@pytest.mark.parametrize("D,G", SHAPES, ids=lambda v: str(v))
def test_int4_small_shapes_all_split_counts(D, G):
    """Several tiles, a ragged tail, two sequences, every supported (D, G)."""
    cfg = workloads.custom_config(2, 2 * G, 2, D, 1000, k_mult=2.0)
    x = workloads.make_int4_inputs(cfg, 8000 + 10 * D + G, seq_lens=(1000, 777))
    ref = ref_int4(x)
    t = upload_int4(x)
    for ns in (0, 1, 2, 3, 7, 8):
        note(f"case int4 D={D} G={G} num_splits={ns}")
        out, lse = run_int4(x, ns, tensors=t)
        check_f32(out, lse, *ref, f"int4 D={D} G={G} ns={ns}")


@pytest.mark.parametrize("D,G", [(128, 4), (128, 8), (64, 1), (128, 2), (64, 4), (128, 16)],
                         ids=lambda v: str(v))
def test_int4_edge_lengths(D, G):
    lens = (0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300)
    cfg = workloads.custom_config(len(lens), 2 * G, 2, D, 300)
    x = workloads.make_int4_inputs(cfg, 8100 + D + G, seq_lens=lens)
    ref = ref_int4(x)
    t = upload_int4(x)
    for ns in (0, 1, 2, 3):
        note(f"case int4 edge lengths D={D} G={G} num_splits={ns}")
        out, lse = run_int4(x, ns, tensors=t)
        check_f32(out, lse, *ref, f"int4 edge D={D} G={G} ns={ns}")
        assert torch.all(out[0] == 0) and torch.all(lse[0] == -float("inf"))


def test_int4_extreme_codes_and_scales():
    """Every code -8 and 7 in alternation, with row scales spread over 2^-10 ..
    2^10: the offset the kernel takes off the codes and the scales it folds in
    must cancel exactly for the extreme codes too."""
    cfg = workloads.custom_config(2, 32, 8, 128, 700)
    x = workloads.make_int4_inputs(cfg, 8200, seq_lens=(700, 333))
    x.k[:] = np.uint8(0x78)            # low nibble -8, high nibble 7
    x.v[:, :, ::2, :] = np.uint8(0x87)  # low 7, high -8 on even rows
    rng = np.random.Generator(np.random.PCG64(8201))
    for s in (x.k_scale, x.v_scale):
        valid = np.isfinite(s)
        s[valid] = np.exp2(rng.uniform(-10, 10, size=int(valid.sum()))).astype(np.float32) / 64
    ref = ref_int4(x)
    t = upload_int4(x)
    for ns in (0, 1):
        note(f"case int4 extreme codes num_splits={ns}")
        out, lse = run_int4(x, ns, tensors=t)
        check_f32(out, lse, *ref, f"int4 extreme codes ns={ns}")


@pytest.mark.parametrize("D,G", [(128, 4), (64, 1), (128, 8), (64, 16)], ids=lambda v: str(v))
def test_int4_bf16_output(D, G):
    cfg = workloads.custom_config(3, 4 * G, 4, D, 2000, k_mult=4.0)
    x = workloads.make_int4_inputs(cfg, 8300 + D + G, seq_lens=(2000, 1, 1234))
    ref_o, ref_l = ref_int4(x)
    mag = mag_int4(x)
    t = upload_int4(x)
    for ns in (0, 1):
        note(f"case int4 bf16-out D={D} G={G} num_splits={ns}")
        out, lse = run_int4(x, ns, out_dtype=torch.bfloat16, tensors=t)
        check_bf16(out, ref_o, mag, f"int4 bf16 D={D} G={G} ns={ns}")
        assert float(np.max(np.abs(lse.cpu().numpy() - ref_l))) <= 1e-4


def test_int4_two_phase_matches_fused_and_is_deterministic():
    cfg = workloads.custom_config(2, 32, 8, 128, 6000)
    x = workloads.make_int4_inputs(cfg, 8400, seq_lens=(6000, 4097))
    q, k, v, ks, vs, sl = t = upload_int4(x)
    o1, l1 = run_int4(x, 0, tensors=t)
    o2, l2 = run_int4(x, 0, tensors=t)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "run to run"
    out, lse, ws = das.das_split_kv_decode_int4(q, k, v, ks, vs, sl, x.scale)
    das.das_lse_combine(sl, 32, 8, 6000, 128, ws, out, lse)
    torch.cuda.synchronize()
    assert float(torch.max(torch.abs(o1 - out))) <= 1e-5
    assert float(torch.max(torch.abs(l1 - lse))) <= 1e-5
    check_f32(out, lse, *ref_int4(x), "int4 two-phase")


@pytest.mark.parametrize("idx", range(5), ids=[c.name for c in workloads.CONFIGS])
def test_int4_named_config_full_size(idx):
    """Every named config at full size with an INT4 cache, in the automatic
    launch configuration the benchmark times, against the oracle over every
    output, with fp32 and bf16 outputs; num_splits=1 must agree (split
    invariance)."""
    cfg = workloads.CONFIGS[idx]
    note(f"case int4 full config {cfg.name}: generating inputs")
    x = workloads.config_int4_inputs(idx)
    t = upload_int4(x)
    note(f"case int4 full config {cfg.name}: auto splits")
    out, lse = run_int4(x, 0, tensors=t)
    note(f"case int4 full config {cfg.name}: oracle on all {len(x.seq_lens)} batch rows")
    ref_o, ref_l = ref_int4(x)
    check_f32(out, lse, ref_o, ref_l, f"int4 {cfg.name} auto")
    note(f"case int4 full config {cfg.name}: bf16 output")
    outb, lseb = run_int4(x, 0, out_dtype=torch.bfloat16, tensors=t)
    check_bf16(outb, ref_o, mag_int4(x), f"int4 {cfg.name} bf16 auto")
    assert torch.equal(lseb, lse), "lse differs between output modes"
    note(f"case int4 full config {cfg.name}: num_splits=1")
    out1, lse1 = run_int4(x, 1, tensors=t)
    d_o = float(torch.max(torch.abs(out1 - out)))
    d_l = float(torch.max(torch.abs(lse1 - lse)))
    note(f"  split invariance: max|out diff| {d_o:.2e}, max|lse diff| {d_l:.2e}")
    assert d_o <= 5e-4 and d_l <= 1e-4
    del t
    torch.cuda.empty_cache()


def test_int4_group_of_16_at_a_405b_shape():
    """GQA groups of 16 heads (Hq=128, Hkv=8, D=128, a Llama-3.1-405B-shaped
    decode) over a 32K-token INT4 cache at full size: the wave state of 16
    heads fills a wave's LDS region of its own.  Automatic plan and one split
    against the oracle over every output."""
    cfg = workloads.custom_config(1, 128, 8, 128, 32768)
    note("case int4 G=16 405B-shaped: generating inputs")
    x = workloads.make_int4_inputs(cfg, 8500, seq_lens=(32768,))
    ref = ref_int4(x)
    t = upload_int4(x)
    for ns in (0, 1):
        note(f"case int4 G=16 405B-shaped: num_splits={ns}")
        out, lse = run_int4(x, ns, tensors=t)
        check_f32(out, lse, *ref, f"int4 G=16 ns={ns}")
