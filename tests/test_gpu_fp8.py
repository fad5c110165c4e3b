"""8-bit (E4M3) K/V cache (FlashDecoding++ post, §4): the HIP path vs the fp64
oracle, element by element, on seeded inputs.  Same tolerances as the bf16
cache: fp32 output max|err| <= 5e-4, LSE max|err| <= 1e-4; bf16 output within
1 bf16 ulp of the rounded oracle where |oracle| >= 2^-5 * m, and within
2^-14 * m + half an ulp everywhere (m = sum_j w_j |v_j| / Z, the oracle's
magnitude form).
Rows past seq_lens hold the E4M3 NaN code in every cache."""
import numpy as np
import pytest
import torch

import decode_attention_split_amd as das
import oracle
import workloads
from gpu_helpers import check_bf16, check_f32, dev, note, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [(D, G) for D in (64, 128) for G in (1, 2, 4, 8, 16)]


def upload_fp8(x: workloads.Fp8Inputs):
    d = dev()
    return (to_dev(x.q), torch.from_numpy(x.k).to(d), torch.from_numpy(x.v).to(d),
            torch.from_numpy(x.k_scale).to(d), torch.from_numpy(x.v_scale).to(d),
            torch.from_numpy(x.seq_lens).to(d))


def run_fp8(x, num_splits=0, out_dtype=torch.float32, tensors=None, fn=None):
    q, k, v, ks, vs, sl = tensors if tensors is not None else upload_fp8(x)
    out, lse = (fn or das.das_decode_attention_fp8)(q, k, v, ks, vs, sl, x.scale,
                                                     out_dtype=out_dtype, num_splits=num_splits)
    torch.cuda.synchronize()
    return out, lse


def ref_fp8(x):
    return oracle.attention_fp8(x.q, x.k, x.v, x.k_scale, x.v_scale, x.seq_lens, x.scale)


def mag_fp8(x):
    return oracle.abs_attention_fp8(x.q, x.k, x.v, x.k_scale, x.v_scale, x.seq_lens, x.scale)


@pytest.mark.parametrize("D,G", SHAPES, ids=lambda v: str(v))
def test_fp8_small_shapes_all_split_counts(D, G):
    """Several tiles, a ragged tail, two sequences, every supported (D, G)."""
    cfg = workloads.custom_config(2, 2 * G, 2, D, 1000, k_mult=2.0)
    x = workloads.make_fp8_inputs(cfg, 5000 + 10 * D + G, seq_lens=(1000, 777))
    ref = ref_fp8(x)
    t = upload_fp8(x)
    for ns in (0, 1, 2, 3, 7, 8):
        note(f"case fp8 D={D} G={G} num_splits={ns}")
        out, lse = run_fp8(x, ns, tensors=t)
        check_f32(out, lse, *ref, f"fp8 D={D} G={G} ns={ns}")


@pytest.mark.parametrize("D,G", [(128, 4), (128, 8), (64, 1), (128, 2)], ids=lambda v: str(v))
def test_fp8_edge_lengths(D, G):
    lens = (0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300)
    cfg = workloads.custom_config(len(lens), 2 * G, 2, D, 300)
    x = workloads.make_fp8_inputs(cfg, 6000 + D + G, seq_lens=lens)
    ref = ref_fp8(x)
    t = upload_fp8(x)
    for ns in (0, 1, 2, 3):
        note(f"case fp8 edge lengths D={D} G={G} num_splits={ns}")
        out, lse = run_fp8(x, ns, tensors=t)
        check_f32(out, lse, *ref, f"fp8 edge D={D} G={G} ns={ns}")
        assert torch.all(out[0] == 0) and torch.all(lse[0] == -float("inf"))


@pytest.mark.parametrize("D,G", [(128, 4), (64, 1), (128, 8)], ids=lambda v: str(v))
def test_fp8_bf16_output(D, G):
    cfg = workloads.custom_config(3, 4 * G, 4, D, 2000, k_mult=4.0)
    x = workloads.make_fp8_inputs(cfg, 7000 + D + G, seq_lens=(2000, 1, 1234))
    ref_o, ref_l = ref_fp8(x)
    mag = mag_fp8(x)
    t = upload_fp8(x)
    for ns in (0, 1):
        note(f"case fp8 bf16-out D={D} G={G} num_splits={ns}")
        out, lse = run_fp8(x, ns, out_dtype=torch.bfloat16, tensors=t)
        check_bf16(out, ref_o, mag, f"fp8 bf16 D={D} G={G} ns={ns}")
        assert float(np.max(np.abs(lse.cpu().numpy() - ref_l))) <= 1e-4


def test_fp8_codes_as_float8_tensor_and_per_tensor_scale():
    """The cache may be passed as torch.float8_e4m3fn; one scale for every
    kv-head is a scale array holding that value."""
    cfg = workloads.custom_config(2, 32, 8, 128, 3000)
    x = workloads.make_fp8_inputs(cfg, 7100, seq_lens=(3000, 2222))
    x.k_scale[:] = np.float32(0.0625)
    x.v_scale[:] = np.float32(0.05)
    ref = ref_fp8(x)
    q, k, v, ks, vs, sl = upload_fp8(x)
    out, lse = run_fp8(x, 0, tensors=(q, k.view(torch.float8_e4m3fn), v.view(torch.float8_e4m3fn),
                                      ks, vs, sl))
    check_f32(out, lse, *ref, "fp8 as float8_e4m3fn, per-tensor scales")


def test_fp8_two_phase_matches_fused_and_is_deterministic():
    cfg = workloads.custom_config(2, 32, 8, 128, 6000)
    x = workloads.make_fp8_inputs(cfg, 7200, seq_lens=(6000, 4097))
    q, k, v, ks, vs, sl = t = upload_fp8(x)
    o1, l1 = run_fp8(x, 0, tensors=t)
    o2, l2 = run_fp8(x, 0, tensors=t)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "run to run"
    out, lse, ws = das.das_split_kv_decode_fp8(q, k, v, ks, vs, sl, x.scale)
    das.das_lse_combine(sl, 32, 8, 6000, 128, ws, out, lse)
    torch.cuda.synchronize()
    assert float(torch.max(torch.abs(o1 - out))) <= 1e-5
    assert float(torch.max(torch.abs(l1 - lse))) <= 1e-5
    check_f32(out, lse, *ref_fp8(x), "fp8 two-phase")


@pytest.mark.parametrize("idx", range(5), ids=[c.name for c in workloads.CONFIGS])
def test_fp8_named_config_full_size(idx):
    """Every named config at full size with an E4M3 cache, in the automatic
    launch configuration the benchmark times, against the oracle over every
    output, with fp32 and bf16 outputs; num_splits=1 must agree (split
    invariance)."""
    cfg = workloads.CONFIGS[idx]
    note(f"case fp8 full config {cfg.name}: generating inputs")
    x = workloads.config_fp8_inputs(idx)
    t = upload_fp8(x)
    note(f"case fp8 full config {cfg.name}: auto splits")
    out, lse = run_fp8(x, 0, tensors=t)
    note(f"case fp8 full config {cfg.name}: oracle on all {len(x.seq_lens)} batch rows")
    ref_o, ref_l = ref_fp8(x)
    check_f32(out, lse, ref_o, ref_l, f"fp8 {cfg.name} auto")
    note(f"case fp8 full config {cfg.name}: bf16 output")
    outb, lseb = run_fp8(x, 0, out_dtype=torch.bfloat16, tensors=t)
    check_bf16(outb, ref_o, mag_fp8(x), f"fp8 {cfg.name} bf16 auto")
    assert torch.equal(lseb, lse), "lse differs between output modes"
    note(f"case fp8 full config {cfg.name}: num_splits=1")
    out1, lse1 = run_fp8(x, 1, tensors=t)
    d_o = float(torch.max(torch.abs(out1 - out)))
    d_l = float(torch.max(torch.abs(lse1 - lse)))
    note(f"  split invariance: max|out diff| {d_o:.2e}, max|lse diff| {d_l:.2e}")
    assert d_o <= 5e-4 and d_l <= 1e-4
    del t
    torch.cuda.empty_cache()
