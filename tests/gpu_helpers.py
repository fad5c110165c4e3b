"""Shared helpers for the GPU tests: upload seeded inputs, run the library,
compare with the fp64 oracle to the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import decode_attention_split_amd as das
import oracle
import workloads

OUT_TOL = 5e-4      # fp32-output mode: max |err| on the output
LSE_TOL = 1e-4      # max |err| on the natural-log LSE
# bf16 output.  Per element, m = sum_j w_j |v_j| / Z (oracle.abs_attention*):
# the magnitude of the terms the output averages (for an INT4 cache, whose
# kernels add the codes offset by 8, that of the offset terms; see
# test_gpu_int4.mag_int4).  Rounding inside the kernels moves the fp32
# result by at most MAG_REL * m:
#   - p enters the p.V products as two bf16 halves whose sum is p to within
#     2^-16 relative: at most 2^-16 * m;
#   - each logit's fp32 sums round by a few 2^-24 of sum_d |q_d k_d| (twice
#     that for INT4, whose codes carry an offset of 8 taken off afterwards),
#     which for these inputs moves each weight by less than 2^-16 relative:
#     at most 2^-16 * m;
#   - exp2, the fp32 accumulations and the merge of the splits: less than
#     2^-16 * m;
#   and MAG_REL = 2^-14 covers the three with room to spare.
# The bf16 output is that result rounded once, so it is within
# MAG_REL * m + half a bf16 ulp of the oracle everywhere (checked), and
# within 1 bf16 ulp of the oracle rounded to bf16 (the stated tolerance,
# checked) wherever MAG_REL * m is below half an ulp of the output, i.e.
# where |oracle| >= 2^9 * MAG_REL * m = BF16_FLOOR * m.  Below that floor the
# output cancels to a small fraction of the values it averages.
MAG_REL = 2.0 ** -14      # = 2^10 * 2^-24
BF16_FLOOR = 2.0 ** 9 * MAG_REL


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def upload(x: workloads.Inputs):
    return (to_dev(x.q), to_dev(x.k), to_dev(x.v), torch.from_numpy(x.seq_lens).to(dev()))


def run(x: workloads.Inputs, num_splits: int = 0, out_dtype=torch.float32, tensors=None):
    q, k, v, sl = tensors if tensors is not None else upload(x)
    out, lse = das.das_decode_attention(q, k, v, sl, x.scale, out_dtype=out_dtype,
                                        num_splits=num_splits)
    torch.cuda.synchronize()
    return out, lse


def check_f32(out: torch.Tensor, lse: torch.Tensor, ref_o: np.ndarray, ref_l: np.ndarray, what: str):
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    eo = float(np.max(np.abs(o - ref_o))) if o.size else 0.0
    finite = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(l), finite), f"{what}: lse finiteness differs"
    assert np.all(l[~finite] == ref_l[~finite]), f"{what}: empty rows must give lse=-inf"
    el = float(np.max(np.abs(l[finite] - ref_l[finite]))) if finite.any() else 0.0
    note(f"  {what}: max|out err| {eo:.3e}  max|lse err| {el:.3e}")
    assert eo <= OUT_TOL, f"{what}: output error {eo:.3e} > {OUT_TOL}"
    assert el <= LSE_TOL, f"{what}: lse error {el:.3e} > {LSE_TOL}"
    return eo, el


def bf16_ordinal(bits: np.ndarray) -> np.ndarray:
    """Map bf16 bit patterns to integers that are consecutive for adjacent values."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 values at |x| (8 significant bits)."""
    _, e = np.frexp(np.abs(x))                  # |x| = f * 2^e, 0.5 <= f < 1
    return np.ldexp(1.0, np.maximum(e - 9, -134))


def check_bf16(out: torch.Tensor, ref_o: np.ndarray, mag: np.ndarray, what: str):
    """bf16 output against the fp64 oracle ``ref_o``, with ``mag`` the
    oracle's magnitude form (sum_j w_j |v_j| / Z) of the same call."""
    got_bits = out.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    want = oracle.round_to_bf16(ref_o)
    want_bits = oracle.bf16_bits_of(want)
    dist = np.abs(bf16_ordinal(got_bits) - bf16_ordinal(want_bits))
    got = workloads.bf16_bits_to_f32(got_bits).astype(np.float64)
    mag = np.asarray(mag, dtype=np.float64)
    assert mag.shape == ref_o.shape, f"{what}: magnitude shape {mag.shape} vs {ref_o.shape}"
    assert np.all(np.abs(ref_o) <= mag * (1 + 1e-12)), f"{what}: |oracle| above its magnitude"
    err = np.abs(got - ref_o)
    strict = np.abs(ref_o) >= BF16_FLOOR * mag
    far = dist > 1
    pos = mag > 0
    # the fp32 pipeline's share of the error: what is left after the final
    # rounding to bf16, in units of 2^-24 m
    beyond = np.maximum(err - half_ulp_bf16(got), 0.0)
    ratio = float(np.max(beyond[pos] / (2.0 ** -24 * mag[pos]))) if pos.any() else 0.0
    rel_far = (float(np.max(np.abs(ref_o[far]) / mag[far])) if far.any() else 0.0)
    note(f"  {what}: max ulp where |ref| >= 2^-5 m: {int(dist[strict].max()) if strict.any() else 0}; "
         f"{int(far.sum())} of {dist.size} elements >1 ulp (largest |ref|/m among them {rel_far:.2e}); "
         f"worst |err| beyond the final rounding {ratio:.1f} x 2^-24 m (bound {MAG_REL / 2.0 ** -24:.0f})")
    assert np.all(dist[strict] <= 1), f"{what}: bf16 output more than 1 ulp from the rounded oracle"
    assert np.all(err <= MAG_REL * mag + half_ulp_bf16(got)), \
        f"{what}: bf16 error above 2^-14 * m + half an ulp"
