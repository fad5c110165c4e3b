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
# bf16 output: ordinal distance <= 1 from the oracle rounded to bf16 where
# |oracle| >= BF16_FLOOR * S, and |err| <= BF16_ABS * S below that, with
# S = max(1, max |oracle|) over the call's output.  An exact fp32 pipeline
# leaves an absolute cancellation error at the scale of the values it
# averages, so the ulp test means something only down to a floor that grows
# with that scale.
BF16_FLOOR = 2.0 ** -12
BF16_ABS = 2.0 ** -19     # the bf16 ulp at 2^-12


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


def check_bf16(out: torch.Tensor, ref_o: np.ndarray, what: str):
    got_bits = out.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    want = oracle.round_to_bf16(ref_o)
    want_bits = oracle.bf16_bits_of(want)
    dist = np.abs(bf16_ordinal(got_bits) - bf16_ordinal(want_bits))
    got = workloads.bf16_bits_to_f32(got_bits).astype(np.float64)
    S = max(1.0, float(np.max(np.abs(ref_o)))) if ref_o.size else 1.0
    big = np.abs(ref_o) >= BF16_FLOOR * S
    literal = int(np.count_nonzero(dist > 1))
    worst_small = float(np.max(np.abs(got - ref_o)[~big])) if (~big).any() else 0.0
    note(f"  {what}: bf16 max ulp (|ref|>=2^-12*S, S={S:.3g}) {int(dist[big].max()) if big.any() else 0}, "
         f"elements >1 ulp anywhere {literal} of {dist.size}, worst |err| below floor {worst_small:.2e}")
    assert np.all(dist[big] <= 1), f"{what}: bf16 output more than 1 ulp from the rounded oracle"
    assert worst_small <= BF16_ABS * S, \
        f"{what}: near-zero bf16 error {worst_small:.2e} > 2^-19 * {S:.3g}"
