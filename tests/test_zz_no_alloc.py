"""das_decode_attention_noalloc (the entry point for callers that cannot
allocate device memory) against das_decode_attention, through the C ABI.

It shares the plan and the kernels of das_decode_attention and only takes its
workspace from the library's static per-device array, so on the same inputs
its outputs must be bitwise those of das_decode_attention (and within the
fp32-output tolerance of the fp64 oracle).  Two calls in a row, the second
with a smaller input: the array keeps the first call's partials and counters,
which must not reach the second result."""
import ctypes

import numpy as np
import pytest
import torch

import decode_attention_split_amd as das
import oracle
import workloads
from gpu_helpers import check_f32, note, upload


def _noalloc(lib, q, k, v, sl, scale, out, lse, ns):
    B, Hq, D = q.shape
    Hkv, Smax = k.shape[1], k.shape[2]
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    code = das.DAS_BF16 if out.dtype == torch.bfloat16 else das.DAS_F32
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.das_decode_attention_noalloc(P(q), P(k), P(v), P(sl), B, Hq, Hkv, Smax, D,
                                            ctypes.c_float(scale), P(out), code, P(lse), ns,
                                            stream)


def test_noalloc_refuses_a_workspace_beyond_its_array():
    """Beyond DAS_NOALLOC_SCRATCH_BYTES of workspace the call returns
    DAS_EWORKSPACE before anything is launched (fake pointers, forced plan)."""
    lib = das.load_library()
    B, Hq, Hkv, Smax, D, ns = 256, 64, 8, 65536, 128, 64
    need = das.das_decode_workspace_bytes(B, Hq, Hkv, Smax, D, ns)
    assert need > das.DAS_NOALLOC_SCRATCH_BYTES
    f = ctypes.c_void_p(256)
    rc = lib.das_decode_attention_noalloc(f, f, f, f, B, Hq, Hkv, Smax, D, ctypes.c_float(0.1),
                                          f, das.DAS_F32, f, ns, None)
    assert rc == das.DAS_EWORKSPACE
    # an invalid shape is reported as das_decode_attention reports it
    rc = lib.das_decode_attention_noalloc(f, f, f, f, 1, 12, 8, 64, 128, ctypes.c_float(0.1),
                                          f, das.DAS_F32, f, 4, None)
    assert rc == das.DAS_EINVAL


@pytest.mark.gpu
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_noalloc_matches_decode_attention_two_calls_in_a_row(out_dtype):
    lib = das.load_library()
    cases = [
        # (B, Hq, Hkv, D, Smax, lengths, num_splits): the second call is smaller
        (4, 32, 8, 128, 12000, (12000, 7001, 4097, 1), 0),
        (2, 16, 8, 128, 3000, (3000, 1234), 0),
        (1, 8, 8, 64, 2000, (1999,), 7),
    ]
    for i, (B, Hq, Hkv, D, Smax, lens, ns) in enumerate(cases):
        note(f"case noalloc {i}: B={B} Hq={Hq} Hkv={Hkv} D={D} Smax={Smax} ns={ns} {out_dtype}")
        x = workloads.make_inputs(workloads.custom_config(B, Hq, Hkv, D, Smax), 9100 + i,
                                  seq_lens=lens)
        q, k, v, sl = upload(x)
        want_o, want_l = das.das_decode_attention(q, k, v, sl, x.scale, out_dtype=out_dtype,
                                                  num_splits=ns)
        out = torch.full((B, Hq, D), float("nan"), dtype=out_dtype, device=q.device)
        lse = torch.full((B, Hq), float("nan"), device=q.device)
        assert _noalloc(lib, q, k, v, sl, x.scale, out, lse, ns) == das.DAS_OK
        torch.cuda.synchronize()
        assert torch.equal(out, want_o) and torch.equal(lse, want_l), \
            f"case {i}: noalloc differs from das_decode_attention"
        if out_dtype == torch.float32:
            check_f32(out, lse, *oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale),
                      f"noalloc case {i}")
