"""das_merge_attn_states and the two-phase entry points against the oracle."""
import math

import numpy as np
import pytest
import torch

import decode_attention_split_amd as das
import oracle
import workloads
from gpu_helpers import check_f32, dev, note, run, upload

pytestmark = pytest.mark.gpu


def _states(rows, D, seed):
    rng = np.random.default_rng(seed)
    o = [rng.standard_normal((rows, D)).astype(np.float32) for _ in range(2)]
    s = [(rng.standard_normal(rows) * 10).astype(np.float32) for _ in range(2)]
    s[0][::7] = -np.inf
    s[1][::11] = -np.inf
    return o, s


@pytest.mark.parametrize("D", [64, 128])
def test_merge_matches_oracle_and_is_symmetric(D):
    o, s = _states(1000, D, D)
    ta = [torch.from_numpy(v).to(dev()) for v in o]
    ts = [torch.from_numpy(v).to(dev()) for v in s]
    mo, ml = das.das_merge_attn_states(ta[0], ts[0], ta[1], ts[1])
    ro, rl = oracle.merge(o[0].astype(np.float64), s[0].astype(np.float64),
                          o[1].astype(np.float64), s[1].astype(np.float64))
    torch.cuda.synchronize()
    check_f32(mo, ml, ro, rl, f"merge D={D}")
    so, sl = das.das_merge_attn_states(ta[1], ts[1], ta[0], ts[0])
    torch.cuda.synchronize()
    assert torch.equal(mo, so) and torch.equal(ml, sl), "merge must be bitwise symmetric"
    ident_o, ident_l = das.das_merge_attn_states(ta[0], ts[0], torch.zeros_like(ta[0]),
                                                 torch.full_like(ts[0], -math.inf))
    torch.cuda.synchronize()
    fin = torch.isfinite(ts[0])
    assert torch.allclose(ident_o[fin], ta[0][fin], atol=1e-6)
    assert torch.allclose(ident_l[fin], ts[0][fin], atol=1e-6)


def test_merge_in_place_and_bf16():
    o, s = _states(333, 128, 5)
    ta = [torch.from_numpy(v).to(dev()) for v in o]
    ts = [torch.from_numpy(v).to(dev()) for v in s]
    want_o, want_l = das.das_merge_attn_states(ta[0], ts[0], ta[1], ts[1])
    a_o, a_l = ta[0].clone(), ts[0].clone()
    das.das_merge_attn_states(a_o, a_l, ta[1], ts[1], o_out=a_o, lse_out=a_l)
    torch.cuda.synchronize()
    assert torch.equal(a_o, want_o) and torch.equal(a_l, want_l)
    bo, bl = das.das_merge_attn_states(ta[0].bfloat16(), ts[0], ta[1].bfloat16(), ts[1])
    ro, rl = oracle.merge(ta[0].bfloat16().double().cpu().numpy(), s[0].astype(np.float64),
                          ta[1].bfloat16().double().cpu().numpy(), s[1].astype(np.float64))
    torch.cuda.synchronize()
    assert float(torch.max(torch.abs(bo.double().cpu() - torch.from_numpy(ro)))) <= 2 ** -7 * 8
    assert float(np.max(np.abs(bl.cpu().numpy()[np.isfinite(rl)] - rl[np.isfinite(rl)]))) <= 1e-5


def test_merging_two_half_sequences_equals_whole():
    """Decode over rows [0, m) and [m, L) separately, merge on the GPU: equals decode over [0, L)."""
    cfg = workloads.custom_config(2, 16, 4, 128, 3000, k_mult=4.0)
    x = workloads.make_inputs(cfg, 77, seq_lens=(3000, 2100))
    m = 1300
    q, k, v, sl = upload(x)
    whole_o, whole_l = run(x, 0, tensors=(q, k, v, sl))
    first = das.das_decode_attention(q, k, v, torch.clamp(sl, max=m), x.scale)
    second = das.das_decode_attention(q, k[:, :, m:].contiguous(), v[:, :, m:].contiguous(),
                                      torch.clamp(sl - m, min=0), x.scale)
    mo, ml = das.das_merge_attn_states(first[0], first[1], second[0], second[1])
    torch.cuda.synchronize()
    ref = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    check_f32(mo, ml, *ref, "merged halves")
    assert float(torch.max(torch.abs(mo - whole_o))) <= 5e-4


def test_merge_is_associative_over_three_parts_of_a_sequence():
    """Decode over three parts of the rows, merge them on the GPU in both
    groupings ((a b) c and a (b c)): each equals the oracle's attention over
    the whole sequence, and the two agree to rounding.  The merge is exact in
    real arithmetic; the groupings differ in the fp32 rounding of the
    intermediate state, above all of its LSE (half an ulp of |lse| each),
    which enters a weight exp(lse - max): a relative change of the weights of
    about ulp(|lse|), so of the output by that times max |o| of the parts."""
    cfg = workloads.custom_config(3, 16, 4, 128, 3000, k_mult=4.0)
    x = workloads.make_inputs(cfg, 78, seq_lens=(3000, 2500, 700))
    q, k, v, sl = upload(x)
    cuts = (0, 1000, 2000, 3000)
    parts = []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        # rows [lo, hi) of each sequence (none where the sequence ends before lo)
        part_len = torch.clamp(torch.clamp(sl, max=hi) - lo, min=0)
        parts.append(das.das_decode_attention(q, k[:, :, lo:hi].contiguous(),
                                              v[:, :, lo:hi].contiguous(), part_len, x.scale))
    (ao, al), (bo, bl), (co, cl) = parts
    ab = das.das_merge_attn_states(ao, al, bo, bl)
    left = das.das_merge_attn_states(ab[0], ab[1], co, cl)
    bc = das.das_merge_attn_states(bo, bl, co, cl)
    right = das.das_merge_attn_states(ao, al, bc[0], bc[1])
    torch.cuda.synchronize()
    ref = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    check_f32(left[0], left[1], *ref, "(a b) c")
    check_f32(right[0], right[1], *ref, "a (b c)")
    # the third sequence ends inside part a: parts b and c are empty there
    # (lse -inf, the merge's identity), and both groupings give part a's state
    for got in (left, right):
        assert torch.allclose(got[0][2], ao[2], rtol=0, atol=1e-6)
        assert torch.allclose(got[1][2], al[2], rtol=0, atol=1e-6)
    lses = torch.cat([al, bl, cl])
    lse_max = float(torch.max(torch.abs(lses[torch.isfinite(lses)])))
    ulp = 2.0 ** (math.floor(math.log2(lse_max)) - 23)     # fp32 ulp at max |lse|
    o_max = max(float(torch.max(torch.abs(t))) for t in (ao, bo, co))
    d_o = float(torch.max(torch.abs(left[0] - right[0])))
    d_l = float(torch.max(torch.abs(left[1] - right[1])))
    note(f"  groupings differ by {d_o:.3e} (out), {d_l:.3e} (lse); ulp(max|lse|) {ulp:.3e}")
    assert d_o <= 4 * ulp * o_max + 2.0 ** -20 * o_max
    assert d_l <= 4 * ulp


def test_two_phase_entry_points_match_the_fused_call():
    """das_split_kv_decode + das_lse_combine (two kernels) computes what the fused
    das_decode_attention computes; only the merge's summation order differs."""
    cfg = workloads.CONFIGS[1]
    x = workloads.make_inputs(cfg, 5, smax=4096, seq_lens=(4000,))
    q, k, v, sl = upload(x)
    o1, l1 = das.das_decode_attention(q, k, v, sl, x.scale, num_splits=0)
    out, lse, ws = das.das_split_kv_decode(q, k, v, sl, x.scale, num_splits=0)
    das.das_lse_combine(sl, cfg.Hq, cfg.Hkv, 4096, cfg.D, ws, out, lse, num_splits=0)
    torch.cuda.synchronize()
    assert float(torch.max(torch.abs(o1 - out))) <= 1e-5
    assert float(torch.max(torch.abs(l1 - lse))) <= 1e-5
    ref = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    check_f32(out, lse, *ref, "two-phase entry points")


def test_fused_merge_leaves_counters_zero_and_repeats_exactly():
    """The arrival counters at the start of the workspace are back at zero after
    every call, so back-to-back calls on one workspace give bitwise the same result."""
    cfg = workloads.custom_config(3, 32, 8, 128, 6000)
    x = workloads.make_inputs(cfg, 6, seq_lens=(6000, 2500, 129))
    q, k, v, sl = upload(x)
    need = das.das_decode_workspace_bytes(3, 32, 8, 6000, 128, 7)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    first = das.das_decode_attention(q, k, v, sl, x.scale, num_splits=7, workspace=ws)
    torch.cuda.synchronize()
    counters = ws[:das.DAS_WORKSPACE_COUNTER_BYTES].view(torch.int32)
    assert int(torch.count_nonzero(counters)) == 0
    for _ in range(3):
        again = das.das_decode_attention(q, k, v, sl, x.scale, num_splits=7, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(again[0], first[0]) and torch.equal(again[1], first[1])
    assert int(torch.count_nonzero(counters)) == 0
    ref = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    check_f32(*first, *ref, "fused merge, forced 7 splits")


def test_fused_merge_over_many_counter_slots():
    """512 (b, kv-head) pairs merged in one launch (B = 64, 2 splits: 4 split
    workgroups per CU, the most the fused call takes), each with its own
    arrival counter on its own cache line: every pair's output matches the
    oracle, a repeat is bitwise equal, and every counter is back at zero."""
    cfg = workloads.custom_config(64, 32, 8, 128, 512)
    rng = np.random.Generator(np.random.PCG64(7100))
    lens = rng.integers(1, 512, size=64, endpoint=True)
    x = workloads.make_inputs(cfg, 7101, seq_lens=lens)
    q, k, v, sl = upload(x)
    ns, _ = das.das_plan(64, 8, 4, 512, 128, 2)
    assert ns == 2
    assert 64 * 8 * ns <= 4 * torch.cuda.get_device_properties(0).multi_processor_count
    need = das.das_decode_workspace_bytes(64, 32, 8, 512, 128, ns)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    note("case fused merge, B=64 x Hkv=8 pairs, 2 splits")
    first = das.das_decode_attention(q, k, v, sl, x.scale, num_splits=ns, workspace=ws)
    again = das.das_decode_attention(q, k, v, sl, x.scale, num_splits=ns, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(again[0], first[0]) and torch.equal(again[1], first[1])
    assert int(torch.count_nonzero(ws[:das.DAS_WORKSPACE_COUNTER_BYTES])) == 0
    check_f32(*first, *oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale),
              "fused merge over 512 pairs")


def test_graph_capture_replays_match_eager():
    cfg = workloads.custom_config(4, 32, 8, 128, 4096)
    x = workloads.make_inputs(cfg, 9, seq_lens=(4096, 1000, 1, 3000))
    q, k, v, sl = upload(x)
    eager_o, eager_l = das.das_decode_attention(q, k, v, sl, x.scale)
    out = torch.empty_like(eager_o)
    lse = torch.empty_like(eager_l)
    ws = torch.zeros(max(das.das_decode_workspace_bytes(4, 32, 8, 4096, 128), 16),
                     dtype=torch.uint8, device=dev())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        das.das_decode_attention(q, k, v, sl, x.scale, out=out, lse_out=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        das.das_decode_attention(q, k, v, sl, x.scale, out=out, lse_out=lse, workspace=ws)
    for i in range(4):
        out.fill_(float("nan"))
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_o) and torch.equal(lse, eager_l), f"replay {i}"
        _ = (torch.ones(1000, device=dev()) * 2).sum().item()   # eager work between replays
    note("graph replays match eager")


def _replays_match(run, outs, what):
    """Capture run() (which writes into the tensors `outs`) in a HIP graph
    after one eager call, replay it several times with eager work between the
    replays, and check every replay against the eager result, bit for bit."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(4):
        for t in outs:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(outs, eager):
            assert torch.equal(t, e), f"{what}: replay {i}"
        _ = (torch.ones(1000, device=dev()) * 2).sum().item()   # eager work between replays
    note(f"  {what}: graph replays match eager")


def test_graph_capture_of_the_other_entry_points():
    """Paged INT4 and E4M3 calls (fused merge and the separate merge kernel),
    the no-allocation entry point and merge_attn_states, each captured in a
    HIP graph and replayed."""
    from test_gpu_paged import upload_paged

    # paged INT4, small batch: fused merge
    cfg = workloads.custom_config(3, 32, 8, 128, 3000, k_mult=2.0)
    x = workloads.make_paged_inputs(cfg, 9300, 64, workloads.PAGED_HND, seq_lens=(3000, 1700, 5),
                                    int4=True)
    q, kp, vp, bt, sl, ks, vs = upload_paged(x)
    out = torch.empty((3, 32, 128), device=dev())
    lse = torch.empty((3, 32), device=dev())
    smax = x.block_table.shape[1] * x.page_size
    ws = torch.zeros(max(das.das_decode_workspace_bytes(3, 32, 8, smax, 128), 16),
                     dtype=torch.uint8, device=dev())
    _replays_match(lambda: das.das_decode_attention_paged(
        q, kp, vp, bt, sl, x.base.scale, x.page_size, x.layout, k_scale=ks, v_scale=vs, out=out,
        lse_out=lse, workspace=ws, kv_dtype=das.DAS_INT4), (out, lse), "paged INT4, fused merge")

    # E4M3 pool, B=64: the separate merge kernel
    rng = np.random.Generator(np.random.PCG64(9301))
    lens = rng.integers(1, 2048, size=64, endpoint=True)
    cfg = workloads.custom_config(64, 32, 8, 128, 2048)
    x = workloads.make_paged_inputs(cfg, 9302, 64, workloads.PAGED_NHD, seq_lens=lens, fp8=True)
    q, kp, vp, bt, sl, ks, vs = upload_paged(x)
    out = torch.empty((64, 32, 128), device=dev())
    lse = torch.empty((64, 32), device=dev())
    smax = x.block_table.shape[1] * x.page_size
    ws = torch.zeros(max(das.das_decode_workspace_bytes(64, 32, 8, smax, 128), 16),
                     dtype=torch.uint8, device=dev())
    _replays_match(lambda: das.das_decode_attention_paged(
        q, kp, vp, bt, sl, x.base.scale, x.page_size, x.layout, k_scale=ks, v_scale=vs, out=out,
        lse_out=lse, workspace=ws), (out, lse), "paged E4M3, separate merge kernel")

    # the no-allocation entry point
    cfg = workloads.custom_config(2, 16, 4, 128, 5000)
    x = workloads.make_inputs(cfg, 9303, seq_lens=(5000, 2222))
    q, k, v, sl = upload(x)
    out = torch.empty((2, 16, 128), device=dev())
    lse = torch.empty((2, 16), device=dev())
    _replays_match(lambda: das.das_decode_attention_noalloc(q, k, v, sl, x.scale, out=out,
                                                            lse_out=lse),
                   (out, lse), "no-allocation entry point")

    # merge_attn_states
    o, sv = _states(777, 128, 9304)
    ta = [torch.from_numpy(t).to(dev()) for t in o]
    ts = [torch.from_numpy(t).to(dev()) for t in sv]
    mo = torch.empty_like(ta[0])
    ml = torch.empty_like(ts[0])
    _replays_match(lambda: das.das_merge_attn_states(ta[0], ts[0], ta[1], ts[1], o_out=mo,
                                                     lse_out=ml), (mo, ml), "merge_attn_states")


def test_many_split_workgroups_take_the_two_kernel_merge():
    """B*Hkv*NS above 4 workgroups per CU: das_decode_attention merges with a
    second kernel instead of the fused last-workgroup merge; same results."""
    cfg = workloads.custom_config(16, 32, 8, 128, 2048)
    lens = [2048, 1, 0, 777, 2047, 1500, 128, 129, 1024, 2000, 5, 1800, 256, 900, 1999, 64]
    x = workloads.make_inputs(cfg, 8, seq_lens=lens)
    q, k, v, sl = upload(x)
    ref = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    for ns in (16, 9):   # 16*8*16 = 2048 and 16*8*9 = 1152 split workgroups
        out, lse = das.das_decode_attention(q, k, v, sl, x.scale, num_splits=ns)
        torch.cuda.synchronize()
        check_f32(out, lse, *ref, f"two-kernel merge ns={ns}")


def test_fused_merge_ignores_whatever_the_partial_slots_held():
    """The fused merge reads only the slots of this call's non-empty splits,
    each written by this call before its workgroup is counted.  Garbage,
    another input's partials (left by the phase-1 entry point) or another
    shape's leftovers in the partial area never reach the result."""
    cfg = workloads.custom_config(2, 32, 8, 128, 5000)
    x = workloads.make_inputs(cfg, 10, seq_lens=(5000, 3100))
    y = workloads.make_inputs(cfg, 11, seq_lens=(4900, 5000))
    qx, kx, vx, slx = upload(x)
    qy, ky, vy, sly = upload(y)
    ns = 9
    need = das.das_decode_workspace_bytes(2, 32, 8, 5000, 128, ns)
    clean = torch.zeros(need, dtype=torch.uint8, device=dev())
    want_o, want_l = das.das_decode_attention(qx, kx, vx, slx, x.scale, num_splits=ns,
                                              workspace=clean)
    torch.cuda.synchronize()
    check_f32(want_o, want_l, *oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale),
              "fused merge, clean workspace")

    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    cb = das.DAS_WORKSPACE_COUNTER_BYTES
    g = torch.Generator(device="cpu").manual_seed(3)
    junk = torch.randint(1, 255, (need - cb,), dtype=torch.uint8, generator=g)
    ws[cb:] = junk.to(dev())                                   # garbage, no zero byte
    got = das.das_decode_attention(qx, kx, vx, slx, x.scale, num_splits=ns, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(got[0], want_o) and torch.equal(got[1], want_l), "after garbage"

    # another input's partials, written by the phase-1 entry point and never merged
    das.das_split_kv_decode(qy, ky, vy, sly, y.scale, num_splits=ns, workspace=ws)
    got = das.das_decode_attention(qx, kx, vx, slx, x.scale, num_splits=ns, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(got[0], want_o) and torch.equal(got[1], want_l), "after phase-1 leftovers"

    # a different split count puts other shapes' slots over these ones
    das.das_split_kv_decode(qy, ky, vy, sly, y.scale, num_splits=5, workspace=ws)
    got = das.das_decode_attention(qx, kx, vx, slx, x.scale, num_splits=ns, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(got[0], want_o) and torch.equal(got[1], want_l), "after another plan"
    counters = ws[:cb].view(torch.int32)
    assert int(torch.count_nonzero(counters)) == 0


def test_counters_left_nonzero_fail_loudly():
    """A workspace whose arrival counters were never zeroed (here set, from
    the host, to a count no call can reach) turns the fused merge's outputs
    into NaN instead of leaving stale ones; once zeroed, the same workspace
    gives the exact result again."""
    cfg = workloads.custom_config(2, 32, 8, 128, 5000)
    x = workloads.make_inputs(cfg, 12, seq_lens=(5000, 3100))
    q, k, v, sl = upload(x)
    ns = 9
    need = das.das_decode_workspace_bytes(2, 32, 8, 5000, 128, ns)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    cb = das.DAS_WORKSPACE_COUNTER_BYTES
    ws[:cb].view(torch.int32).fill_(0x7FFF0000)
    out, lse = das.das_decode_attention(q, k, v, sl, x.scale, num_splits=ns, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(out)) and torch.all(torch.isnan(lse)), "garbage counters: NaN"
    ws[:cb].zero_()
    out, lse = das.das_decode_attention(q, k, v, sl, x.scale, num_splits=ns, workspace=ws)
    torch.cuda.synchronize()
    check_f32(out, lse, *oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale), "after zeroing")
    assert int(torch.count_nonzero(ws[:cb])) == 0
