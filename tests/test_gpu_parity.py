"""HIP path vs the fp64 oracle, element by element, on seeded inputs.

Tolerances: fp32 output max|err| <= 5e-4, LSE max|err| <= 1e-4; bf16 output
within 1 bf16 ulp of the oracle rounded to bf16 where |oracle| >= 2^-5 * m
and within 2^-14 * m + half an ulp everywhere, m = sum_j w_j |v_j| / Z per
element (the oracle's magnitude form).  Rows past seq_lens are NaN in every cache."""
import numpy as np
import pytest
import torch

import decode_attention_split_amd as das
import oracle
import workloads
from gpu_helpers import check_bf16, check_f32, note, run, to_dev, upload

pytestmark = pytest.mark.gpu

SHAPES = [(D, G) for D in (64, 128) for G in (1, 2, 4, 8, 16)]


@pytest.mark.parametrize("D,G", SHAPES, ids=lambda v: str(v))
def test_small_shapes_all_split_counts(D, G):
    """Several tiles, a ragged tail, two sequences, every supported (D, G)."""
    cfg = workloads.custom_config(2, 2 * G, 2, D, 1000, k_mult=2.0)
    x = workloads.make_inputs(cfg, 1000 + 10 * D + G, seq_lens=(1000, 777))
    ref = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    t = upload(x)
    for ns in (0, 1, 2, 3, 7, 8):
        note(f"case D={D} G={G} num_splits={ns}")
        out, lse = run(x, ns, tensors=t)
        check_f32(out, lse, *ref, f"D={D} G={G} ns={ns}")


@pytest.mark.parametrize("D,G", [(128, 4), (128, 8), (64, 1), (128, 2), (128, 16)],
                         ids=lambda v: str(v))
def test_edge_lengths(D, G):
    """Lengths around the 16/32-row tiles and the 128-row chunk quantum, with
    empty splits (forced split counts larger than a sequence needs) and L=0."""
    lens = (0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300)
    cfg = workloads.custom_config(len(lens), 2 * G, 2, D, 300)
    x = workloads.make_inputs(cfg, 2000 + D + G, seq_lens=lens)
    ref = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    t = upload(x)
    for ns in (0, 1, 2, 3):
        note(f"case edge lengths D={D} G={G} num_splits={ns}")
        out, lse = run(x, ns, tensors=t)
        check_f32(out, lse, *ref, f"edge D={D} G={G} ns={ns}")
        assert torch.all(out[0] == 0) and torch.all(lse[0] == -float("inf"))


@pytest.mark.parametrize("D,G", [(128, 4), (64, 1), (128, 8), (64, 16)], ids=lambda v: str(v))
def test_bf16_output(D, G):
    cfg = workloads.custom_config(3, 4 * G, 4, D, 2000, k_mult=4.0)
    x = workloads.make_inputs(cfg, 3000 + D + G, seq_lens=(2000, 1, 1234))
    ref_o, ref_l = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    mag = oracle.abs_attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    t = upload(x)
    for ns in (0, 1):
        note(f"case bf16 D={D} G={G} num_splits={ns}")
        out, lse = run(x, ns, out_dtype=torch.bfloat16, tensors=t)
        assert out.dtype == torch.bfloat16
        check_bf16(out, ref_o, mag, f"bf16 D={D} G={G} ns={ns}")
        lse_err = float(np.max(np.abs(lse.cpu().numpy() - ref_l)))
        assert lse_err <= 1e-4


def test_deterministic_run_to_run():
    x = workloads.make_inputs(workloads.custom_config(2, 32, 8, 128, 5000), 4000, seq_lens=(5000, 4097))
    t = upload(x)
    a = run(x, 0, tensors=t)
    b = run(x, 0, tensors=t)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("idx", range(5), ids=[c.name for c in workloads.CONFIGS])
def test_named_config_full_size(idx):
    """Every named config at its full size, in the automatic launch configuration
    the benchmark times, against the oracle over all outputs; then the same
    inputs with num_splits=1 (split invariance)."""
    cfg = workloads.CONFIGS[idx]
    note(f"case full config {cfg.name}: generating inputs")
    x = workloads.config_inputs(idx)
    ns, chunk = das.das_plan(len(x.seq_lens), cfg.Hkv, cfg.G, x.k.shape[2], cfg.D)
    note(f"case full config {cfg.name}: plan ns={ns} chunk={chunk}; oracle")
    ref = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    t = upload(x)
    note(f"case full config {cfg.name}: auto splits")
    out, lse = run(x, 0, tensors=t)
    check_f32(out, lse, *ref, f"{cfg.name} auto")
    note(f"case full config {cfg.name}: num_splits=1")
    out1, lse1 = run(x, 1, tensors=t)
    check_f32(out1, lse1, *ref, f"{cfg.name} ns=1")
    d_o = float(torch.max(torch.abs(out1 - out)))
    d_l = float(torch.max(torch.abs(lse1 - lse)))
    note(f"  split invariance: max|out diff| {d_o:.2e}, max|lse diff| {d_l:.2e}")
    assert d_o <= 5e-4 and d_l <= 1e-4
    note(f"case full config {cfg.name}: bf16 output")
    outb, lseb = run(x, 0, out_dtype=torch.bfloat16, tensors=t)
    mag = oracle.abs_attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    check_bf16(outb, ref[0], mag, f"{cfg.name} bf16 auto")
    assert float(np.max(np.abs(lseb.cpu().numpy() - ref[1]))) <= 1e-4
    del t
    torch.cuda.empty_cache()


def test_many_forced_splits_and_empty_ones():
    """Forced split counts far above the automatic plan (64 and more, chunks
    down to the 128-row quantum) on a batch whose short sequences leave most
    splits empty, against the oracle."""
    lens = (16384, 9000, 300, 129, 1, 0)
    cfg = workloads.custom_config(len(lens), 32, 8, 128, 16384)
    x = workloads.make_inputs(cfg, 4100, seq_lens=lens)
    ref = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    t = upload(x)
    for ns in (64, 100, 128):
        got_ns, chunk = das.das_plan(len(lens), 8, 4, 16384, 128, ns)
        note(f"case forced splits {ns}: plan ns={got_ns} chunk={chunk}")
        out, lse = run(x, ns, tensors=t)
        check_f32(out, lse, *ref, f"forced ns={ns}")


def test_largest_batch_grid():
    """The largest batch the grid takes (B = 65,535 sequences, the grid's
    third dimension), lengths 0 ... 16 including empty ones: one split each,
    every output written directly."""
    B = 65535
    rng = np.random.Generator(np.random.PCG64(4200))
    lens = rng.integers(0, 16, size=B, endpoint=True)
    cfg = workloads.custom_config(B, 2, 1, 64, 16)
    x = workloads.make_inputs_bulk(cfg, 4201, lens)
    ref = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    note(f"case largest batch B={B}: plan {das.das_plan(B, 1, 2, 16, 64)}")
    out, lse = run(x)
    check_f32(out, lse, *ref, f"B={B}")


def test_large_batch_many_split_workgroups():
    """16,384 sequences of up to 320 rows, two splits each where the length
    needs them: 32,768 split workgroups, phase 2 as the separate merge kernel
    over 32,768 (b, query head) rows."""
    B = 16384
    rng = np.random.Generator(np.random.PCG64(4300))
    lens = rng.integers(0, 320, size=B, endpoint=True)
    cfg = workloads.custom_config(B, 2, 1, 64, 320)
    x = workloads.make_inputs_bulk(cfg, 4301, lens)
    ref = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    ns, chunk = das.das_plan(B, 1, 2, 320, 64, 2)
    note(f"case large batch B={B}: plan ns={ns} chunk={chunk}")
    assert ns == 2
    out, lse = run(x, 2)
    check_f32(out, lse, *ref, f"B={B} ns=2")


def _int4_rows(codes, scales):
    """Dequantised INT4 rows (two's-complement nibbles, element 2i low) in fp64."""
    lo = (codes & 15).astype(np.int16)
    hi = (codes >> 4).astype(np.int16)
    n = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.int16)
    n[..., 0::2] = np.where(lo >= 8, lo - 16, lo)
    n[..., 1::2] = np.where(hi >= 8, hi - 16, hi)
    return n.astype(np.float64) * scales[..., None].astype(np.float64)


@pytest.mark.parametrize("kind", ["bf16", "int4"])
def test_closed_forms(kind):
    """Checks that need no oracle: with every logit zero (a zero softmax
    scale) the output is the plain mean of the sequence's V rows and the LSE
    is ln L, over the automatic plan and forced split counts; a one-row
    sequence returns its V row (p = 1): bit for bit from a bf16 cache (fp32
    and bf16 output), and from an INT4 cache to within the 2^-16 relative
    error of carrying the row's V scale as two bf16 halves."""
    lens = (5000, 1, 777, 64)
    cfg = workloads.custom_config(len(lens), 16, 4, 128, 5000)
    dv = torch.device("cuda:0")
    if kind == "bf16":
        x = workloads.make_inputs(cfg, 4500, seq_lens=lens)
        q, k, v, sl = upload(x)
        rows = lambda b, g, L: workloads.bf16_bits_to_f32(x.v[b, g, :L]).astype(np.float64)
        call = lambda scale, ns, od: das.das_decode_attention(q, k, v, sl, scale, out_dtype=od,
                                                              num_splits=ns)
    else:
        x = workloads.make_int4_inputs(cfg, 4501, seq_lens=lens)
        q = to_dev(x.q)
        k, v = torch.from_numpy(x.k).to(dv), torch.from_numpy(x.v).to(dv)
        ks, vs = torch.from_numpy(x.k_scale).to(dv), torch.from_numpy(x.v_scale).to(dv)
        sl = torch.from_numpy(x.seq_lens).to(dv)
        rows = lambda b, g, L: _int4_rows(x.v[b, g, :L], x.v_scale[b, g, :L])
        call = lambda scale, ns, od: das.das_decode_attention_int4(
            q, k, v, ks, vs, sl, scale, out_dtype=od, num_splits=ns)
    B, Hq, D = x.q.shape
    Hkv = x.k.shape[1]
    G = Hq // Hkv
    want = np.zeros((B, Hq, D))
    for b, L in enumerate(lens):
        for h in range(Hq):
            want[b, h] = rows(b, h // G, L).mean(axis=0)
    want_l = np.repeat(np.log(np.asarray(lens, dtype=np.float64))[:, None], Hq, axis=1)
    for ns in (0, 1, 3, 9):
        note(f"case closed form {kind}: zero scale, num_splits={ns}")
        out, lse = call(0.0, ns, torch.float32)
        torch.cuda.synchronize()
        check_f32(out, lse, want, want_l, f"{kind} zero scale ns={ns}")
    # the one-row sequence (b = 1), at the workload's own scale
    for od in (torch.float32, torch.bfloat16):
        out, _ = call(x.scale, 0, od)
        torch.cuda.synchronize()
        got = out[1].float().cpu().numpy().astype(np.float64)
        for h in range(Hq):
            row = rows(1, h // G, 1)[0]
            if kind == "int4":
                if od == torch.float32:
                    assert np.all(np.abs(got[h] - row) <= 2.0 ** -16 * np.abs(row)), \
                        f"int4: one-row sequence, head {h}: not its V row"
                continue
            if od == torch.bfloat16:
                row = workloads.bf16_bits_to_f32(
                    workloads.f32_to_bf16_bits(row.astype(np.float32))).astype(np.float64)
            assert np.array_equal(got[h], row.astype(np.float32).astype(np.float64)), \
                f"bf16: one-row sequence, head {h}, {od}: not its V row"


def test_million_token_sequence():
    """One sequence of 1,000,003 rows (Hq = 8, Hkv = 2, D = 64): the automatic
    plan's chunk reaches its 8,192-row cap, so the call runs over a hundred
    splits per kv-head, all merged in the launch by the last split to arrive,
    and the last split ends in a ragged tile.  Against the oracle, bf16 and
    INT4 caches; split invariance against one split."""
    L = 1_000_003
    cfg = workloads.custom_config(1, 8, 2, 64, L)
    x = workloads.make_inputs(cfg, 4400)
    ns, chunk = das.das_plan(1, 2, 4, L, 64, 0)
    note(f"case million-token sequence: plan ns={ns} chunk={chunk}")
    assert chunk == 8192 and ns >= 100
    ref = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    t = upload(x)
    out, lse = run(x, tensors=t)
    check_f32(out, lse, *ref, f"L={L} auto")
    one = run(x, 1, tensors=t)
    check_f32(*one, *ref, f"L={L} one split")
    del t
    y = workloads.make_int4_inputs(cfg, 4401)
    dv = torch.device("cuda:0")
    q = to_dev(y.q)
    k, v = torch.from_numpy(y.k).to(dv), torch.from_numpy(y.v).to(dv)
    ks, vs = torch.from_numpy(y.k_scale).to(dv), torch.from_numpy(y.v_scale).to(dv)
    sl = torch.from_numpy(y.seq_lens).to(dv)
    o4, l4 = das.das_decode_attention_int4(q, k, v, ks, vs, sl, y.scale)
    torch.cuda.synchronize()
    check_f32(o4, l4, *oracle.attention_int4(y.q, y.k, y.v, y.k_scale, y.v_scale, y.seq_lens,
                                             y.scale), f"INT4 L={L} auto")
    del q, k, v, ks, vs, sl, o4, l4
    torch.cuda.empty_cache()


def _steer_keys(x, ramps):
    """Give every (batch row, kv-head) a designed logit profile along the
    sequence: valid row j of K becomes a quarter of its random value plus
    ramps[b][j] / scale times q0 / |q0|^2 (q0 the group's first query head),
    rounded to bf16.  Head q0 then sees logits close to ramps[b][j] (natural
    log units); the group's other heads see small multiples of it.  Rows past
    the sequence keep their NaN marker."""
    B, Hkv, _, D = x.k.shape
    G = x.q.shape[1] // Hkv
    q = workloads.bf16_bits_to_f32(x.q).astype(np.float64)
    bits = x.k.copy()
    for b in range(B):
        L = int(x.seq_lens[b])
        for g in range(Hkv):
            u = q[b, g * G]
            k = workloads.bf16_bits_to_f32(x.k[b, g, :L]).astype(np.float64) * 0.25
            k += np.outer(np.asarray(ramps[b][:L]) / x.scale, u / np.dot(u, u))
            bits[b, g, :L] = workloads.f32_to_bf16_bits(k.astype(np.float32))
    x.k = bits
    return x


@pytest.mark.parametrize("D,G", [(128, 4), (128, 8), (64, 1), (128, 2), (64, 4), (128, 16)],
                         ids=lambda v: str(v))
def test_rising_falling_and_spiking_logits(D, G):
    """Logit profiles that move the running max in every way the online
    softmax meets (random keys hardly do): a slow rise over the whole
    sequence (the max grows a little in every tile, so rescaling waits for
    many tiles and the weights p reach the largest values the kernel lets
    them grow to), a sawtooth rising 5.5 per 32-row tile and dropping back
    every 12 tiles, a single late spike 30 above the rest, and a slow fall
    (the first tile holds the max throughout)."""
    lens = (3000, 2000, 2500, 1500)
    j = np.arange(3000, dtype=np.float64)
    spike = np.zeros(3000)
    spike[2500 - 5:2500] = 30.0
    ramps = [0.02 * j, 5.5 * ((j // 32) % 12), spike, -0.02 * j]
    cfg = workloads.custom_config(len(lens), 2 * G, 2, D, 3000)
    x = _steer_keys(workloads.make_inputs(cfg, 4200 + D + G, seq_lens=lens), ramps)
    ref = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    # the profiles did steer the logits: the spike sequence's LSE sits near 30
    assert np.all(ref[1][2, ::G] > 25.0)
    t = upload(x)
    for ns in (0, 1, 3, 8):
        note(f"case steered logits D={D} G={G} num_splits={ns}")
        out, lse = run(x, ns, tensors=t)
        check_f32(out, lse, *ref, f"steered D={D} G={G} ns={ns}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_group_of_16_at_a_405b_shape(fmt):
    """GQA groups of 16 heads (Hq=128, Hkv=8, D=128: a Llama-3.1-405B-shaped
    decode) over a 32K-token cache at full size, in the automatic plan, with
    the oracle over every output; num_splits=1 must agree."""
    cfg = workloads.custom_config(1, 128, 8, 128, 32768)
    note(f"case G=16 405B-shaped {fmt}: generating inputs")
    d = torch.device("cuda:0")
    if fmt == "bf16":
        x = workloads.make_inputs(cfg, 4300, seq_lens=(32768,))
        ref = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
        t = upload(x)
        call = lambda ns: run(x, ns, tensors=t)
    else:
        x = workloads.make_fp8_inputs(cfg, 4301, seq_lens=(32768,))
        ref = oracle.attention_fp8(x.q, x.k, x.v, x.k_scale, x.v_scale, x.seq_lens, x.scale)
        q = to_dev(x.q)
        k, v = torch.from_numpy(x.k).to(d), torch.from_numpy(x.v).to(d)
        ks, vs = torch.from_numpy(x.k_scale).to(d), torch.from_numpy(x.v_scale).to(d)
        sl = torch.from_numpy(x.seq_lens).to(d)

        def call(ns):
            o, l = das.das_decode_attention_fp8(q, k, v, ks, vs, sl, x.scale, num_splits=ns)
            torch.cuda.synchronize()
            return o, l
    for ns in (0, 1):
        note(f"case G=16 405B-shaped {fmt}: num_splits={ns}")
        out, lse = call(ns)
        check_f32(out, lse, *ref, f"G=16 {fmt} ns={ns}")


def test_call_on_a_side_stream():
    """A call on a stream other than torch's current one: the workspace, out
    and lse the binding allocates are created on that stream (their zero-fill
    ordered before the launch), while the current stream keeps allocating and
    freeing memory; the results match the oracle every time."""
    cfg = workloads.custom_config(2, 32, 8, 128, 6000)
    x = workloads.make_inputs(cfg, 4400, seq_lens=(6000, 4321))
    ref = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    q, k, v, sl = upload(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())   # the inputs are ready on the side stream
    results = []
    for i in range(6):
        # churn on the current stream: blocks freed here are reused at once
        junk = torch.full((1 << 22,), float(i), device=q.device)
        del junk
        out, lse = das.das_decode_attention(q, k, v, sl, x.scale, num_splits=7, stream=side)
        results.append((out, lse))
    side.synchronize()
    torch.cuda.synchronize()
    for i, (out, lse) in enumerate(results):
        check_f32(out, lse, *ref, f"side stream call {i}")
