"""Benchmark: KV-cache read GB/s (and µs per call) of split-KV decode attention.

One step = one decode-attention call (das_decode_attention: phase 1 with
the phase-2 merge fused into the last workgroup of each (batch row,
kv-head), a single kernel launch; on grids of more than 4 split workgroups
per CU phase 2 runs as a second, small kernel) over the synthetic workload,
with every input already resident in HBM.  K/V are rotated over several
copies so that repeated steps read from HBM rather than from the 256 MB
last-level cache.  The default workload is the largest named config that
fits one GPU: the batched variable-length GQA decode (B=64, Hq=32, Hkv=8,
D=128, lengths U[512, 16384], 2.36 GB of K/V per call).

Prints one JSON line on stdout.  Also reports the achieved algorithmic HBM
bandwidth of the call's kernels against the MI355X peak, measured with HIP
events on the launch stream around the timed launches; for reference only,
the same calls replayed from one HIP graph and the median of calls issued
one at a time after a cache flush; the fp64 CPU oracle's throughput on a
bounded sample of the same workload (the reported CPU baseline); and, in
``config.per_config``, every named config timed in the same process
(bf16 K/V: automatic plan with fp32 and bf16 output, and one split; E4M3
and INT4 caches and page pools with the automatic plan).  Progress goes to
stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV-cache read GB/s (% of HBM peak) and µs per decode-attention call"
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, 8 TB/s
LLC_BYTES = 256 << 20     # MI355X Infinity Cache


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3,
                    help="index into workloads.CONFIGS (default 3: the batched varlen GQA "
                         "decode, B=64, the largest config)")
    ap.add_argument("--splits", type=int, default=0, help="0 = automatic plan")
    ap.add_argument("--hq", type=int, default=0,
                    help="query heads instead of the config's own (same kv-heads, lengths and "
                         "seed), e.g. --config 1 --hq 128 for groups of 16 heads")
    ap.add_argument("--out-dtype", choices=("f32", "bf16"), default="f32")
    ap.add_argument("--kv-dtype", choices=("bf16", "fp8", "int4"), default="bf16",
                    help="K/V cache element: bf16, E4M3 codes with per-kv-head scales, or "
                         "INT4 codes with per-row scales")
    ap.add_argument("--paged", type=int, default=0,
                    help="page size in rows: time the paged entry point over a shuffled pool")
    ap.add_argument("--paged-layout", choices=("hnd", "nhd"), default="hnd")
    ap.add_argument("--copies", type=int, default=0, help="K/V copies to rotate; 0 = auto")
    ap.add_argument("--isolated", action=argparse.BooleanOptionalAction, default=True,
                    help="also time 100 calls one by one, each after a 1 GiB cache flush and "
                         "between its own events (median; reported beside, never as, the value)")
    ap.add_argument("--graph", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the calls replayed from one HIP graph (reported beside, "
                         "never as, the value)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time for the oracle baseline; 0 skips it")
    ap.add_argument("--op", choices=("decode", "merge"), default="decode",
                    help="decode: the decode-attention call (the headline); merge: "
                         "das_merge_attn_states alone, at one decode step's rows and at a "
                         "bandwidth-sized call")
    ap.add_argument("--table", action=argparse.BooleanOptionalAction, default=True,
                    help="also time every named config (bf16 K/V) in this process: automatic "
                         "plan with fp32 and bf16 output, and one split")
    ap.add_argument("--table-steps", type=int, default=50,
                    help="back-to-back launches timed per table row")
    ap.add_argument("--table-warmup", type=int, default=5)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain device copy of known size (counter calibration)")
    return ap.parse_args()


COPY_BYTES = 256 << 20


def calibrate_copy() -> None:
    """A plain 256 MiB device-to-device copy, 10 times: the reference whose
    FETCH_SIZE / WRITE_SIZE counters scale the decode kernel's counters."""
    import torch

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                      "launches": 10}), flush=True)


def bench_merge(args) -> None:
    """das_merge_attn_states ([SGL-PAR] "Constraints": the LSE merge of two
    partial states, as a sequence-parallel decode ends with) on fp32 states
    of D = 128: HBM bytes per call 3 * rows * (D + 1) * 4 (two states read,
    one written).  Times args.steps calls back to back after args.warmup,
    with HIP events on the launch stream, at rows = 2048 (one decode step of
    B=64 x Hq=32) and rows = 2^20."""
    import ctypes

    import torch

    import decode_attention_split_amd as das

    lib = das.load_library()
    dev = torch.device("cuda:0")
    D = 128
    sizes = []
    for rows in (2048, 1 << 20):
        g = torch.Generator().manual_seed(rows)
        o_a = torch.randn(rows, D, generator=g).to(dev)
        o_b = torch.randn(rows, D, generator=g).to(dev)
        lse_a = (4 * torch.randn(rows, generator=g)).to(dev)
        lse_b = (4 * torch.randn(rows, generator=g)).to(dev)
        o_out, lse_out = torch.empty_like(o_a), torch.empty_like(lse_a)
        ptrs = [ctypes.c_void_p(t.data_ptr()) for t in (o_a, lse_a, o_b, lse_b, o_out, lse_out)]
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

        def call():
            rc = lib.das_merge_attn_states(*ptrs, rows, D, das.DAS_F32, stream)
            if rc != 0:
                raise RuntimeError(f"das_merge_attn_states: status {rc}")

        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / args.steps * 1e3
        nbytes = 3 * rows * (D + 1) * 4
        sizes.append({"rows": rows, "D": D, "bytes_per_call": nbytes, "us_per_call": round(us, 3),
                      "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                      "pct_of_hbm_peak": round(100 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)})
    big = sizes[-1]
    print(json.dumps({
        "metric": "merge_attn_states HBM GB/s (% of peak) and us per call",
        "value": big["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(big["us_per_call"] / 1e3, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "merge_attn_states_f32_d128", "sizes": sizes},
        "roofline": {"bound": "hbm", "kernel": "merge_attn_states", "achieved": big["GB/s"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(big["GB/s"] / HBM_PEAK_GBS, 4), "traffic": None},
    }), flush=True)


def kernel_source_digest() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in ("decode_attention_split_amd/csrc/das_kernels.hip",
                "decode_attention_split_amd/csrc/das_internal.h",
                "decode_attention_split_amd/csrc/das_api.cpp"):
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counters_path(workload: str, kv_dtype: str = "bf16", page_size: int = 0,
                  layout: str = "hnd") -> str:
    """The committed counter summary of a workload, cache format and pool."""
    name = "split_kv_decode" + ("_paged" if page_size else "") + \
        {"bf16": "", "fp8": "_e4m3", "int4": "_int4"}[kv_dtype] + "_" + workload + \
        (f"_p{page_size}_{layout}" if page_size else "") + "_counters.json"
    return os.path.join(ROOT, "profiles", name)


def measured_traffic(workload: str, ns: int, kv_dtype: str = "bf16", page_size: int = 0,
                     layout: str = "hnd"):
    """HBM bytes per launch from the committed counter summary, when it was
    taken on the current kernel source and this workload; otherwise None."""
    path = counters_path(workload, kv_dtype, page_size, layout)
    try:
        with open(path) as fh:
            doc = json.load(fh)
    except (OSError, ValueError):
        return None
    if doc.get("kernel_source_sha256") != kernel_source_digest() or doc.get("num_splits") != ns:
        return None
    return doc.get("hbm_bytes_per_launch")


def cpu_baseline(x, target_s: float):
    """Time the fp64 oracle on a bounded sample of the workload: whole calls,
    repeated until about target_s seconds, or a prefix of batch rows when one
    call alone would take much longer."""
    import numpy as np
    import oracle

    threads = oracle.max_threads()
    B = len(x.seq_lens)
    rows = B
    # probe with one batch row to size the sample
    t = time.perf_counter()
    oracle.attention(x.q[:1], x.k[:1], x.v[:1], x.seq_lens[:1], x.scale)
    one = time.perf_counter() - t
    per_row = max(one, 1e-4)
    if per_row * B > 3 * target_s:
        rows = max(1, int(target_s / per_row))
    q, k, v, sl = x.q[:rows], x.k[:rows], x.v[:rows], x.seq_lens[:rows]
    sample_bytes = int(sl.astype(np.int64).sum()) * x.k.shape[1] * x.k.shape[3] * 4
    calls = 0
    t0 = time.perf_counter()
    while True:
        oracle.attention(q, k, v, sl, x.scale)
        calls += 1
        el = time.perf_counter() - t0
        if el >= target_s or calls >= 1000:
            break
    gbs = sample_bytes * calls / el / 1e9
    sample = (f"{calls} oracle call(s) over {rows} of {B} batch row(s) "
              f"({sample_bytes / 1e6:.1f} MB of K+V per call) in {el:.1f} s")
    # the same sample on one thread, for a quarter of the time (at least one call)
    oracle.set_threads(1)
    try:
        calls1 = 0
        t1 = time.perf_counter()
        while True:
            oracle.attention(q, k, v, sl, x.scale)
            calls1 += 1
            el1 = time.perf_counter() - t1
            if el1 >= target_s / 4 or calls1 >= 1000:
                break
    finally:
        oracle.set_threads(threads)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": sample, "us_per_call": round(el / calls * 1e6 * B / rows, 1),
            "one_thread": {"value": round(sample_bytes * calls1 / el1 / 1e9, 4), "unit": "GB/s",
                           "calls": calls1, "seconds": round(el1, 1)},
            "cpu": cpu_model()}


def fused_merge(B: int, Hkv: int, ns: int, cus: int) -> str:
    """How das_decode_attention runs phase 2 for this plan: in the decode
    kernel (the last workgroup of each (b, kv-head) merges), as a second
    kernel (lse_combine: more than 4 split workgroups per CU, or more
    (b, kv-head) pairs than the library's 65536 arrival counters), or not at
    all (a single split writes the output directly)."""
    if ns <= 1:
        return "none (one split)"
    if B * Hkv <= 65536 and B * Hkv * ns <= 4 * cus:
        return "fused"
    return "two kernels"


class Workload:
    """One config's inputs resident in HBM (K/V rotated over several copies so
    that back-to-back calls read from HBM, not from the last-level cache),
    with prepared library calls."""

    def __init__(self, args, config: int, kv_dtype: str = "bf16", paged: int = 0,
                 paged_layout: str = "hnd", hq: int = 0, copies: int = 0, x=None):
        import numpy as np
        import torch

        import decode_attention_split_amd as das
        import workloads

        self.torch, self.das = torch, das
        dev = torch.device("cuda:0")
        cfg = workloads.CONFIGS[config]
        if hq:
            import dataclasses
            cfg = dataclasses.replace(cfg, name=f"{cfg.name}_hq{hq}", Hq=hq,
                                      description=f"{cfg.description}, Hq={hq} instead")
        self.cfg = cfg
        self.kv_dtype = kv_dtype
        int4 = kv_dtype == "int4"
        fp8 = kv_dtype == "fp8"
        self.quant = quant = fp8 or int4      # codes plus fp32 scales
        self.paged = None
        if paged:
            layout = workloads.PAGED_HND if paged_layout == "hnd" else workloads.PAGED_NHD
            self.paged = workloads.make_paged_inputs(cfg, 42 + config, paged, layout, fp8=fp8,
                                                     int4=int4, base=x)
            x = self.paged.base
        elif x is None:
            if int4:
                x = workloads.make_int4_inputs(cfg, 42 + config)
            else:
                x = (workloads.make_fp8_inputs if fp8 else workloads.make_inputs)(cfg, 42 + config)
        self.x = x
        B, Hq, D = x.q.shape
        Hkv, Smax = x.k.shape[1], x.k.shape[2]
        self.kv_bytes = x.kv_bytes
        if self.paged is not None:
            # the paged plan: Smax = max_blocks * page size, chunks rounded up to whole pages
            Smax = self.paged.block_table.shape[1] * self.paged.page_size
        self.B, self.Hq, self.Hkv, self.Smax, self.D = B, Hq, Hkv, Smax, D
        self.kv_code = das.DAS_INT4 if int4 else (das.DAS_E4M3 if fp8 else das.DAS_BF16)
        self.cus = torch.cuda.get_device_properties(dev).multi_processor_count

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(dev)

        self.q = up(x.q)
        self.sl = torch.from_numpy(x.seq_lens).to(dev)
        k_scale = v_scale = None
        alloc = x.k.nbytes + x.v.nbytes
        if quant:
            if int4 and self.paged is not None:
                # an INT4 pool's row scales live in pools laid out like it
                k_scale = torch.from_numpy(self.paged.k_scale_pool).to(dev)
                v_scale = torch.from_numpy(self.paged.v_scale_pool).to(dev)
            else:
                k_scale = torch.from_numpy(x.k_scale).to(dev)
                v_scale = torch.from_numpy(x.v_scale).to(dev)
            if int4:
                alloc += x.k_scale.nbytes + x.v_scale.nbytes
        src_k, src_v = ((self.paged.k_pool, self.paged.v_pool) if self.paged is not None
                        else (x.k, x.v))
        if quant:
            k0, v0 = torch.from_numpy(src_k).to(dev), torch.from_numpy(src_v).to(dev)
        else:
            k0, v0 = up(src_k), up(src_v)
        self.table = None
        if self.paged is not None:
            alloc = self.paged.k_pool.nbytes + self.paged.v_pool.nbytes
            if int4:
                alloc += self.paged.k_scale_pool.nbytes + self.paged.v_scale_pool.nbytes
            self.table = torch.from_numpy(self.paged.block_table).to(dev)
        self.copies = copies or max(1, min(16, math.ceil(4 * LLC_BYTES / alloc)))
        self.ks, self.vs = [k0], [v0]
        self.kss, self.vss = [k_scale], [v_scale]
        for _ in range(self.copies - 1):
            self.ks.append(k0.clone())
            self.vs.append(v0.clone())
            # an INT4 cache's row scales are streamed with its codes: rotate them too
            self.kss.append(k_scale.clone() if int4 else k_scale)
            self.vss.append(v_scale.clone() if int4 else v_scale)
        self.k_scale, self.v_scale = k_scale, v_scale
        self.ws = {}

    def plan(self, splits: int):
        ns, chunk = self.das.das_plan_kv(self.kv_code, self.B, self.Hkv, self.Hq // self.Hkv,
                                         self.Smax, self.D, splits)
        if self.paged is not None and chunk % self.paged.page_size:
            P = self.paged.page_size
            chunk = -(-chunk // P) * P
            ns = -(-self.Smax // chunk)
        return ns, chunk

    def workspace(self, splits: int):
        if splits not in self.ws:
            n = self.das.das_decode_workspace_bytes(self.B, self.Hq, self.Hkv, self.Smax, self.D,
                                                    splits)
            # zero-filled: the workspace starts with the library's arrival counters
            self.ws[splits] = self.torch.zeros(max(n, 16), dtype=self.torch.uint8,
                                               device=self.q.device)
        return self.ws[splits]

    def calls(self, splits: int, out, lse, stream=None):
        """One prepared decode-attention call per K/V copy."""
        das, ws = self.das, self.workspace(splits)
        if self.paged is not None:
            return [das.prepare_decode_paged(self.q, self.ks[c], self.vs[c], self.table, self.sl,
                                             self.x.scale, self.paged.page_size,
                                             self.paged.layout, out, lse, splits, ws,
                                             stream=stream, k_scale=self.kss[c],
                                             v_scale=self.vss[c], kv_dtype=self.kv_code)
                    for c in range(self.copies)]
        if self.quant:
            name = ("das_decode_attention_int4" if self.kv_dtype == "int4"
                    else "das_decode_attention_fp8")
            return [das.prepare_decode(name, self.q, self.ks[c], self.vs[c], self.sl,
                                       self.x.scale, out, lse, splits, ws, stream=stream,
                                       k_scale=self.kss[c], v_scale=self.vss[c])
                    for c in range(self.copies)]
        return [das.prepare_decode("das_decode_attention", self.q, self.ks[c], self.vs[c],
                                   self.sl, self.x.scale, out, lse, splits, ws, stream=stream)
                for c in range(self.copies)]

    def outputs(self, out_dtype: str):
        torch = self.torch
        dt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
        return (torch.empty((self.B, self.Hq, self.D), dtype=dt, device=self.q.device),
                torch.empty((self.B, self.Hq), dtype=torch.float32, device=self.q.device))

    def event_us(self, calls, n: int, warmup: int, reps: int = 3) -> float:
        """µs per call: the median over `reps` runs of the average over n
        back-to-back launches, each run timed by a pair of HIP events on the
        launch stream (torch's current stream).  The warm-up is at least
        `warmup` calls and at least 20 ms of them, so that a row measured
        after the GPU sat idle (the CPU baseline runs before the table) does
        not catch it with its clocks still low; the median drops a single
        run that something else on the GPU slowed."""
        torch = self.torch
        t0 = time.perf_counter()
        i = 0
        while i < warmup or time.perf_counter() - t0 < 0.02:
            calls[i % len(calls)]()
            i += 1
            if i % 8 == 0:
                torch.cuda.synchronize()   # keep the host clock in step with the GPU
        torch.cuda.synchronize()
        runs = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                calls[i % len(calls)]()
                i += 1
            e1.record()
            torch.cuda.synchronize()
            runs.append(e0.elapsed_time(e1) / n * 1e3)
        return sorted(runs)[len(runs) // 2]

    def row(self, splits: int, out_dtype: str, n: int, warmup: int) -> dict:
        """One line of the per-config table."""
        out, lse = self.outputs(out_dtype)
        us = self.event_us(self.calls(splits, out, lse), n, warmup)
        ns, chunk = self.plan(splits)
        gbs = self.kv_bytes / (us * 1e-6) / 1e9
        pool = None
        if self.paged is not None:
            pool = (f"P={self.paged.page_size} "
                    f"{'HND' if self.paged.layout == self.das.DAS_PAGED_HND else 'NHD'}")
        return {"workload": self.cfg.name, "G": self.Hq // self.Hkv, "kv_dtype": self.kv_dtype,
                "paged": pool, "splits": "auto" if splits == 0 else splits,
                "plan": f"{ns} x {chunk}", "merge": fused_merge(self.B, self.Hkv, ns, self.cus),
                "out_dtype": out_dtype, "kv_bytes": self.kv_bytes, "us_per_call": round(us, 2),
                "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                "launches": f"median of 3 x {n}"}


# Page pools of the table's paged rows: page size and layout per cache format.
TABLE_POOLS = {"bf16": (256, "hnd"), "fp8": (64, "hnd"), "int4": (256, "hnd")}


def per_config_table(args, headline: "Workload") -> list:
    """Every named config in this process, µs per call by HIP events (the
    median of three runs of args.table_steps back-to-back launches):
    - bf16 K/V: the automatic plan with fp32 output, the same with bf16
      output, and one split (the unsplit kernel the pages start from);
    - the 32K-token cache of config 1 with other GQA groups: Hq = 8 and 16
      (G = 1, 2: the vector-ALU path at long context, the per-head grid of
      [FD++] §2) and Hq = 128 (G = 16);
    - the E4M3 and INT4 caches on configs 1-4, and page pools of each
      format ([FD++] §4 and §6) on configs 1-3 (bf16) and 3 (all three),
      with the automatic plan and fp32 output."""
    import workloads

    rows = []
    n = len(workloads.CONFIGS)

    def run(w, variants):
        for splits, out_dtype in variants:
            rows.append(w.row(splits, out_dtype, args.table_steps, args.table_warmup))
        label = w.cfg.name + ("" if w.kv_dtype == "bf16" else f" {w.kv_dtype}") + \
            ("" if w.paged is None else " paged")
        print(f"bench: table {label} done", file=sys.stderr, flush=True)

    def paged_rows(kv, idx, x):
        P, layout = TABLE_POOLS[kv]
        p = Workload(args, idx, kv, P, layout, x=x)
        run(p, ((0, "f32"),))
        del p

    # Freed device memory stays with torch's allocator (no empty_cache): memory
    # handed back to the driver is cleared by it in the background, which
    # slows the next rows' HBM stream for tens of milliseconds.
    auto = ((0, "f32"),)
    for idx in range(n):
        if headline is not None and idx == args.config and headline.kv_dtype == "bf16" \
                and headline.paged is None and not args.hq:
            w = headline
        else:
            w = Workload(args, idx)
        run(w, ((0, "f32"), (0, "bf16"), (1, "f32")))
        if 1 <= idx <= 3:   # the same rows from a bf16 page pool
            paged_rows("bf16", idx, w.x)
        if w is not headline:
            del w
    for hq in (8, 16, 128):
        w = Workload(args, 1, hq=hq)
        run(w, auto)
        del w
    for kv in ("fp8", "int4"):
        for idx in range(1, n):
            w = Workload(args, idx, kv)
            run(w, auto)
            if idx == 3:
                paged_rows(kv, idx, w.x)
            del w
    return rows


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.stderr.write("bench.py measures one GPU: this build has no multi-GPU path "
                         "(each GPU would run the same kernel on its own share of the "
                         "sequences); run with --gpus 1.\n")
        sys.exit(2)
    if args.op == "merge":
        bench_merge(args)
        return

    import numpy as np
    import torch

    import decode_attention_split_amd as das

    das.load_library()
    w = Workload(args, args.config, args.kv_dtype, args.paged, args.paged_layout, args.hq,
                 args.copies)
    cfg, x = w.cfg, w.x
    B, Hq, Hkv, Smax, D = w.B, w.Hq, w.Hkv, w.Smax, w.D
    kv_bytes = w.kv_bytes
    ns, chunk = w.plan(args.splits)
    out, lse = w.outputs(args.out_dtype)
    calls = w.calls(args.splits, out, lse)
    copies = w.copies

    # The timed region: exactly K steps, bracketed by synchronizes.  Each step
    # is one decode-attention call (one kernel launch, two where phase 2 runs
    # as its own kernel) on torch's current stream, so the events around the K
    # back-to-back launches give the call's average duration on the GPU.
    for i in range(args.warmup):
        calls[i % copies]()
    torch.cuda.synchronize()
    K = args.steps
    ev_start = torch.cuda.Event(enable_timing=True)
    ev_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_start.record()
    for i in range(K):
        calls[(args.warmup + i) % copies]()
    ev_end.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kernel_ms = ev_start.elapsed_time(ev_end) / K
    ms_per_step = elapsed / K * 1e3
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = kv_bytes / (kernel_ms * 1e-3) / 1e9
    print(f"bench: timed {K} steps of {cfg.name}", file=sys.stderr, flush=True)

    # For reference only (not `value`): the same K calls captured in one HIP
    # graph and replayed, as a serving engine issues a decode step.  The
    # library allocates and synchronises nothing, so its calls capture as is.
    graph_us = None
    if args.graph:
        gs = torch.cuda.Stream()
        gcalls = w.calls(args.splits, out, lse, stream=gs)
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=gs):
            for i in range(K):
                gcalls[i % copies]()
        graph.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record()
        graph.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_us = round(g0.elapsed_time(g1) / K * 1e3, 2)
        del graph

    # Also for reference: calls one at a time, each after a 1 GiB write that
    # evicts the cache (4x the 256 MB Infinity Cache) and between its own
    # pair of events; the median of 100.
    isolated_us = None
    if args.isolated:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=out.device)
        n = 100
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            flush.fill_(i & 255)
            evs[i][0].record()
            calls[i % copies]()
            evs[i][1].record()
        torch.cuda.synchronize()
        isolated_us = round(sorted(a.elapsed_time(b) for a, b in evs)[n // 2] * 1e3, 2)
        del flush

    quant, paged = w.quant, w.paged
    fp8, int4 = args.kv_dtype == "fp8", args.kv_dtype == "int4"
    merge = fused_merge(B, Hkv, ns, w.cus)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8-e4m3 K/V, bf16 q" if fp8 else
                  "int4 K/V with fp32 row scales, bf16 q" if int4 else "bf16"),
        "data": "synthetic",
        "config": {
            "workload": cfg.name,
            "description": cfg.description,
            "B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "Smax": Smax,
            "tokens": int(x.seq_lens.astype(np.int64).sum()),
            "kv_bytes": kv_bytes,
            "num_splits": ns, "chunk": chunk, "merge": merge,
            "out_dtype": args.out_dtype,
            "kv_dtype": args.kv_dtype,
            "paged": ({"page_size": paged.page_size, "layout": args.paged_layout}
                      if paged is not None else None),
            "kv_copies_rotated": copies,
            # value = kv_bytes / (host wall clock over the K timed steps, from
            # before the first launch to after the final synchronize) / K
            "value_clock": "host wall clock over the timed steps, incl. the final synchronize",
            "us_per_call": round(ms_per_step * 1e3, 2),
            "us_per_call_hip_events": round(kernel_ms * 1e3, 3),
            "us_per_call_graph_replay": graph_us,
            "us_per_call_isolated_median": isolated_us,
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("split_kv_decode + lse_combine" if merge == "two kernels"
                       else "split_kv_decode"),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if (args.hq or args.splits or args.out_dtype != "f32")
                       else measured_traffic(cfg.name, ns, args.kv_dtype, args.paged,
                                             args.paged_layout),
            "kernel_us": round(kernel_ms * 1e3, 3),
        },
    }
    if args.cpu_seconds > 0 and not quant and paged is None:
        result["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
        print("bench: cpu baseline done", file=sys.stderr, flush=True)
    if args.table:
        del calls
        result["config"]["per_config"] = per_config_table(args, w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
