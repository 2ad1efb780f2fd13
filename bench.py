#!/usr/bin/env python3
"""Benchmark: grouped-query attention decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one ``gqa_decode`` call over the whole batch (one kernel launch),
i.e. one layer's attention for one decode step.  Inputs are seeded
synthetic tensors already resident in HBM; before every timed step a 1 GiB
read sweeps the L2 and the Infinity Cache so that K/V come from HBM.
Time per step = (K x [sweep, step] back to back) - (K x [sweep]), over the
stream, i.e. the kernels' device time; isolated single-call times (which
also count a lone launch's dispatch latency) are reported beside it.

Useful bytes per step (the algorithmic traffic; "GQA (Grouped-Query
Attention) 분석", section "KV cache 용량", per layer and step):
    2 * sum_b(L_b) * G * D * s_kv   (K and V rows each read once)
  + |Q| + |O|                        (query in, fp32 output out)
The n_rep-times repeated K/V of a repeat_kv path is NOT counted.

Prints ONE JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import gqa_inputs as gi  # noqa: E402

METRIC = "GQA decode attention µs/step + achieved KV-read HBM GB/s (% of peak)"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
FLUSH_BYTES = 1 << 30
KERNEL_SOURCES = [os.path.join(ROOT, "grouped_query_attention_decode_amd", "csrc", f)
                  for f in ("gqa_kernels.hip", "gqa_api.cpp", "gqa_internal.h", "gqa_chunkmap.h")] + \
    [os.path.join(ROOT, "grouped_query_attention_decode_amd", "build.py")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Accounting
# ---------------------------------------------------------------------------
def kv_elem_bytes(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def kv_bytes(G, D, sum_len, dtype: str) -> int:
    """K and V rows each read once: 2 * sum_b(L_b) * G * D * s ("GQA
    (Grouped-Query Attention) 분석", section "KV cache 용량", per layer)."""
    return 2 * sum_len * G * D * kv_elem_bytes(dtype)


def q_bytes(B, H, D, sq, dtype: str) -> int:
    return B * H * sq * D * kv_elem_bytes(dtype)


def o_bytes(B, H, D, sq) -> int:
    return B * H * sq * D * 4      # fp32 output


def repeat_kv_bytes(B, H, D, sum_len, dtype: str) -> int:
    """What a repeat_kv path materialises per layer for K (and again for V):
    the cache expanded to one KV head per query head ("Same GQA, Different
    Execution Cost Across Backends", section 2).  Never allocated here; only
    reported beside the useful bytes."""
    return sum_len * H * D * kv_elem_bytes(dtype)


def useful_bytes(B, H, G, D, sq, sum_len, dtype: str) -> int:
    return kv_bytes(G, D, sum_len, dtype) + q_bytes(B, H, D, sq, dtype) + o_bytes(B, H, D, sq)


def code_cache_bytes(B, H, G, D, sq, sum_len, scales: bool) -> int:
    """useful_bytes for an 8-bit cache (fp8 E4M3 or int8 codes, one byte per
    K/V element) with bf16 queries: plus the two [G] fp32 scale arrays when
    the call reads them (not for a pool read with unit scales)."""
    return 2 * sum_len * G * D + q_bytes(B, H, D, sq, "bf16") + o_bytes(B, H, D, sq) + (2 * G * 4 if scales else 0)


def page_table_bytes(seq_lens, T: int, page_size: int) -> int:
    """Block-table entries a paged call reads: one int32 per page that holds
    a row below L_b (L_b clamped to [0, T])."""
    return 4 * sum((min(max(int(L), 0), T) + page_size - 1) // page_size for L in seq_lens)


def flops(H, D, sq, sum_len) -> int:
    """2 FLOP per multiply-add; scores and weighted sum each H*sq*L*D MACs
    ("질의 헤드는 그대로, 키·값 헤드만 줄인다", section on what shrinks: the
    attention body's multiply count has no g term)."""
    return 4 * H * sq * sum_len * D


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _counter_rows(run_dir: str, counter: str) -> dict:
    """Per-kernel values of one counter from a rocprofv3 --pmc csv run."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % run_dir)
    out = {}
    for path in files:
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter:
                    out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def write_traffic_record(args) -> int:
    """profiles/traffic_<workload>[_<mode>].json from two rocprofv3 --pmc runs
    of this benchmark with --copy-probe (FETCH_SIZE, then WRITE_SIZE): the
    decode kernel's KiB per dispatch, each scaled by what the same counter
    reads for the 1 GiB device copy (1 GiB read, 1 GiB written)."""
    fetch_dir, write_dir = args.traffic_record
    fe = _counter_rows(fetch_dir, "FETCH_SIZE")
    wr = _counter_rows(write_dir, "WRITE_SIZE")
    ours = [k for k in fe if "gqa::" in k]
    kn = max(ours, key=lambda k: sum(fe[k]) / len(fe[k]))      # the dominant (decode) kernel
    cp = [k for k in fe if "copyBuffer" in k]
    if len(cp) != 1 or cp[0] not in wr or kn not in wr:
        raise SystemExit("expected one copy kernel and the decode kernel in both runs")
    kib = 1 << 20                                               # the copy moves 1 GiB each way
    cf, cw = max(fe[cp[0]]), max(wr[cp[0]])
    rs, ws = kib / cf, kib / cw
    f = sum(fe[kn]) / len(fe[kn])
    w = sum(wr[kn]) / len(wr[kn])
    name = args.workload if args.mode == "decode" else "%s_%s" % (args.workload, args.mode)
    extra = "" if args.mode == "decode" else " --mode %s" % args.mode
    rec = {
        "kernel": kn.split("(")[0].replace("void ", "").replace("gqa::", ""),
        "workload": name,
        "kernel_source_sha": kernel_source_sha(),
        "dispatches": len(fe[kn]),
        "fetch_size_kib_per_dispatch": f,
        "write_size_kib_per_dispatch": w,
        "read_scale": rs,
        "write_scale": ws,
        "calibration": "1 GiB device copy (%s): FETCH_SIZE %.1f KiB, WRITE_SIZE %.1f KiB for %d KiB "
                       "each way" % (cp[0].split("(")[0], cf, cw, kib),
        "hbm_bytes_per_launch": int(round((f * rs + w * ws) * 1024)),
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s -o run -- python3 bench.py --no-cpu "
            "--steps 5 --warmup 1 --copy-probe --workload %s%s" % (fetch_dir, args.workload, extra),
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s -o run -- python3 bench.py --no-cpu "
            "--steps 5 --warmup 1 --copy-probe --workload %s%s" % (write_dir, args.workload, extra),
            "python3 bench.py --workload %s%s --traffic-record %s %s" % (args.workload, extra, fetch_dir,
                                                                         write_dir)],
    }
    out = os.path.join(ROOT, "profiles", "traffic_%s.json" % name)
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec, indent=1))
    return 0


def load_traffic(workload: str, sha: str):
    """HBM bytes per split launch from committed rocprofv3 counter runs, or
    None when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != sha:
        return None
    return t


def kernel_name(plan):
    """The decode kernel a plan launches (the dominant kernel of a step)."""
    if plan["path"] != 2:
        return {1: "decode_valu", 3: "decode_mqk"}[plan["path"]]
    if plan["waves_per_group"] == 1:
        return "decode_mfa"                  # one-wave 16 x 16 kernel
    if plan["row_block"] == 16:
        return "decode_mfs"                  # row-split workgroups of the 16 x 16 kernel
    return "decode_mfw" if os.environ.get("GQA_MFX") == "0" else "decode_mfx"


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on the host cores
# ---------------------------------------------------------------------------

def cpu_model() -> str:
    """The host CPU's model name (as lscpu prints it), from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _time_oracle(args, threads: int, seconds: float):
    import oracle
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.decode_f64(*args, threads=threads)
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return passes, el


def cpu_baseline(x_cpu, w, sum_len, seconds: float):
    """The float64 oracle timed on the host: the whole workload on the
    threads this process may use (at most 16: the CPU share of one GPU on
    the box), and single-threaded on the first sequences (a bounded sample
    of the same workload, scaled to the whole by its useful bytes)."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    threads = max(1, min(16, os.cpu_count() or 1))
    q = x_cpu["q"].double().numpy()
    k = x_cpu["k"].double().numpy()
    v = x_cpu["v"].double().numpy()
    sl = x_cpu["seq_lens"].numpy().astype(np.int32)
    scale = 1.0 / math.sqrt(w.D)
    passes, el = _time_oracle((q, k, v, sl, scale), threads, seconds)
    per = el / passes
    ub = useful_bytes(w.B, w.H, w.G, w.D, w.sq, sum_len, w.dtype)
    # single thread: the first nb sequences
    nb = max(1, min(w.B, 2))
    sl1 = sl[:nb]
    sum1 = int(np.clip(sl1, 0, w.T).sum())
    p1, el1 = _time_oracle((q[:nb], k[:nb], v[:nb], sl1, scale), 1, seconds)
    ub1 = useful_bytes(nb, w.H, w.G, w.D, w.sq, sum1, w.dtype)
    return {"value": ub / per / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "whole workload (%d sequences), %d passes in %.1f s, float64, "
                      "%d threads; %.1f ms per pass" % (w.B, passes, el, threads, per * 1e3),
            "single_thread": {"value": ub1 / (el1 / p1) / 1e9, "unit": "GB/s", "cores": 1,
                              "sample": "first %d sequence(s) (%d cache rows), %d passes in %.1f s"
                                        % (nb, sum1, p1, el1)},
            "host": {"cpu_model": cpu_model(), "logical_cpus": os.cpu_count(),
                     "threads_used": threads}}


def parity_spot_check(args, w, x, out, extra):
    """Part of the CPU-baseline leg: the float64 oracle on sequence 0 of this
    very run, against the last step's output (max abs error)."""
    import numpy as np
    import oracle
    b = 0
    xb = {k: v[b:b + 1].cpu() for k, v in x.items()}
    scale = 1.0 / math.sqrt(w.D)
    codes = args.mode if args.mode in ("fp8", "int8") else args.page_codes if args.mode == "paged" else "none"
    if codes != "none":
        kq, vq, ks, vs = extra
        fn = oracle.decode_fp8_f64 if codes == "fp8" else oracle.decode_int8_f64
        want = fn(xb["q"], kq[b:b + 1].cpu(), vq[b:b + 1].cpu(), ks.cpu(), vs.cpu(), xb["seq_lens"], scale,
                  threads=8)
        if args.mode == "paged":
            out = out * vs[0].item()      # the V scale a caller applies to a pool read with unit scales
    elif args.mode == "append":
        kn, vn = extra
        # the cache already holds the appended rows (every step stores the same ones)
        want, _, _ = oracle.decode_append_f64(xb["q"], kn[b:b + 1].cpu(), vn[b:b + 1].cpu(), xb["k"],
                                              xb["v"], xb["seq_lens"], scale, threads=8)
    else:
        want = oracle.decode_f64(xb["q"], xb["k"], xb["v"], xb["seq_lens"], scale, threads=8)
    return float(np.abs(out[b:b + 1].double().cpu().numpy() - want).max())


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------
def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=gi.HEADLINE, choices=sorted(gi.WORKLOADS))
    ap.add_argument("--workgroups", type=int, default=0)
    ap.add_argument("--path", default="auto", choices=["auto", "valu", "mfma", "mfma_qk"])
    ap.add_argument("--merge", default="auto", choices=["auto", "kernel", "combine"])
    ap.add_argument("--mode", default="decode", choices=["decode", "append", "paged", "fp8", "int8"],
                    help="decode: gqa_decode; append: gqa_decode_append (the sq new tokens' K/V "
                         "stored and attended in one pass); paged: gqa_decode_paged over a "
                         "randomly ordered page pool; fp8: gqa_decode_fp8 over E4M3 codes with "
                         "per-KV-head scales (amax / 448)")
    ap.add_argument("--page-size", type=int, default=16)
    ap.add_argument("--page-codes", default="none", choices=["none", "fp8", "int8"],
                    help="paged mode: a pool of 8-bit codes read with unit scales -- E4M3 of the "
                         "cache values, or int8 round(32 x value) with 1/32 folded into the score "
                         "scale and applied to the output")
    ap.add_argument("--flush-mib", type=int, default=FLUSH_BYTES >> 20,
                    help="size of the read sweep before every step, in MiB (at least twice the "
                         "256 MB Infinity Cache)")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the cache sweep (warm-cache numbers; not HBM rates)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also time a plain 1 GiB device copy (bandwidth reference, "
                         "and the calibration kernel for HBM byte counters)")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="host only: write profiles/traffic_<workload>.json from two rocprofv3 "
                         "--pmc runs of this command with --copy-probe (FETCH_SIZE, then WRITE_SIZE)")
    args = ap.parse_args(argv)
    if args.traffic_record:
        return write_traffic_record(args)
    if not args.no_flush and args.flush_mib < 512:
        print("--flush-mib must be at least 512 (twice the 256 MB Infinity Cache)", file=sys.stderr)
        return 2

    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2
    if os.environ.get("WORLD_SIZE", "1") not in ("", "1"):
        print("bench.py runs on exactly one GPU (WORLD_SIZE=%s)" % os.environ["WORLD_SIZE"],
              file=sys.stderr)
        return 2

    import torch
    import grouped_query_attention_decode_amd as gqa
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    gqa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    w = gi.WORKLOADS[args.workload]
    log("[bench] workload %s: drawing inputs on the GPU" % w.name)
    x = gi.make_inputs(w, device=dev)
    sum_len = int(x["seq_lens"].clamp(0, w.T).sum().item())
    ub = useful_bytes(w.B, w.H, w.G, w.D, w.sq, sum_len, w.dtype)
    path = {"auto": gqa.PATH_AUTO, "valu": gqa.PATH_VALU, "mfma": gqa.PATH_MFMA,
            "mfma_qk": gqa.PATH_MFMA_QK}[args.path]
    shape = gqa.shape_of(x["q"], x["k"])
    merge = {"auto": gqa.MERGE_AUTO, "kernel": gqa.MERGE_IN_KERNEL, "combine": gqa.MERGE_COMBINE}[args.merge]
    plan = gqa.plan(shape, path=path, workgroups=args.workgroups, merge=merge)
    log("[bench] plan %s" % plan)
    out = torch.empty(x["q"].shape, dtype=torch.float32, device=dev)
    flush_bytes = args.flush_mib << 20
    flush = torch.empty(flush_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    stream = torch.cuda.current_stream(dev)

    if args.mode == "append":
        gen = torch.Generator(device=dev).manual_seed(w.seed + 7)
        kn = torch.randn(w.B, w.G, w.sq, w.D, generator=gen, device=dev).to(x["k"].dtype)
        vn = torch.randn(w.B, w.G, w.sq, w.D, generator=gen, device=dev).to(x["k"].dtype)
        ub += 2 * w.B * w.G * w.sq * w.D * kv_elem_bytes(w.dtype)      # the stored rows

        def call():
            gqa.decode_append(x["q"], kn, vn, x["k"], x["v"], x["seq_lens"], None, out, path=path,
                              workgroups=args.workgroups, merge=merge, stream=stream)
    elif args.mode == "paged":
        ps = args.page_size
        n = w.T // ps
        perm = torch.randperm(w.B * n, generator=torch.Generator().manual_seed(w.seed + 11))
        page_scale, pscore = 1.0, None
        if args.page_codes == "fp8":
            kc = x["k"].float().to(torch.float8_e4m3fn).view(torch.uint8)
            vc = x["v"].float().to(torch.float8_e4m3fn).view(torch.uint8)
        elif args.page_codes == "int8":
            page_scale = 1.0 / 32
            kc = torch.round(x["k"].float() * 32).clamp(-128, 127).to(torch.int8)
            vc = torch.round(x["v"].float() * 32).clamp(-128, 127).to(torch.int8)
        else:
            kc, vc = x["k"], x["v"]
        if args.page_codes != "none":
            pscore = page_scale / math.sqrt(w.D)
            ub = code_cache_bytes(w.B, w.H, w.G, w.D, w.sq, sum_len, scales=False)
        kp = torch.empty(w.B * n, w.G, ps, w.D, dtype=kc.dtype, device=dev)
        vp = torch.empty_like(kp)
        idx = perm.view(w.B, n).to(dev)
        kp[idx.reshape(-1)] = kc.view(w.B, w.G, n, ps, w.D).transpose(1, 2).reshape(w.B * n, w.G, ps, w.D)
        vp[idx.reshape(-1)] = vc.view(w.B, w.G, n, ps, w.D).transpose(1, 2).reshape(w.B * n, w.G, ps, w.D)
        bt = idx.to(torch.int32).contiguous()
        ub += page_table_bytes(x["seq_lens"].tolist(), w.T, ps)

        def call():
            gqa.decode_paged(x["q"], kp, vp, bt, x["seq_lens"], pscore, out, path=path,
                             workgroups=args.workgroups, merge=merge, stream=stream)
    elif args.mode == "fp8":
        def quant(t):
            amax = t.float().abs().amax(dim=(0, 2, 3)).clamp_min(1e-6)
            sc = (amax / 448.0).float().contiguous()
            return (t.float() / sc.view(1, -1, 1, 1)).to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), sc
        kq, ks = quant(x["k"])
        vq, vs = quant(x["v"])
        plan = gqa.plan(gqa.shape_of(x["q"], kq), path=path, workgroups=args.workgroups, merge=merge)
        log("[bench] fp8 plan %s" % plan)
        ub = code_cache_bytes(w.B, w.H, w.G, w.D, w.sq, sum_len, scales=True)

        def call():
            gqa.decode_fp8(x["q"], kq, vq, ks, vs, x["seq_lens"], None, out,
                           workgroups=args.workgroups, merge=merge, stream=stream)
    elif args.mode == "int8":
        def quant8(t):
            amax = t.float().abs().amax(dim=(0, 2, 3)).clamp_min(1e-6)
            sc = (amax / 127.0).float().contiguous()
            return torch.round(t.float() / sc.view(1, -1, 1, 1)).clamp(-128, 127).to(torch.int8).contiguous(), sc
        kq, ks = quant8(x["k"])
        vq, vs = quant8(x["v"])
        plan = gqa.plan(gqa.shape_of(x["q"], kq), path=path, workgroups=args.workgroups, merge=merge)
        log("[bench] int8 plan %s" % plan)
        ub = code_cache_bytes(w.B, w.H, w.G, w.D, w.sq, sum_len, scales=True)

        def call():
            gqa.decode_int8(x["q"], kq, vq, ks, vs, x["seq_lens"], None, out,
                            workgroups=args.workgroups, merge=merge, stream=stream)
    else:
        def call():
            gqa.decode(x["q"], x["k"], x["v"], x["seq_lens"], None, out, path=path,
                       workgroups=args.workgroups, merge=merge, stream=stream)

    for _ in range(args.warmup):
        if not args.no_flush:
            flush.sum()
        call()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]

    # (1) Each step alone: events right around the decode call.  This also
    #     counts the dispatch latency of a lone launch (a few us).
    log("[bench] timing %d isolated steps" % K)
    torch.cuda.synchronize()
    for i in range(K):
        if not args.no_flush:
            flush.sum()
        ev[i][0].record(stream)
        call()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    iso_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]

    # (2) The timed region, bracketed by synchronize on both sides: K steps
    #     back to back, each after the cache sweep, in blocks that alternate
    #     with blocks of the same number of sweeps alone; per step, the
    #     difference of the two totals.  Launches queue behind the sweeps, so
    #     dispatch latency is hidden as in a decode loop and the difference is
    #     the kernels' device time -- what rocprofv3 reports per launch.
    #     Alternating short blocks cancels slow drift of the sweep's own speed
    #     (clocks, power), which two long loops one after the other do not.
    nblk = min(K, 10)
    sizes = [K // nblk + (1 if b < K % nblk else 0) for b in range(nblk)]
    ev_run = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nblk)]
    ev_swp = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nblk)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for b in range(nblk):
        ev_run[b][0].record(stream)
        for i in range(sizes[b]):
            if not args.no_flush:
                flush.sum()
            call()
        ev_run[b][1].record(stream)
        ev_swp[b][0].record(stream)
        for i in range(sizes[b]):
            if not args.no_flush:
                flush.sum()
        ev_swp[b][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    run_ms = sum(e[0].elapsed_time(e[1]) for e in ev_run)
    swp_ms = sum(e[0].elapsed_time(e[1]) for e in ev_swp)
    ms = (run_ms - swp_ms) / K
    blk_us = sorted((ev_run[b][0].elapsed_time(ev_run[b][1]) - ev_swp[b][0].elapsed_time(ev_swp[b][1]))
                    / sizes[b] * 1e3 for b in range(nblk))
    step_ms = iso_ms
    q = statistics.quantiles(step_ms, n=10) if K >= 10 else [min(step_ms)] * 9

    # warm-cache reference (labelled; never reported as an HBM rate)
    warm = []
    for i in range(min(K, 20)):
        ev[i][0].record(stream)
        call()
        ev[i][1].record(stream)
        torch.cuda.synchronize()
        warm.append(ev[i][0].elapsed_time(ev[i][1]))

    gbs = ub / (ms * 1e-3) / 1e9
    achieved = gbs      # one kernel per step: the step is the kernel
    sha = kernel_source_sha()
    mode_key = args.mode + ("_" + args.page_codes if args.mode == "paged" and args.page_codes != "none" else "")
    traffic = load_traffic(w.name if args.mode == "decode" else "%s_%s" % (w.name, mode_key), sha)
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "G": w.G, "D": w.D, "T": w.T,
            "sq": w.sq, "seq_lens": ("uniform [%d, %d], seed %d" % (w.ragged[0], w.ragged[1], w.seed)
                                     if w.ragged else "all T"),
            "sum_seq_lens": sum_len,
            "kv_dtype": {"fp8": "fp8_e4m3", "int8": "int8"}.get(
                args.page_codes if args.mode == "paged" else args.mode, w.dtype),
            "out_dtype": "f32",
            "cache": "no sweep (warm)" if args.no_flush else "%d MiB read sweep before each step" % args.flush_mib,
            "path": {1: "valu", 2: "mfma", 3: "mfma_qk"}.get(plan["path"], "?"),
            "workgroups": plan["workgroups"],
            "waves_per_group": plan["waves_per_group"],
            "combine_kernel": bool(plan["combine"]),
            "mode": args.mode,
            **({"page_size": args.page_size, "page_codes": args.page_codes} if args.mode == "paged" else {}),
        },
        "us_per_step": round(ms * 1e3, 2),
        "timing": "device time per step: K steps back to back after cache sweeps, minus as many sweeps alone, in %d alternating blocks" % nblk,
        "block_us_min_max": [round(blk_us[0], 2), round(blk_us[-1], 2)],
        "isolated_call_us_p10": round(q[0] * 1e3, 2),
        "isolated_call_us_p50": round(statistics.median(step_ms) * 1e3, 2),
        "isolated_call_us_p90": round(q[8] * 1e3, 2),
        "frac_of_peak_hbm": round(gbs / PEAK_HBM_GBS, 4),
        "useful_bytes": ub,
        "flops": flops(w.H, w.D, w.sq, sum_len),
        "warm_cache_us_per_step": round(statistics.median(warm) * 1e3, 2),
        "wall_ms_per_step_incl_two_sweeps": round(wall / K * 1e3, 4),
        # the cache sweeps timed alone are a measured read-bandwidth probe: a
        # 1 GiB fp32 sum (torch's reduction kernel) per sweep
        "read_probe": (None if args.no_flush else {
            "bytes": flush_bytes, "us": round(swp_ms / K * 1e3, 2),
            "gbs": round(flush_bytes / (swp_ms / K * 1e-3) / 1e9, 1),
            "kernel": "torch sum over a %d MiB fp32 tensor" % args.flush_mib}),
        "max_abs_err_vs_oracle_b0": None,
        "roofline": {
            "bound": "hbm",
            "kernel": kernel_name(plan),
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": (None if traffic is None else traffic["hbm_bytes_per_launch"]),
            "algorithmic_bytes_per_launch": ub,
        },
        "cpu_baseline": None,
    }
    if args.copy_probe:
        src_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev).fill_(2.0)
        dst_buf = torch.empty_like(src_buf)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(10):
            flush.sum()
            e0.record(stream)
            dst_buf.copy_(src_buf)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        result["copy_probe"] = {"bytes_read": FLUSH_BYTES, "bytes_written": FLUSH_BYTES,
                                "us": round(statistics.median(times) * 1e3, 2),
                                "gbs_read_plus_write": round(2 * FLUSH_BYTES / (statistics.median(times) * 1e-3) / 1e9, 1)}
        del src_buf, dst_buf
    if traffic is not None:
        result["roofline"]["traffic_over_algorithmic"] = round(
            traffic["hbm_bytes_per_launch"] / ub, 3)
    if not args.no_cpu:
        # the CPU-baseline leg: the only part of this script that runs the oracle
        log("[bench] timing the float64 oracle on the host (~%.0f s)" % args.cpu_seconds)
        del flush
        extra = (kq, vq, ks, vs) if args.mode in ("fp8", "int8") else (kn, vn) if args.mode == "append" else None
        if args.mode == "paged" and args.page_codes != "none":
            one = torch.full((w.G,), page_scale)
            extra = (kc, vc, one, one)
        try:
            result["max_abs_err_vs_oracle_b0"] = parity_spot_check(args, w, x, out, extra)
        except Exception as e:  # noqa: BLE001
            log("[bench] parity spot check skipped: %s" % e)
        xc = {k: v.cpu() for k, v in x.items()}
        result["cpu_baseline"] = cpu_baseline(xc, w, sum_len, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
