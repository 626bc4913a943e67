"""Benchmark of the batch-invariant GEMM and attention kernels on one MI355X.

One step = one pass of the whole hot path over the seeded synthetic workload
of the bf16 linear / addmm configuration (K = 4096, N in {4096, 14336},
M in {1, 2, 3, 4, 7, 8, 16, 33, 64, 128, 256}, bias added, alpha = beta = 1)
plus the bf16 causal GQA attention sweep (Hq = 32, Hkv = 8, D = 128, KV cache
1024, q_len in {1, 2, 4, 8, 9, 16, 64}).

The step is captured as HIP graphs, one per kernel configuration, replayed
back to back; events between the replays time each configuration inside the
timed region, which gives the per-launch average of the dominant kernel for
the roofline.  Weight matrices rotate through enough copies to exceed the
256 MB Infinity Cache, so weight reads come from HBM.  After timing, the
outputs of every batch size are compared bit for bit with the largest batch
(GEMM) and with the longest query chunk (attention).

Prints one JSON line on stdout; progress goes to stderr.

Profiling helpers (used to make the summaries kept under profiles/):
  --pmc-pass ORDER.json   run one step eagerly (no graphs) after a 256 MiB
                          calibration copy and write the dispatch order, for
                          `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE`;
  --summarize-pmc FETCH_DIR WRITE_DIR --order ORDER.json --out FILE.md
                          per-launch HBM traffic of every kernel group,
                          scaled by the calibration copy;
  --summarize-stats KERNEL_STATS.csv --out FILE.md --title T --cmd C
                          the rocprofv3 kernel statistics as a table.
The roofline's "traffic" is read from the committed traffic summary and
reported only while the kernel sources still hash to the value recorded
when the counters were taken.
"""
from __future__ import annotations

import argparse
import contextlib
import csv
import ctypes
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # dense bf16 MFMA
CSRC = os.path.join(ROOT, "invariant_deterministic_gemm_amd", "csrc")
TRAFFIC_MD = os.path.join(ROOT, "profiles", "bench_step_bf16_gemm_sweep_sdpa_sweep_hbm_traffic.md")
CALIB_BYTES = 256 * 2 ** 20     # bytes read and bytes written by the calibration copy
# sources whose text fixes each kernel family's memory traffic
FAMILY_SOURCES = {
    "gemm": ["device.h", "gemm.h", "gemm_common.h", "gemm16.h", "gemm16_store.h", "gemm16.hip", "gemm.hip", "api.hip"],
    "sdpa": ["device.h", "sdpa.h", "sdpa.hip", "api.hip"],
}


def family_hash(family: str) -> str:
    h = hashlib.sha256()
    for f in FAMILY_SOURCES[family]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-cells", action="store_true", help="skip the per-cell roofline table")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--samples", type=int, default=200, help="timed graph replays per graded cell")
    ap.add_argument("--cell", action="append", default=[], choices=sorted(CELLS),
                    help="measure only these cells (no step, no CPU baseline); repeatable")
    ap.add_argument("--eager", action="store_true", help="with --cell: direct calls instead of graph replays")
    ap.add_argument("--summarize-counters", metavar="DIR", action="append", default=[],
                    help="per-dispatch averages of the counters under DIR for kernels matching --kernel")
    ap.add_argument("--kernel", action="append", default=[])
    ap.add_argument("--pmc-pass", metavar="ORDER_JSON", default=None,
                    help="run one eager step for counter collection and write its dispatch order")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None)
    ap.add_argument("--summarize-stats", metavar="KERNEL_STATS_CSV", default=None)
    ap.add_argument("--order", default=None)
    ap.add_argument("--out", default=None)
    ap.add_argument("--title", default="")
    ap.add_argument("--cmd", action="append", default=[])
    return ap.parse_args()


def build_step(torch, bi, lib, _native, synthetic, dev):
    """Inputs of the step, its launches and their grouping by kernel configuration."""
    K = synthetic.CFG2["K"]
    Ms = synthetic.CFG2["M_values"]
    Ns = synthetic.CFG2["N_values"]
    Mmax = max(Ms)
    t0 = time.time()
    data = {}
    copies = {N: rotation(2.0 * N * K) for N in Ns}     # >= 2 x 256 MB of weights per N
    for N in Ns:
        d = synthetic.cfg2_inputs(N, M_max=Mmax)
        w = d["w"].to(dev)
        ws = [w] + [w.clone() for _ in range(copies[N] - 1)]
        # addmm(b, x, W^T) with W^T the transposed view of the (N, K) weight, as a linear layer calls it
        wts = [wc.t() for wc in ws]
        data[N] = dict(x=d["x"].to(dev), w=ws, wt=wts, b=d["b"].to(dev),
                       sha=synthetic.sha256(d["w"]))
    c3 = synthetic.cfg3_inputs(B=1, S=synthetic.CFG3["S"])
    q3, k3, v3 = (c3[n].to(dev) for n in ("q", "k", "v"))
    S3 = synthetic.CFG3["S"]
    Lqs = synthetic.CFG3["Lq_values"]
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")

    launches = []     # (group, kind, fn, flops, bytes, meta)
    ctr = {N: 0 for N in Ns}
    for N in Ns:
        dN = data[N]
        for M in Ms:
            for form in ("linear", "addmm"):
                i = ctr[N] % copies[N]
                ctr[N] += 1
                kname = lib.bi_gemm_kernel_name(M, N, K, _native.BI_BF16, 0).decode()
                if form == "linear":
                    fn = (lambda x=dN["x"][:M], w=dN["w"][i], b=dN["b"]: bi.bi_linear(x, w, b))
                else:
                    fn = (lambda x=dN["x"][:M], wt=dN["wt"][i], b=dN["b"]: bi.bi_addmm(b, x, wt, 1.0, 1.0))
                flops = 2.0 * M * N * K + M * N
                nbytes = 2.0 * (M * K + N * K + M * N + N)
                launches.append((kname, "gemm", fn, flops, nbytes, dict(N=N, M=M, form=form)))
    for L in Lqs:
        sname = lib.bi_sdpa_kernel_name(1, 32, 8, L, S3, 128, _native.BI_BF16).decode()
        fn = (lambda L=L: bi.bi_sdpa(q3[:, :, S3 - L:], k3, v3, causal=True))
        nbytes = 2.0 * (2 * 8 * S3 * 128 + 2 * 32 * L * 128)
        vis = sum(S3 - L + i + 1 for i in range(L))
        flops = 4.0 * 32 * 128 * vis
        launches.append((sname, "sdpa", fn, flops, nbytes, dict(Lq=L)))

    groups = {}
    for rec in launches:
        groups.setdefault(rec[0], []).append(rec)
    return dict(K=K, Ms=Ms, Ns=Ns, data=data, q3=q3, k3=k3, v3=v3, S3=S3, launches=launches,
                groups=groups, names=list(groups))


def main():
    args = parse()
    if args.summarize_stats:
        summarize_stats(args)
        return
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library runs on one GPU and has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import invariant_deterministic_gemm_amd as bi
    import synthetic
    from invariant_deterministic_gemm_amd import _native

    lib = _native.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.cell:
        # chosen cells only (used for the profiles of single kernels)
        global EAGER
        EAGER = args.eager
        if EAGER:
            _calibration_copy(torch)
        ctx = Ctx(torch, bi, lib, dev, synthetic, args.samples)
        cells = measure_cells(ctx, args.cell)
        print(json.dumps({"cells": cells}), flush=True)
        return
    st = build_step(torch, bi, lib, _native, synthetic, dev)
    if args.pmc_pass:
        pmc_pass(torch, st, args.pmc_pass)
        return
    K, Ms, Ns, data = st["K"], st["Ms"], st["Ns"], st["data"]
    q3, k3, v3, S3 = st["q3"], st["k3"], st["v3"], st["S3"]
    launches, groups, names = st["launches"], st["groups"], st["names"]

    # warm every path eagerly once, then capture one graph per group
    for rec in launches:
        rec[2]()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for rec in launches:
            rec[2]()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs, outs = {}, {}
    for g in names:
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            outs[g] = [rec[2]() for rec in groups[g]]
        graphs[g] = gr
    torch.cuda.synchronize()
    log(f"captured {len(names)} graphs over {len(launches)} launches")

    def run_step(evs=None):
        for j, g in enumerate(names):
            if evs is not None:
                evs[j][0].record()
            graphs[g].replay()
            if evs is not None:
                evs[j][1].record()

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    K_steps = args.steps
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in names] for _ in range(K_steps)]
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(K_steps + 1)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    step_ev[0].record()
    for s in range(K_steps):
        run_step(evs[s])
        step_ev[s + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gpu_ms = step_ev[0].elapsed_time(step_ev[-1])
    ms_per_step = wall * 1e3 / K_steps
    group_ms = {g: sum(evs[s][j][0].elapsed_time(evs[s][j][1]) for s in range(K_steps)) / K_steps
                for j, g in enumerate(names)}
    log(f"timed {K_steps} steps: wall {ms_per_step:.3f} ms/step, gpu events {gpu_ms / K_steps:.3f} ms/step")

    gemm_flops = sum(r[3] for r in launches if r[1] == "gemm")
    gemm_ms = sum(group_ms[g] for g in names if groups[g][0][1] == "gemm")
    sdpa_bytes = sum(r[4] for r in launches if r[1] == "sdpa")
    sdpa_ms = sum(group_ms[g] for g in names if groups[g][0][1] == "sdpa")
    # whole-step GEMM throughput over the wall-clock step (attention time included in the denominator)
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12

    # ------------------------------------------------------------ bit checks (outside the timed region)
    diff_rows = 0
    checked_rows = 0
    for N in Ns:
        dN = data[N]
        for form in ("linear", "addmm"):
            if form == "linear":
                ref = bi.bi_linear(dN["x"], dN["w"][0], dN["b"])
            else:
                ref = bi.bi_addmm(dN["b"], dN["x"], dN["wt"][0], 1.0, 1.0)
            for g in names:
                for rec, out in zip(groups[g], outs[g]):
                    meta = rec[5]
                    if rec[1] != "gemm" or meta["N"] != N or meta["form"] != form:
                        continue
                    M = meta["M"]
                    neq = (out.view(torch.int16) != ref[:M].view(torch.int16)).any(dim=1)
                    diff_rows += int(neq.sum().item())
                    checked_rows += M
    ref_o = bi.bi_sdpa(q3[:, :, S3 - 64:], k3, v3, causal=True)
    for rec, out in ((r, o) for g in names for r, o in zip(groups[g], outs[g]) if r[1] == "sdpa"):
        L = rec[5]["Lq"]
        neq = (out.view(torch.int16) != ref_o[:, :, 64 - L:].view(torch.int16)).any(dim=-1)
        diff_rows += int(neq.sum().item())
        checked_rows += int(neq.numel())
    log(f"bit check: {diff_rows} of {checked_rows} rows differ")

    # ------------------------------------------------------------ dominant kernel roofline
    dom = max(names, key=lambda g: group_ms[g])
    dl = groups[dom]
    avg_ms = group_ms[dom] / len(dl)
    if dl[0][1] == "gemm" and all(r[5]["M"] <= 64 for r in dl):
        bound, unit, peak = "hbm", "GB/s", HBM_PEAK_GBPS
        per_launch = sum(r[4] for r in dl) / len(dl)
        achieved = per_launch / (avg_ms * 1e-3) / 1e9
    elif dl[0][1] == "gemm":
        bound, unit, peak = "mfma", "TFLOP/s", BF16_PEAK_TFLOPS
        per_launch = sum(r[3] for r in dl) / len(dl)
        achieved = per_launch / (avg_ms * 1e-3) / 1e12
    else:
        bound, unit, peak = "hbm", "GB/s", HBM_PEAK_GBPS
        per_launch = sum(r[4] for r in dl) / len(dl)
        achieved = per_launch / (avg_ms * 1e-3) / 1e9
    roofline = {"bound": bound, "kernel": dom, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(dom, dl[0][1]),
                "launches_per_step": len(dl), "avg_launch_us": round(avg_ms * 1e3, 3),
                "algorithmic_per_launch": per_launch}

    # ------------------------------------------------------------ per-cell table (outside the step)
    cells = {}
    if not args.no_cells:
        cells = measure_cells(Ctx(torch, bi, lib, dev, synthetic, args.samples, data))

    # ------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(torch, synthetic, args)

    out = {
        "metric": "invariant GEMM TFLOP/s + SDPA GB/s at 1 GPU; bit-differing rows across batch = 0",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bf16 linear+addmm K=4096 N={4096,14336} M-sweep {1..256} "
                               "+ bf16 causal GQA SDPA Hq=32 Hkv=8 D=128 S=1024 q_len-sweep",
                   "global_batch": sum(Ms), "seq_len": S3, "parallelism": "none (1 GPU)"},
        "gemm_tflops_gpu_time": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 3),
        "sdpa_GBps": round(sdpa_bytes / (sdpa_ms * 1e-3) / 1e9, 2),
        "bit_differing_rows": diff_rows,
        "bit_checked_rows": checked_rows,
        "group_ms": {g: round(v, 4) for g, v in group_ms.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cells": cells,
        "input_sha256": {str(N): data[N]["sha"] for N in Ns},
    }
    print(json.dumps(out), flush=True)


ROTATE_BYTES = 512 * 2 ** 20     # inputs rotate through >= 2 x the 256 MB Infinity Cache, so reads are cold


def rotation(nbytes: float) -> int:
    """Copies of an input of nbytes that together exceed ROTATE_BYTES."""
    return max(1, -(-ROTATE_BYTES // int(nbytes)))


def _pct(sorted_vals, q):
    return sorted_vals[min(len(sorted_vals) - 1, int(round(q * (len(sorted_vals) - 1))))]


EAGER = False    # --eager: cells call their kernels directly instead of replaying graphs (counter runs)


def _time_graph(torch, fn, reps=20, samples=200, warm=10, keep=True):
    """Per-call time of fn replayed from a captured graph (reps calls per replay).

    At least `warm` warm-up replays, and about 30 ms of them so clocks have settled; then `samples`
    replays, each bracketed by its own pair of events.  Returns the median and p95 per-call time in us,
    the sample count and (keep=True) every per-call sample in ns."""
    if EAGER:
        return _time_eager(torch, fn, reps, samples, keep)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    once = time.perf_counter() - t0
    for _ in range(max(warm, min(200, int(0.03 / max(once, 1e-6)) + 1))):
        g.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
    for a, b in evs:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    ns = [a.elapsed_time(b) * 1e6 / reps for a, b in evs]
    srt = sorted(ns)
    out = {"us": round(_pct(srt, 0.5) / 1e3, 3), "p95_us": round(_pct(srt, 0.95) / 1e3, 3), "n": samples}
    if keep:
        out["samples_ns"] = [int(round(v)) for v in ns]
    del g
    return out


def _time_eager(torch, fn, reps, samples, keep):
    """As _time_graph with direct calls (one warm-up round), for counter collection runs."""
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
    for a, b in evs:
        a.record()
        for _ in range(reps):
            fn()
        b.record()
    torch.cuda.synchronize()
    ns = sorted(a.elapsed_time(b) * 1e6 / reps for a, b in evs)
    out = {"us": round(_pct(ns, 0.5) / 1e3, 3), "p95_us": round(_pct(ns, 0.95) / 1e3, 3), "n": samples}
    if keep:
        out["samples_ns"] = [int(round(v)) for v in ns]
    return out


class Ctx:
    """What the cells share: modules, device, sample count, the measured ceilings and the weights."""

    def __init__(self, torch, bi, lib, dev, synthetic, samples, data=None):
        self.torch, self.bi, self.lib, self.dev, self.synthetic = torch, bi, lib, dev, synthetic
        self.samples = samples
        self.data = data or {}
        self.ceil = None

    def weights(self, N):
        """The bf16 linear workload's x (256, 4096), bias and a rotation set of W (N, 4096) copies."""
        if N not in self.data:
            d = self.synthetic.cfg2_inputs(N, M_max=256)
            w = d["w"].to(self.dev)
            ws = [w] + [w.clone() for _ in range(rotation(w.numel() * 2) - 1)]
            self.data[N] = dict(x=d["x"].to(self.dev), w=ws, wt=[c.t() for c in ws], b=d["b"].to(self.dev),
                                sha=self.synthetic.sha256(d["w"]))
        return self.data[N]

    def frac(self, value, kind):
        """Fraction of the measured ceiling ("hbm": GB/s, "mfma": TFLOP/s), or None before it is measured."""
        if not self.ceil:
            return None
        top = self.ceil["hbm_stream_read"]["GBps"] if kind == "hbm" else self.ceil["mfma_bf16"]["TFLOPs"]
        return round(value / top, 4)


def _cell(ctx, t, **fields):
    """A cell's record: its fields, then the timing statistics (raw samples last)."""
    rec = dict(fields)
    rec.update({k: v for k, v in t.items() if k != "samples_ns"})
    if "samples_ns" in t:
        rec["samples_ns"] = t["samples_ns"]
    return rec


def cell_ceilings(ctx):
    """What this GPU measurably sustains: a streaming read of 1 GiB (every byte once; best of 1, 2 and 4
    workgroups of 256 threads per CU), the same read of 32 MiB / 112 MiB (the decode weights of N = 4096 /
    14336 at K = 4096) as single launches, once from one buffer read again and again (it stays in the
    last-level cache: "hot") and once rotating through copies of at least 512 MiB as the decode cells do
    ("cold"), and an MFMA-only loop (8 independent bf16 16x16x32 chains per wavefront, 1 and 2 workgroups
    of 4 wavefronts per CU)."""
    torch, lib = ctx.torch, ctx.lib
    sink = torch.zeros(256 * 8 * 256, dtype=torch.int32, device=ctx.dev)

    def stream():                 # the stream a graph capture records (read at each call)
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {}
    best = None
    for nb, cold in ((2 ** 30, False), (32 * 2 ** 20, False), (112 * 2 ** 20, False), (32 * 2 ** 20, True),
                     (112 * 2 ** 20, True)):
        srcs = [torch.empty(nb // 4, dtype=torch.int32, device=ctx.dev).random_(0, 2 ** 30)
                for _ in range(rotation(nb) if cold else 1)]
        for wpc in ((1, 2, 4) if nb == 2 ** 30 else (4,)):
            it = iter(range(10 ** 9))

            def fn(wpc=wpc):
                src = srcs[next(it) % len(srcs)]
                _chk(lib.bi_measure_stream_read(ctypes.c_void_p(src.data_ptr()), nb, ctypes.c_void_p(sink.data_ptr()),
                                                256 * wpc, stream()))
            reps = 4 if nb == 2 ** 30 else (2 * len(srcs) if cold else 20)
            t = _time_graph(torch, fn, reps=reps, samples=min(ctx.samples, 100), keep=False)
            gbps = nb / (t["us"] * 1e-6) / 1e9
            rec = {"bytes": nb, "workgroups_per_cu": wpc, "us": t["us"], "p95_us": t["p95_us"], "GBps": round(gbps, 1),
                   "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4)}
            if cold:
                rec["rotated_copies"] = len(srcs)
            if nb == 2 ** 30:
                if best is None or gbps > best["GBps"]:
                    best = rec
            else:
                out[f"stream_read_{'cold' if cold else 'hot'}_{nb >> 20}MiB"] = rec
        del srcs
    out["hbm_stream_read"] = best
    mbest = None
    for wpc in (1, 2):
        flops = [0.0]

        def fn(wpc=wpc):
            flops[0] = lib.bi_measure_mfma(ctypes.c_void_p(sink.data_ptr()), 256 * wpc, 4096, stream())
            if flops[0] < 0:
                raise RuntimeError("bi_measure_mfma refused its arguments")
        t = _time_graph(torch, fn, reps=4, samples=min(ctx.samples, 100), keep=False)
        tf = flops[0] / (t["us"] * 1e-6) / 1e12
        rec = {"workgroups_per_cu": wpc, "us": t["us"], "TFLOPs": round(tf, 1), "frac_mfma": round(tf / BF16_PEAK_TFLOPS, 4)}
        if mbest is None or tf > mbest["TFLOPs"]:
            mbest = rec
    out["mfma_bf16"] = mbest
    ctx.ceil = out
    return out


def _chk(rc):
    if rc != 0:
        raise RuntimeError(f"bi_measure_stream_read returned {rc}")


def cell_decode_gemm(ctx):
    """bi_linear at M in {1, 2, 4, 8} x N in {4096, 14336, 32000}, K = 4096, bf16, weights cold."""
    torch, bi = ctx.torch, ctx.bi
    K = 4096
    logits = ctx.synthetic.cfg5_inputs(torch.bfloat16, M_max=8)
    wl = logits["w"].to(ctx.dev)
    wls = [wl] + [wl.clone() for _ in range(rotation(wl.numel() * 2) - 1)]
    xl = logits["h"].to(ctx.dev)
    res = []
    for N in (4096, 14336, 32000):
        for M in (1, 2, 4, 8):
            if N == 32000:
                ws, x = wls, xl
            else:
                ws, x = ctx.weights(N)["w"], ctx.weights(N)["x"]
            it = iter(range(10 ** 9))
            fn = (lambda: bi.bi_linear(x[:M], ws[next(it) % len(ws)]))
            t = _time_graph(torch, fn, reps=len(ws) * 2, samples=ctx.samples)
            nbytes = 2.0 * (M * K + N * K + M * N)
            gbps = nbytes / (t["us"] * 1e-6) / 1e9
            same = (ctx.ceil or {}).get(f"stream_read_cold_{(N * K * 2) >> 20}MiB")
            res.append(_cell(ctx, t, M=M, N=N, GBps=round(gbps, 1), frac_hbm=round(gbps / HBM_PEAK_GBPS, 4),
                             frac_ceiling=ctx.frac(gbps, "hbm"),
                             frac_cold_read_same_bytes=round(gbps / same["GBps"], 4) if same else None,
                             rotated_copies=len(ws),
                             kernel=ctx.lib.bi_gemm_kernel_name(M, N, K, bi.BI_BF16, 0).decode()))
    del wls, wl
    return res


def cell_large_m_gemm(ctx):
    """bi_linear at M in {512, 1024, 4096} x N in {4096, 14336}, K = 4096, bf16 (added points above M = 256)."""
    torch, bi = ctx.torch, ctx.bi
    K = 4096
    res = []
    for N in (4096, 14336):
        w = ctx.weights(N)["w"][0]
        for M in (512, 1024, 4096):
            x = ctx.synthetic.randn((M, K), 0x5EED77, 1.0, torch.bfloat16).to(ctx.dev)
            t = _time_graph(torch, lambda: bi.bi_linear(x, w), reps=5, samples=ctx.samples)
            tf = 2.0 * M * N * K / (t["us"] * 1e-6) / 1e12
            res.append(_cell(ctx, t, M=M, N=N, TFLOPs=round(tf, 1), frac_mfma=round(tf / BF16_PEAK_TFLOPS, 4),
                             frac_ceiling=ctx.frac(tf, "mfma"),
                             kernel=ctx.lib.bi_gemm_kernel_name(M, N, K, bi.BI_BF16, 0).decode()))
    return res


def _decode_inputs(torch, dev, B, S, D, seed):
    """Seeded timing-only decode attention inputs, drawn on the GPU generator (multi-GB at the largest
    cells), K / V in enough copies to exceed the rotation size."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    q = torch.randn((B, 32, 1, D), generator=gen, device=dev).to(torch.bfloat16)
    k = torch.randn((B, 8, S, D), generator=gen, device=dev).to(torch.bfloat16)
    v = torch.randn((B, 8, S, D), generator=gen, device=dev).to(torch.bfloat16)
    n = rotation(2.0 * k.numel() * 2)
    kv = [(k, v)] + [(k.clone(), v.clone()) for _ in range(n - 1)]
    return q, kv, gen


def cell_decode_attention(ctx):
    """bi_sdpa decode (q_len 1, causal) on the pages' sweep shape: Hq 32, Hkv 8, D 128, bf16,
    B in {8, 32} x S in {2048, 8192, 32768}; K / V cold."""
    torch, bi, lib = ctx.torch, ctx.bi, ctx.lib
    res = []
    for B, S in ((8, 2048), (8, 8192), (8, 32768), (32, 2048), (32, 8192), (32, 32768)):
        q, kv, _ = _decode_inputs(torch, ctx.dev, B, S, 128, 0x5EED90 + B * 100000 + S)
        ws = torch.empty(max(1, bi.sdpa_workspace_bytes(B, 32, 8, 1, S, 128, torch.bfloat16)), dtype=torch.uint8,
                         device=ctx.dev)
        it = iter(range(10 ** 9))

        def fn():
            k, v = kv[next(it) % len(kv)]
            return bi.bi_sdpa(q, k, v, causal=True, workspace=ws)
        t = _time_graph(torch, fn, reps=max(4, 2 * len(kv)), samples=ctx.samples)
        nbytes = 2.0 * (B * 8 * S * 128 * 2 + 2 * B * 32 * 128)
        gbps = nbytes / (t["us"] * 1e-6) / 1e9
        res.append(_cell(ctx, t, B=B, S=S, GBps=round(gbps, 1), frac_hbm=round(gbps / HBM_PEAK_GBPS, 4),
                         frac_ceiling=ctx.frac(gbps, "hbm"), rotated_copies=len(kv),
                         kernel=lib.bi_sdpa_kernel_name(B, 32, 8, 1, S, 128, bi.BI_BF16).decode()))
        del q, kv, ws
    return res


def cell_attention_forms(ctx):
    """Sinks, a boolean (uint8) and an additive (bf16) padding mask over (B, 1, 1, S) on the decode shape,
    each as a ratio to the plain causal call; head dims 64 and 256 in decode and 2048-token prefill."""
    torch, bi, lib = ctx.torch, ctx.bi, ctx.lib
    ns = min(ctx.samples, 50)
    res = []
    for B, S in ((8, 8192), (32, 8192)):
        q, kv, gen = _decode_inputs(torch, ctx.dev, B, S, 128, 0x5EED91 + B * 100000 + S)
        ws = torch.empty(lib.bi_sdpa_workspace_bytes(B, 32, 8, 1, S, 128, bi.BI_BF16), dtype=torch.uint8, device=ctx.dev)
        sinks = torch.randn((32,), generator=gen, device=ctx.dev)
        keep = torch.rand((B, 1, 1, S), generator=gen, device=ctx.dev) > 0.1
        m8 = keep.to(torch.uint8)
        madd = torch.where(keep, torch.randn((B, 1, 1, S), generator=gen, device=ctx.dev),
                           torch.full((), float("-inf"), device=ctx.dev)).to(torch.bfloat16)
        it = iter(range(10 ** 9))

        def kvn():
            return kv[next(it) % len(kv)]
        forms = (("causal", lambda: bi.bi_sdpa(q, *kvn(), causal=True, workspace=ws)),
                 ("causal+sinks", lambda: bi.bi_sdpa(q, *kvn(), causal=True, workspace=ws, sinks=sinks)),
                 ("bool mask", lambda: bi.bi_sdpa(q, *kvn(), mask=m8, workspace=ws)),
                 ("additive mask", lambda: bi.bi_sdpa(q, *kvn(), mask=madd, workspace=ws)))
        base = None
        for name, fn in forms:
            t = _time_graph(torch, fn, reps=max(4, 2 * len(kv)), samples=ns, keep=False)
            base = base or t["us"]
            gbps = 2.0 * (B * 8 * S * 128 * 2) / (t["us"] * 1e-6) / 1e9
            res.append(_cell(ctx, t, B=B, S=S, D=128, form=name, GBps=round(gbps, 1),
                             frac_hbm=round(gbps / HBM_PEAK_GBPS, 4), over_causal=round(t["us"] / base, 3)))
        del q, kv, ws
    for D in (64, 256):
        B, S = 8, 8192
        q, kv, gen = _decode_inputs(torch, ctx.dev, B, S, D, 0x5EED92 + D)
        ws = torch.empty(lib.bi_sdpa_workspace_bytes(B, 32, 8, 1, S, D, bi.BI_BF16), dtype=torch.uint8, device=ctx.dev)
        it = iter(range(10 ** 9))

        def fn():
            k, v = kv[next(it) % len(kv)]
            return bi.bi_sdpa(q, k, v, causal=True, workspace=ws)
        t = _time_graph(torch, fn, reps=max(4, 2 * len(kv)), samples=ns, keep=False)
        gbps = 2.0 * (B * 8 * S * D * 2) / (t["us"] * 1e-6) / 1e9
        res.append(_cell(ctx, t, B=B, S=S, D=D, form="causal decode", GBps=round(gbps, 1),
                         frac_hbm=round(gbps / HBM_PEAK_GBPS, 4),
                         kernel=lib.bi_sdpa_kernel_name(B, 32, 8, 1, S, D, bi.BI_BF16).decode()))
        qp = torch.randn((1, 32, 2048, D), generator=gen, device=ctx.dev).to(torch.bfloat16)
        kp = torch.randn((1, 8, 2048, D), generator=gen, device=ctx.dev).to(torch.bfloat16)
        wsp = torch.empty(max(1, lib.bi_sdpa_workspace_bytes(1, 32, 8, 2048, 2048, D, bi.BI_BF16)), dtype=torch.uint8,
                          device=ctx.dev)
        t = _time_graph(torch, lambda: bi.bi_sdpa(qp, kp, kp, causal=True, workspace=wsp), reps=2, samples=ns,
                        keep=False)
        tf = 4.0 * 32 * D * (2048 * 2049 / 2) / (t["us"] * 1e-6) / 1e12
        res.append(_cell(ctx, t, B=1, Lq=2048, S=2048, D=D, form="causal prefill", TFLOPs=round(tf, 1),
                         frac_mfma=round(tf / BF16_PEAK_TFLOPS, 4),
                         kernel=lib.bi_sdpa_kernel_name(1, 32, 8, 2048, 2048, D, bi.BI_BF16).decode()))
        del q, kv, ws, qp, kp, wsp
    return res


def cell_prefill_attention(ctx):
    """Long causal prefill (query chunk = whole cache), Hq 32, Hkv 8, D 128, bf16, at 4096 and 8192
    tokens; flops of the causally visible pairs only."""
    torch, bi = ctx.torch, ctx.bi
    res = []
    for S in (4096, 8192):
        gen = torch.Generator(device=ctx.dev)
        gen.manual_seed(0x5EED95 + S)
        q = torch.randn((1, 32, S, 128), generator=gen, device=ctx.dev).to(torch.bfloat16)
        k = torch.randn((1, 8, S, 128), generator=gen, device=ctx.dev).to(torch.bfloat16)
        v = torch.randn((1, 8, S, 128), generator=gen, device=ctx.dev).to(torch.bfloat16)
        t = _time_graph(torch, lambda: bi.bi_sdpa(q, k, v, causal=True), reps=2, samples=ctx.samples)
        flops = 4.0 * 32 * 128 * (S * (S + 1) / 2)
        tf = flops / (t["us"] * 1e-6) / 1e12
        res.append(_cell(ctx, t, B=1, Lq=S, S=S, TFLOPs=round(tf, 1), frac_mfma=round(tf / BF16_PEAK_TFLOPS, 4),
                         frac_ceiling=ctx.frac(tf, "mfma"),
                         kernel=ctx.lib.bi_sdpa_kernel_name(1, 32, 8, S, S, 128, bi.BI_BF16).decode()))
        del q, k, v
    return res


def cell_quantized_gemm(ctx):
    """bi_quantized_linear, 4-bit, groups of 64, K = 4096, M in {1, 4, 16, 64, 256} x N in {4096, 14336};
    packed weights cold; bytes = packed words + scales + biases + x + y; rows checked against M = 256."""
    torch, bi = ctx.torch, ctx.bi
    K = 4096
    res = []
    differing = 0
    for N in (4096, 14336):
        d = ctx.weights(N)
        wq, sc, sb = bi.quantize(d["w"][0], 4, 64)
        qbytes = wq.numel() * 4 + sc.numel() * 2 * 2
        qs = [(wq, sc, sb)] + [(wq.clone(), sc.clone(), sb.clone()) for _ in range(rotation(qbytes) - 1)]
        xq = d["x"]
        full = bi.bi_quantized_linear(xq, wq, sc, sb, 4, 64)
        for M in (1, 4, 16, 64, 256):
            it = iter(range(10 ** 9))
            t = _time_graph(torch, lambda: bi.bi_quantized_linear(xq[:M], *qs[next(it) % len(qs)], 4, 64),
                            reps=len(qs), samples=min(ctx.samples, 50), keep=False)
            nbytes = qbytes + 2.0 * (M * K + M * N)
            gbps = nbytes / (t["us"] * 1e-6) / 1e9
            tf = 2.0 * M * N * K / (t["us"] * 1e-6) / 1e12
            part = bi.bi_quantized_linear(xq[:M], wq, sc, sb, 4, 64)
            differing += int((part.view(torch.int16) != full[:M].view(torch.int16)).any(dim=1).sum().item())
            res.append(_cell(ctx, t, M=M, N=N, bits=4, group_size=64, GBps=round(gbps, 1),
                             frac_hbm=round(gbps / HBM_PEAK_GBPS, 4), TFLOPs=round(tf, 1)))
        del qs
    return {"cells": res, "rows_differing_from_M256": differing}


def cell_comparator(ctx):
    """The batch-variant comparators beside the invariant path (the cost of invariance and the negative
    control).  GEMM: the bf16 linear workload (K = 4096, N in {4096, 14336}, every M of the sweep), where
    bi_variant_linear runs the same kernel as bi_linear for each M with M-keyed split-K; rows of each M
    that differ from the same rows at M = 256 (nonzero for the variant, 0 for bi_linear).  Attention:
    bi_variant_sdpa (split length from G * q_len and S) against bi_sdpa on the q_len sweep at a 1024-key
    cache and on decode at B = 8, S = 8192; elements of single-token decodes (Hq 16, Hkv 8) that change
    when the cache grows from 4000 to 4200 keys with the new keys masked."""
    torch, bi, lib = ctx.torch, ctx.bi, ctx.lib
    ns = min(ctx.samples, 50)
    inv_us = var_us = 0.0
    diff_var = diff_inv = 0
    per = []
    for N in (4096, 14336):
        dN = ctx.weights(N)
        ws = dN["w"]
        full_var = bi.bi_variant_linear(dN["x"], ws[0], dN["b"])
        full_inv = bi.bi_linear(dN["x"], ws[0], dN["b"])
        for M in ctx.synthetic.CFG2["M_values"]:
            x = dN["x"][:M]
            it1, it2 = iter(range(10 ** 9)), iter(range(10 ** 9))
            ti = _time_graph(torch, lambda: bi.bi_linear(x, ws[next(it1) % len(ws)], dN["b"]),
                             reps=len(ws), samples=ns, keep=False)
            tv = _time_graph(torch, lambda: bi.bi_variant_linear(x, ws[next(it2) % len(ws)], dN["b"]),
                             reps=len(ws), samples=ns, keep=False)
            inv_us += ti["us"]
            var_us += tv["us"]
            v = bi.bi_variant_linear(x, ws[0], dN["b"])
            y = bi.bi_linear(x, ws[0], dN["b"])
            dv = int((v.view(torch.int16) != full_var[:M].view(torch.int16)).any(dim=1).sum().item())
            di = int((y.view(torch.int16) != full_inv[:M].view(torch.int16)).any(dim=1).sum().item())
            diff_var += dv
            diff_inv += di
            per.append({"M": M, "N": N, "invariant_us": ti["us"], "variant_us": tv["us"],
                        "splits": int(lib.bi_variant_splits(M)),
                        "kernel": lib.bi_gemm_kernel_name(M, N, 4096, bi.BI_BF16, 0).decode(),
                        "variant_rows_differing": dv})
    gemm = {"invariant_ms": round(inv_us / 1e3, 4), "variant_ms": round(var_us / 1e3, 4),
            "invariant_over_variant_time": round(inv_us / var_us, 4),
            "variant_rows_differing_from_M256": diff_var, "invariant_rows_differing_from_M256": diff_inv,
            "per_shape": per}
    # attention: cost on the q_len sweep and on a decode batch
    c3 = ctx.synthetic.cfg3_inputs(B=1, S=1024)
    q3, k3, v3 = (c3[n].to(ctx.dev) for n in ("q", "k", "v"))
    att = {"qlen_sweep": []}
    tot_i = tot_v = 0.0
    for L in ctx.synthetic.CFG3["Lq_values"]:
        qq = q3[:, :, 1024 - L:]
        ti = _time_graph(torch, lambda: bi.bi_sdpa(qq, k3, v3, causal=True), reps=10, samples=ns, keep=False)
        tv = _time_graph(torch, lambda: bi.bi_variant_sdpa(qq, k3, v3, causal=True), reps=10, samples=ns, keep=False)
        tot_i += ti["us"]
        tot_v += tv["us"]
        att["qlen_sweep"].append({"Lq": L, "invariant_us": ti["us"], "variant_us": tv["us"]})
    att["qlen_sweep_invariant_over_variant_time"] = round(tot_i / tot_v, 4)
    q, kv, _ = _decode_inputs(torch, ctx.dev, 8, 8192, 128, 0x5EED93)
    wsd = torch.empty(max(1, bi.sdpa_workspace_bytes(8, 32, 8, 1, 8192, 128, torch.bfloat16)), dtype=torch.uint8,
                      device=ctx.dev)
    it1, it2 = iter(range(10 ** 9)), iter(range(10 ** 9))
    ti = _time_graph(torch, lambda: bi.bi_sdpa(q, *kv[next(it1) % len(kv)], causal=True, workspace=wsd),
                     reps=2 * len(kv), samples=ns, keep=False)
    tv = _time_graph(torch, lambda: bi.bi_variant_sdpa(q, *kv[next(it2) % len(kv)], causal=True),
                     reps=2 * len(kv), samples=ns, keep=False)
    att["decode_B8_S8192"] = {"invariant_us": ti["us"], "variant_us": tv["us"],
                              "invariant_over_variant_time": round(ti["us"] / tv["us"], 4)}
    del q, kv, wsd
    # negative control: context growth with the new keys masked (config 4 shapes)
    c4 = ctx.synthetic.cfg4_inputs(torch.bfloat16)
    q4, k4, v4 = (c4[n].to(ctx.dev) for n in ("q", "k", "v"))
    dv = di = 0
    for n0 in (4000, 4096):
        base_v = bi.bi_variant_sdpa(q4, k4[:, :, :n0], v4[:, :, :n0])
        base_i = bi.bi_sdpa(q4, k4[:, :, :n0], v4[:, :, :n0])
        for n in range(n0 + 1, 4201, 25):
            mask = torch.zeros(1, 1, 1, n, dtype=torch.bool, device=ctx.dev)
            mask[..., :n0] = True
            dv += int((bi.bi_variant_sdpa(q4, k4[:, :, :n], v4[:, :, :n], mask=mask).view(torch.int16)
                       != base_v.view(torch.int16)).sum())
            di += int((bi.bi_sdpa(q4, k4[:, :, :n], v4[:, :, :n], mask=mask).view(torch.int16)
                       != base_i.view(torch.int16)).sum())
    att["context_growth_elements_differing"] = {"variant": dv, "invariant": di}
    return {"gemm": gemm, "attention": att}


def cell_e2e(ctx):
    """The random-weight decoder end to end: decode steps and a 256-token prefill, each under
    batch_invariant_mode, under the batch-variant comparator kernels and with stock PyTorch."""
    return e2e_run(ctx.torch, ctx.bi, ctx.dev, ctx.synthetic)


CELLS = {
    "ceilings": cell_ceilings,
    "decode_gemm": cell_decode_gemm,
    "large_m_gemm": cell_large_m_gemm,
    "decode_attention": cell_decode_attention,
    "prefill_attention": cell_prefill_attention,
    "attention_forms": cell_attention_forms,
    "quantized_gemm": cell_quantized_gemm,
    "comparator": cell_comparator,
    "e2e": cell_e2e,
}


def measure_cells(ctx, names=None):
    cells = {}
    for name in names or list(CELLS):
        t0 = time.time()
        cells[name] = CELLS[name](ctx)
        log(f"cell {name} measured in {time.time() - t0:.1f}s")
    return cells


@contextlib.contextmanager
def _variant_mode(torch, bi):
    """F.linear and F.scaled_dot_product_attention on the batch-variant comparator kernels
    (bi_variant_linear with its M-keyed split-K, bi_variant_sdpa with its shape-keyed splits); every
    other op runs stock.  The end-to-end analogue of the kernels' comparator, installed the way
    batch_invariant_mode installs its routes (the two functions replaced while the block runs)."""
    import torch.nn.functional as F
    lin, att = F.linear, F.scaled_dot_product_attention

    def linear(x, w, bias=None):
        return bi.bi_variant_linear(x, w, bias)

    def sdpa(q, k, v, attn_mask=None, dropout_p=0.0, is_causal=False, scale=None, enable_gqa=False):
        assert attn_mask is None and dropout_p == 0.0 and (not is_causal or q.shape[2] == k.shape[2])
        return bi.bi_variant_sdpa(q, k, v, causal=is_causal, scale=scale)

    F.linear, F.scaled_dot_product_attention = linear, sdpa
    try:
        yield
    finally:
        F.linear, F.scaled_dot_product_attention = lin, att


def e2e_run(torch, bi, dev, synthetic):
    """A random-weight 4-layer decoder (hidden 2048, 16 / 4 heads of 128, SwiGLU 5632, vocab 32000):
    batch 8 with 128-token prompts and 32 greedy decode steps (time per decode step), and a prefill of
    8 x 256 tokens (time per prefill), each under batch_invariant_mode, under the batch-variant comparator
    kernels and with stock PyTorch; how many of the 32000 last-position logits of one sequence move
    between batch 1 and batch 8 in each."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import tiny_transformer as tt
    cfg = tt.TinyConfig(layers=4)
    W = tt.make_weights(cfg, 0x5EEDE5, dev)
    prompts = synthetic.randint((8, 128), 0x5EEDE6, 0, cfg.vocab, torch.int64).to(dev)
    long_prompts = synthetic.randint((8, 256), 0x5EEDE7, 0, cfg.vocab, torch.int64).to(dev)
    steps = 32
    modes = {"invariant": lambda: bi.batch_invariant_mode(), "variant": lambda: _variant_mode(torch, bi),
             "stock": lambda: _nullcontext()}

    def decode(name, p):
        with torch.no_grad(), modes[name]():
            logits, cache = tt.forward(cfg, W, p, None, 0)
            tok = logits[:, -1].float().argmax(-1, keepdim=True)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            pos = p.shape[1]
            for _ in range(steps):
                logits, cache = tt.forward(cfg, W, tok, cache, pos)
                tok = logits[:, -1].float().argmax(-1, keepdim=True)
                pos += 1
            b.record()
            b.synchronize()
            return a.elapsed_time(b) / steps, logits[:, -1]

    def prefill(name, p, reps=5):
        with torch.no_grad(), modes[name]():
            tt.forward(cfg, W, p, None, 0)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                logits, _ = tt.forward(cfg, W, p, None, 0)
            b.record()
            b.synchronize()
            return a.elapsed_time(b) / reps, logits[:, -1]

    for name in modes:                      # warm-up every path
        decode(name, prompts)
    out = {"model": "4 layers, hidden 2048, 16/4 heads x 128, SwiGLU 5632, vocab 32000, bf16, random weights",
           "decode": {"batch": 8, "prompt": 128, "decode_steps": steps},
           "prefill": {"batch": 8, "tokens": 256}}
    for name in modes:
        ms, last8 = decode(name, prompts)
        _, last1 = decode(name, prompts[:1])
        n = int((last1[0].view(torch.int16) != last8[0].view(torch.int16)).sum())
        out["decode"][name] = {"ms_per_decode_step": round(ms, 3), "tokens_per_s": round(8 * 1e3 / ms, 1),
                               "logits_differing_batch1_vs_batch8": n}
        ms, l8 = prefill(name, long_prompts)
        _, l1 = prefill(name, long_prompts[:1], reps=1)
        n = int((l1[0].view(torch.int16) != l8[0].view(torch.int16)).sum())
        out["prefill"][name] = {"ms_per_prefill": round(ms, 3), "tokens_per_s": round(8 * 256 * 1e3 / ms, 1),
                                "logits_differing_batch1_vs_batch8": n}
    for ph, key in (("decode", "ms_per_decode_step"), ("prefill", "ms_per_prefill")):
        inv = out[ph]["invariant"][key]
        out[ph]["invariant_over_stock_time"] = round(inv / out[ph]["stock"][key], 4)
        out[ph]["invariant_over_variant_time"] = round(inv / out[ph]["variant"][key], 4)
    return out


class _nullcontext:
    def __enter__(self):
        return None

    def __exit__(self, *a):
        return False


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(torch, synthetic, args):
    """The float64 CPU oracle, as it stands, on the host's OpenMP threads: the linear workload (whole passes
    of the M = 256 batch at both N) for about --cpu-seconds, then the attention q_len sweep (q_len 1 ... 64
    against the 1024-key cache, Hq 32, Hkv 8, D 128) for about as long."""
    import oracle
    if args.cpu_threads > 0:
        oracle.set_threads(args.cpu_threads)
    threads = oracle.threads()
    Ms = synthetic.CFG2["M_values"]
    inputs = [synthetic.cfg2_inputs(N, M_max=max(Ms)) for N in synthetic.CFG2["N_values"]]
    flops = 0.0
    passes = 0
    t0 = time.perf_counter()
    while passes == 0 or time.perf_counter() - t0 < args.cpu_seconds:
        for d in inputs:
            # the largest batch of the sweep: its rows contain every smaller batch's rows
            oracle.linear(d["x"], d["w"], d["b"])
            flops += 2.0 * d["x"].shape[0] * d["w"].shape[0] * d["w"].shape[1]
        passes += 1
    t = time.perf_counter() - t0
    log(f"cpu oracle linear: {flops / 1e9:.1f} GFLOP in {t:.1f}s on {threads} threads ({passes} passes)")
    c3 = synthetic.cfg3_inputs(B=1, S=synthetic.CFG3["S"])
    S3 = synthetic.CFG3["S"]
    abytes = 0.0
    apasses = 0
    t1 = time.perf_counter()
    while apasses == 0 or time.perf_counter() - t1 < args.cpu_seconds:
        for L in synthetic.CFG3["Lq_values"]:
            oracle.sdpa(c3["q"][:, :, S3 - L:], c3["k"], c3["v"], causal=True)
            abytes += 2.0 * (2 * 8 * S3 * 128 + 2 * 32 * L * 128)
        apasses += 1
    ta = time.perf_counter() - t1
    log(f"cpu oracle attention: {abytes / 1e6:.1f} MB in {ta:.1f}s ({apasses} passes)")
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"{passes} passes of the float64 oracle linear on the M=256 batch (x 256x4096, bias) "
                      "for N=4096 and N=14336, i.e. every row of the GEMM sweep once per pass",
            "seconds": round(t, 2),
            "attention": {"value": round(abytes / ta / 1e9, 6), "unit": "GB/s",
                          "sample": f"{apasses} passes of the float64 oracle attention over the bf16 causal GQA "
                                    "q_len sweep {1,2,4,8,9,16,64} against the 1024-key cache (Hq 32, Hkv 8, D 128), "
                                    "bytes counted as on the GPU (K and V once per KV head, q and o)",
                          "seconds": round(ta, 2)}}


# ---------------------------------------------------------------- profiling helpers
def _calibration_copy(torch):
    """An elementwise copy that reads and writes CALIB_BYTES each, dispatched before any library kernel, so
    counter summaries can scale FETCH_SIZE / WRITE_SIZE to bytes."""
    src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def pmc_pass(torch, st, order_path):
    """One eager pass for counter collection: a calibration copy of known size, then every launch
    of the step once, in order; writes which kernel group each of our dispatches belongs to."""
    src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 2.0, out=dst)              # reads and writes CALIB_BYTES each
    torch.cuda.synchronize()
    order = []
    for rec in st["launches"]:
        rec[2]()
        order.append({"group": rec[0], "kind": rec[1], "dispatches": 2 if "combine" in rec[0] else 1,
                      "algorithmic_bytes": rec[4]})
    torch.cuda.synchronize()
    with open(order_path, "w") as f:
        json.dump({"calibration_bytes": CALIB_BYTES, "launches": order}, f)
    log(f"pmc pass: {len(order)} launches written to {order_path}")


def _counter_rows(d, counter):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                k = int(r["Dispatch_Id"])
                e = per.setdefault(k, [r["Kernel_Name"], 0.0])
                e[1] += float(r["Counter_Value"])
    return [(k, v[0], v[1]) for k, v in sorted(per.items())]


def _attribute(rows, order, calib_bytes):
    """Calibration factor and per-group counter totals from one counter's dispatch rows."""
    ours = [(k, n, v) for k, n, v in rows if "bi::" in n]
    first = ours[0][0] if ours else None
    calib = [v for k, n, v in rows if "bi::" not in n and (first is None or k < first)]
    big = max(calib) if calib else 0.0
    if big * 1024 < 0.5 * calib_bytes:
        raise SystemExit("calibration copy not found among the dispatches")
    factor = calib_bytes / (big * 1024)       # counter reads KiB
    expect = sum(o["dispatches"] for o in order)
    if len(ours) != expect:
        raise SystemExit(f"{len(ours)} library dispatches in the counters, {expect} expected")
    tot = {}
    it = iter(ours)
    for o in order:
        for _ in range(o["dispatches"]):
            _, _, v = next(it)
            tot[o["group"]] = tot.get(o["group"], 0.0) + v
    return factor, big, tot


def summarize_pmc(args):
    with open(args.order) as f:
        od = json.load(f)
    order, cb = od["launches"], od["calibration_bytes"]
    fdir, wdir = args.summarize_pmc
    ff, fbig, ftot = _attribute(_counter_rows(fdir, "FETCH_SIZE"), order, cb)
    wf, wbig, wtot = _attribute(_counter_rows(wdir, "WRITE_SIZE"), order, cb)
    nl, alg, kind = {}, {}, {}
    for o in order:
        nl[o["group"]] = nl.get(o["group"], 0) + 1
        alg[o["group"]] = alg.get(o["group"], 0.0) + o["algorithmic_bytes"]
        kind[o["group"]] = o["kind"]
    lines = [f"# {args.title or 'HBM traffic per launch of every kernel group of one bench step'}", "",
             "Commands (run from the repository root on one MI355X):", "", "```"] + args.cmd + ["```", "",
             f"Calibration: one elementwise copy reading and writing {cb} bytes each; FETCH_SIZE read "
             f"{fbig:.0f} KiB for it (scale {ff:.4f}), WRITE_SIZE {wbig:.0f} KiB (scale {wf:.4f}).  "
             "Counter values below are scaled by these factors.", "",
             "| kernel group | launches | fetched MB / launch | written MB / launch | traffic MB / launch "
             "| algorithmic MB / launch | traffic / algorithmic |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    groups = {}
    for g in nl:
        fb = ftot[g] * 1024 * ff / nl[g]
        wb = wtot[g] * 1024 * wf / nl[g]
        a = alg[g] / nl[g]
        groups[g] = {"traffic_bytes": round(fb + wb), "fetch_bytes": round(fb), "write_bytes": round(wb),
                     "algorithmic_bytes": round(a), "family": kind[g]}
        lines.append(f"| `{g}` | {nl[g]} | {fb / 1e6:.2f} | {wb / 1e6:.2f} | {(fb + wb) / 1e6:.2f} | "
                     f"{a / 1e6:.2f} | {(fb + wb) / a:.3f} |")
    hashes = {fam: family_hash(fam) for fam in FAMILY_SOURCES}
    lines += ["", "Kernel sources hashed when the counters were taken (bench.py reports the traffic only "
                  "while these still match):", ""]
    lines += [f"- {fam}: `{h}`" for fam, h in hashes.items()]
    lines += ["", "<!-- traffic-json " + json.dumps({"hashes": hashes, "groups": groups}) + " -->", ""]
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def measured_traffic(group, family):
    """Scaled FETCH_SIZE + WRITE_SIZE bytes per launch of a kernel group, from the committed summary,
    or None when there is none or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_MD) as f:
            m = re.search(r"<!-- traffic-json (.*) -->", f.read())
        d = json.loads(m.group(1))
        g = d["groups"][group]
        if d["hashes"].get(g["family"]) != family_hash(g["family"]):
            return None
        return g["traffic_bytes"]
    except (OSError, AttributeError, KeyError, ValueError):
        return None


def summarize_counters(args):
    """Per-dispatch averages of the counters collected under one or more directories (a run per counter
    pass), for the kernels whose names contain one of --kernel, grouped by kernel and grid size; derived:
    instructions per wavefront and per MFMA instruction, busy fractions of the matrix cores, the vector ALUs
    and the LDS over the dispatch's duration at the 2.4 GHz nominal clock (1024 SIMDs, 256 CUs), and HBM
    bytes from FETCH_SIZE / WRITE_SIZE scaled by the calibration copy run first (--cell with --eager)."""
    rows = []
    for d in args.summarize_counters:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for fn in files:
            with open(fn) as f:
                rows += [dict(r, _dir=d) for r in csv.DictReader(f)]
    # calibration: per directory, the largest FETCH_SIZE / WRITE_SIZE of a non-library dispatch before the
    # first library dispatch (the CALIB_BYTES copy of --eager cell runs)
    scale = {}
    for d in args.summarize_counters:
        first = min((int(r["Dispatch_Id"]) for r in rows if r["_dir"] == d and "bi::" in r["Kernel_Name"]), default=None)
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            per = {}
            for r in rows:
                if r["_dir"] == d and r["Counter_Name"] == c and "bi::" not in r["Kernel_Name"] and \
                        (first is None or int(r["Dispatch_Id"]) < first):
                    per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
            if per and max(per.values()) * 1024 > 0.5 * CALIB_BYTES:
                scale[c] = CALIB_BYTES / (max(per.values()) * 1024)
    per = {}
    for r in rows:
        name = r["Kernel_Name"]
        if args.kernel and not any(k in name for k in args.kernel):
            continue
        key = (name, int(r["Grid_Size"]))
        disp = per.setdefault(key, {}).setdefault((r["_dir"], int(r["Dispatch_Id"])), {})
        disp[r["Counter_Name"]] = disp.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        disp["_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    lines = [f"# {args.title}", "", "Commands (run from the repository root on one MI355X):", "", "```"] + args.cmd + \
        ["```", "", "Counter values are per dispatch, averaged over the dispatches of each kernel and grid size (SQ "
         "counters summed over the whole GPU).  Busy fractions divide by the dispatch's duration under counter "
         "collection at the nominal 2.4 GHz clock and are estimates.", ""]
    if scale:
        lines += ["Calibration (a copy of %d bytes each way): " % CALIB_BYTES +
                  ", ".join(f"{c} scale {v:.3f}" for c, v in sorted(scale.items())), ""]
    for (name, grid), disp in sorted(per.items()):
        names = sorted({c for dd in disp.values() for c in dd if not c.startswith("_")})
        cnt = {c: [dd[c] for dd in disp.values() if c in dd] for c in names}
        avg = {c: sum(v) / len(v) for c, v in cnt.items()}
        ns = sorted(dd["_ns"] for dd in disp.values())[len(disp) // 2]
        short = name if len(name) < 100 else name[:97] + "..."
        lines += [f"## `{short}`, grid {grid}", "", f"{max(len(v) for v in cnt.values())} dispatches per counter pass; "
                  f"median duration under collection {ns / 1e3:.1f} us.", "", "| counter | per dispatch |", "|---|---:|"]
        lines += [f"| {c} | {avg[c]:.4g} |" for c in names]
        waves = avg.get("SQ_WAVES")
        mfma = avg.get("SQ_INSTS_MFMA")
        cyc = ns * 2.4
        derived = []
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_TRANS_F32"):
            if c in avg and waves:
                derived.append(f"| {c} per wavefront | {avg[c] / waves:.1f} |")
            if c in avg and mfma and c != "SQ_INSTS_MFMA":
                derived.append(f"| {c} per MFMA instruction | {avg[c] / mfma:.3f} |")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and cyc:
            derived.append(f"| matrix cores busy (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / cycles) | "
                           f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024 / cyc:.3f} |")
        if "SQ_ACTIVE_INST_VALU" in avg and cyc:
            derived.append(f"| vector ALU issue (4 x SQ_ACTIVE_INST_VALU / 1024 SIMDs / cycles) | "
                           f"{4 * avg['SQ_ACTIVE_INST_VALU'] / 1024 / cyc:.3f} |")
        if "SQ_LDS_IDX_ACTIVE" in avg and cyc:
            derived.append(f"| LDS busy (SQ_LDS_IDX_ACTIVE / 256 CUs / cycles) | {avg['SQ_LDS_IDX_ACTIVE'] / 256 / cyc:.3f} |")
        if "SQ_WAIT_ANY" in avg and "SQ_WAVE_CYCLES" in avg:
            derived.append(f"| wave time waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES) | {avg['SQ_WAIT_ANY'] / avg['SQ_WAVE_CYCLES']:.3f} |")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if c in avg and c in scale:
                derived.append(f"| HBM {c.split('_')[0].lower()} MB (scaled) | {avg[c] * 1024 * scale[c] / 1e6:.2f} |")
        if derived:
            lines += ["", "| derived | value |", "|---|---:|"] + derived
        lines.append("")
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def summarize_stats(args):
    """The rocprofv3 kernel statistics as a table, plus (from the kernel trace beside them) the duration of
    every library kernel by grid shape: the cells launch one kernel at several shapes."""
    with open(args.summarize_stats) as f:
        rows = list(csv.DictReader(f))
    lines = [f"# {args.title}", "", "Command (run from the repository root on one MI355X):", "", "```"] + \
        args.cmd + ["```", "",
                    "rocprofv3 kernel statistics (every dispatch of the run: warm-up, graph capture and the "
                    "timed steps):", "",
                    "| kernel | calls | avg us | min us | max us | % time |", "|---|---:|---:|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        if float(r["Percentage"]) < 0.3:
            continue
        name = r["Name"].replace("|", "/")
        if len(name) > 90:
            name = name[:87] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    trace = args.summarize_stats.replace("kernel_stats.csv", "kernel_trace.csv")
    if trace != args.summarize_stats and os.path.exists(trace):
        by = {}
        with open(trace) as f:
            for r in csv.DictReader(f):
                if "bi::" not in r["Kernel_Name"]:
                    continue
                key = (r["Kernel_Name"], int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]),
                       int(r["Workgroup_Size_X"]))
                by.setdefault(key, []).append((float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) / 1e3)
        lines += ["", "Library kernels by launch shape (threads in the grid, workgroup size):", "",
                  "| kernel | grid threads | workgroup | calls | median us | min us | p95 us |",
                  "|---|---:|---:|---:|---:|---:|---:|"]
        for (name, grid, wg), d in sorted(by.items(), key=lambda kv: (kv[0][0], kv[0][1])):
            d.sort()
            short = name.replace("|", "/")
            short = short if len(short) <= 90 else short[:87] + "..."
            lines.append(f"| `{short}` | {grid} | {wg} | {len(d)} | {d[len(d) // 2]:.2f} | {d[0]:.2f} | "
                         f"{d[min(len(d) - 1, int(round(0.95 * (len(d) - 1))))]:.2f} |")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))

if __name__ == "__main__":
    main()
