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
import csv
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
    copies = {4096: 8, 14336: 4}          # > 256 MB of weights per N and layout
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
        cells = measure_cells(bi, lib, torch, dev, synthetic, data, launches, groups, names, group_ms)

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


def _time_graph(torch, fn, reps=20, iters=10):
    """Median per-call ms of fn replayed from a captured graph (reps calls per replay)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    # warm-up replays for about 30 ms, so clocks have settled before timing
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    once = time.perf_counter() - t0
    for _ in range(min(200, int(0.03 / max(once, 1e-6)) + 1)):
        g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) / reps)
    ts.sort()
    return ts[len(ts) // 2]


def measure_cells(bi, lib, torch, dev, synthetic, data, launches, groups, names, group_ms):
    cells = {"decode_gemm": [], "large_m_gemm": [], "decode_attention": [], "prefill_attention": [],
             "comparator": {}, "e2e_decode": {}}
    K = 4096
    # decode GEMM: weights rotate through copies inside one graph, so reads are cold
    logits = synthetic.cfg5_inputs(torch.bfloat16, M_max=8)
    wl = logits["w"].to(dev)
    wls = [wl, wl.clone()]
    xl = logits["h"].to(dev)
    for N in (4096, 14336, 32000):
        for M in (1, 2, 4, 8):
            if N == 32000:
                ws, x = wls, xl
            else:
                ws, x = data[N]["w"], data[N]["x"]
            it = iter(range(10 ** 9))
            fn = (lambda: bi.bi_linear(x[:M], ws[next(it) % len(ws)]))
            ms = _time_graph(torch, fn, reps=len(ws) * 2)
            nbytes = 2.0 * (M * K + N * K + M * N)
            gbps = nbytes / (ms * 1e-3) / 1e9
            cells["decode_gemm"].append({"M": M, "N": N, "us": round(ms * 1e3, 2), "GBps": round(gbps, 1),
                                         "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4),
                                         "kernel": lib.bi_gemm_kernel_name(M, N, K, bi.BI_BF16, 0).decode()})
    del wls, wl
    # large-M GEMM (added points, above the configs' M = 256)
    for N in (4096, 14336):
        w = data[N]["w"][0]
        for M in (512, 1024, 4096):
            x = synthetic.randn((M, K), 0x5EED77, 1.0, torch.bfloat16).to(dev)
            ms = _time_graph(torch, lambda: bi.bi_linear(x, w), reps=5, iters=6)
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            cells["large_m_gemm"].append({"M": M, "N": N, "us": round(ms * 1e3, 1), "TFLOPs": round(tf, 1),
                                          "frac_mfma": round(tf / BF16_PEAK_TFLOPS, 4),
                                          "kernel": lib.bi_gemm_kernel_name(M, N, K, bi.BI_BF16, 0).decode()})
    # decode attention on the pages' sweep shape (Hq 32, Hkv 8, D 128, bf16, q_len 1)
    for B, S in ((8, 2048), (8, 8192), (32, 8192), (32, 32768)):
        # multi-GB timing-only inputs: seeded draws on the GPU generator
        gen = torch.Generator(device=dev)
        gen.manual_seed(0x5EED90 + B * 100000 + S)
        q = torch.randn((B, 32, 1, 128), generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn((B, 8, S, 128), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((B, 8, S, 128), generator=gen, device=dev).to(torch.bfloat16)
        ws = torch.empty(bi.sdpa_workspace_bytes(B, 32, 8, 1, S, 128, torch.bfloat16), dtype=torch.uint8, device=dev)
        ms = _time_graph(torch, lambda: bi.bi_sdpa(q, k, v, causal=True, workspace=ws), reps=4, iters=6)
        nbytes = 2.0 * (B * 8 * S * 128 * 2 + 2 * B * 32 * 128)
        gbps = nbytes / (ms * 1e-3) / 1e9
        cells["decode_attention"].append({"B": B, "S": S, "us": round(ms * 1e3, 1), "GBps": round(gbps, 1),
                                          "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4)})
        del q, k, v, ws
    # the other attention forms on the decode shape: sinks, a boolean (uint8) and an additive (bf16)
    # padding mask over (B, 1, 1, S), each as a ratio to the plain call; head dims 64 and 256
    cells["attention_forms"] = []
    for B, S in ((8, 8192), (32, 8192)):
        gen = torch.Generator(device=dev)
        gen.manual_seed(0x5EED91 + B * 100000 + S)
        q = torch.randn((B, 32, 1, 128), generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn((B, 8, S, 128), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((B, 8, S, 128), generator=gen, device=dev).to(torch.bfloat16)
        ws = torch.empty(lib.bi_sdpa_workspace_bytes(B, 32, 8, 1, S, 128, bi.BI_BF16), dtype=torch.uint8, device=dev)
        sinks = torch.randn((32,), generator=gen, device=dev)
        keep = torch.rand((B, 1, 1, S), generator=gen, device=dev) > 0.1
        m8 = keep.to(torch.uint8)
        madd = torch.where(keep, torch.randn((B, 1, 1, S), generator=gen, device=dev),
                           torch.full((), float("-inf"), device=dev)).to(torch.bfloat16)
        forms = (("causal", lambda: bi.bi_sdpa(q, k, v, causal=True, workspace=ws)),
                 ("causal+sinks", lambda: bi.bi_sdpa(q, k, v, causal=True, workspace=ws, sinks=sinks)),
                 ("bool mask", lambda: bi.bi_sdpa(q, k, v, mask=m8, workspace=ws)),
                 ("additive mask", lambda: bi.bi_sdpa(q, k, v, mask=madd, workspace=ws)))
        base = None
        for name, fn in forms:
            ms = _time_graph(torch, fn, reps=4, iters=6)
            base = base or ms
            gbps = 2.0 * (B * 8 * S * 128 * 2) / (ms * 1e-3) / 1e9
            cells["attention_forms"].append({"B": B, "S": S, "D": 128, "form": name, "us": round(ms * 1e3, 1),
                                             "GBps": round(gbps, 1), "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4),
                                             "over_causal": round(ms / base, 3)})
        del q, k, v, ws
    for D in (64, 256):
        B, S = 8, 8192
        gen = torch.Generator(device=dev)
        gen.manual_seed(0x5EED92 + D)
        q = torch.randn((B, 32, 1, D), generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn((B, 8, S, D), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((B, 8, S, D), generator=gen, device=dev).to(torch.bfloat16)
        ws = torch.empty(lib.bi_sdpa_workspace_bytes(B, 32, 8, 1, S, D, bi.BI_BF16), dtype=torch.uint8, device=dev)
        ms = _time_graph(torch, lambda: bi.bi_sdpa(q, k, v, causal=True, workspace=ws), reps=4, iters=6)
        gbps = 2.0 * (B * 8 * S * D * 2) / (ms * 1e-3) / 1e9
        cells["attention_forms"].append({"B": B, "S": S, "D": D, "form": "causal decode", "us": round(ms * 1e3, 1),
                                         "GBps": round(gbps, 1), "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4),
                                         "kernel": lib.bi_sdpa_kernel_name(B, 32, 8, 1, S, D, bi.BI_BF16).decode()})
        qp = torch.randn((1, 32, 2048, D), generator=gen, device=dev).to(torch.bfloat16)
        kp = torch.randn((1, 8, 2048, D), generator=gen, device=dev).to(torch.bfloat16)
        wsp = torch.empty(lib.bi_sdpa_workspace_bytes(1, 32, 8, 2048, 2048, D, bi.BI_BF16), dtype=torch.uint8, device=dev)
        ms = _time_graph(torch, lambda: bi.bi_sdpa(qp, kp, kp, causal=True, workspace=wsp), reps=2, iters=4)
        tf = 4.0 * 32 * D * (2048 * 2049 / 2) / (ms * 1e-3) / 1e12
        cells["attention_forms"].append({"B": 1, "Lq": 2048, "S": 2048, "D": D, "form": "causal prefill",
                                         "us": round(ms * 1e3, 1), "TFLOPs": round(tf, 1),
                                         "frac_mfma": round(tf / BF16_PEAK_TFLOPS, 4),
                                         "kernel": lib.bi_sdpa_kernel_name(1, 32, 8, 2048, 2048, D, bi.BI_BF16).decode()})
        del q, k, v, ws, qp, kp, wsp
    # long causal prefill (query chunk = whole cache): workspace-free kernel, flops of visible pairs
    for S in (4096, 8192):
        gen = torch.Generator(device=dev)
        gen.manual_seed(0x5EED95 + S)
        q = torch.randn((1, 32, S, 128), generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn((1, 8, S, 128), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((1, 8, S, 128), generator=gen, device=dev).to(torch.bfloat16)
        ms = _time_graph(torch, lambda: bi.bi_sdpa(q, k, v, causal=True), reps=2, iters=5)
        flops = 4.0 * 32 * 128 * (S * (S + 1) / 2)
        tf = flops / (ms * 1e-3) / 1e12
        cells["prefill_attention"].append({"B": 1, "Lq": S, "S": S, "us": round(ms * 1e3, 1), "TFLOPs": round(tf, 1),
                                           "frac_mfma": round(tf / BF16_PEAK_TFLOPS, 4),
                                           "kernel": lib.bi_sdpa_kernel_name(1, 32, 8, S, S, 128, bi.BI_BF16).decode()})
        del q, k, v
    # quantized linear (4-bit, groups of 64): packed weights rotate through copies so reads are cold;
    # bytes = packed words + scales + biases + x + y; rows checked against M = 256 on raw bits
    cells["quantized_gemm"] = []
    for N in (4096, 14336):
        wq, sc, sb = bi.quantize(data[N]["w"][0], 4, 64)
        qbytes = wq.numel() * 4 + sc.numel() * 2 * 2
        qs = [(wq, sc, sb)] + [(wq.clone(), sc.clone(), sb.clone()) for _ in range(max(1, -(-512 * 2**20 // qbytes)) - 1)]
        xq = data[N]["x"]
        full = bi.bi_quantized_linear(xq, wq, sc, sb, 4, 64)
        differing = 0
        for M in (1, 4, 16, 64, 256):
            it = iter(range(10 ** 9))
            ms = _time_graph(torch, lambda: bi.bi_quantized_linear(xq[:M], *qs[next(it) % len(qs)], 4, 64),
                             reps=len(qs), iters=5)
            nbytes = qbytes + 2.0 * (M * K + M * N)
            gbps = nbytes / (ms * 1e-3) / 1e9
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            lin = next((c["us"] for c in cells["decode_gemm"] if c["M"] == M and c["N"] == N), None)
            part = bi.bi_quantized_linear(xq[:M], wq, sc, sb, 4, 64)
            differing += int((part.view(torch.int16) != full[:M].view(torch.int16)).any(dim=1).sum().item())
            cells["quantized_gemm"].append({"M": M, "N": N, "bits": 4, "group_size": 64, "us": round(ms * 1e3, 2),
                                            "GBps": round(gbps, 1), "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4),
                                            "TFLOPs": round(tf, 1),
                                            "over_bf16_linear": round(ms * 1e3 / lin, 3) if lin else None})
        cells.setdefault("quantized_rows_differing_from_M256", 0)
        cells["quantized_rows_differing_from_M256"] += differing
        del qs
    # batch-variant comparator on the linear half of the step: cost ratio and negative control
    inv_ms = var_ms = 0.0
    diff = 0
    for N in (4096, 14336):
        dN = data[N]
        ws = dN["w"]
        full_var = bi.bi_variant_linear(dN["x"], ws[0], dN["b"])
        for M in synthetic.CFG2["M_values"]:
            x = dN["x"][:M]
            it1, it2 = iter(range(10 ** 9)), iter(range(10 ** 9))
            inv_ms += _time_graph(torch, lambda: bi.bi_linear(x, ws[next(it1) % len(ws)], dN["b"]),
                                  reps=len(ws), iters=5)
            var_ms += _time_graph(torch, lambda: bi.bi_variant_linear(x, ws[next(it2) % len(ws)], dN["b"]),
                                  reps=len(ws), iters=5)
            v = bi.bi_variant_linear(x, dN["w"][0], dN["b"])
            diff += int((v.view(torch.int16) != full_var[:M].view(torch.int16)).any(dim=1).sum().item())
    cells["comparator"] = {"invariant_ms": round(inv_ms, 4), "variant_ms": round(var_ms, 4),
                           "invariant_over_variant_time": round(inv_ms / var_ms, 4),
                           "variant_rows_differing_from_M256": diff}
    cells["e2e_decode"] = e2e_decode(torch, bi, dev, synthetic)
    return cells


def e2e_decode(torch, bi, dev, synthetic):
    """A random-weight 4-layer decoder (hidden 2048, 16 / 4 heads of 128, SwiGLU 5632, vocab 32000),
    batch 8, 128-token prompts, 32 greedy decode steps: time per decode step under
    batch_invariant_mode and with stock PyTorch (the batch-variant comparator), and how many of the
    32000 last-position logits of one sequence move between batch 1 and batch 8 in each."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import tiny_transformer as tt
    cfg = tt.TinyConfig(layers=4)
    W = tt.make_weights(cfg, 0x5EEDE5, dev)
    prompts = synthetic.randint((8, 128), 0x5EEDE6, 0, cfg.vocab, torch.int64).to(dev)
    steps = 32

    def run(invariant: bool, p):
        ctx = bi.batch_invariant_mode() if invariant else _nullcontext()
        with torch.no_grad(), ctx:
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

    for inv in (True, False):               # warm-up both paths
        run(inv, prompts)
    out = {"model": "4 layers, hidden 2048, 16/4 heads x 128, SwiGLU 5632, vocab 32000, bf16, random weights",
           "batch": 8, "prompt": 128, "decode_steps": steps}
    for name, inv in (("invariant", True), ("stock", False)):
        ms, last8 = run(inv, prompts)
        _, last1 = run(inv, prompts[:1])
        # decode logits of sequence 0 after 32 steps, alone vs in the batch of 8
        n = int((last1[0].view(torch.int16) != last8[0].view(torch.int16)).sum())
        out[name] = {"ms_per_decode_step": round(ms, 3), "tokens_per_s": round(8 * 1e3 / ms, 1),
                     "logits_differing_batch1_vs_batch8": n}
    out["invariant_over_stock_time"] = round(out["invariant"]["ms_per_decode_step"] /
                                             out["stock"]["ms_per_decode_step"], 4)
    return out


class _nullcontext:
    def __enter__(self):
        return None

    def __exit__(self, *a):
        return False


def cpu_baseline(torch, synthetic, args):
    import numpy as np  # noqa: F401
    import oracle
    if args.cpu_threads > 0:
        oracle.set_threads(args.cpu_threads)
    threads = oracle.threads()
    Ms = synthetic.CFG2["M_values"]
    inputs = [synthetic.cfg2_inputs(N, M_max=max(Ms)) for N in synthetic.CFG2["N_values"]]
    flops = 0.0
    passes = 0
    t0 = time.perf_counter()
    # whole passes over the sample until at least args.cpu_seconds have gone by
    while passes == 0 or time.perf_counter() - t0 < args.cpu_seconds:
        for d in inputs:
            # the largest batch of the sweep: its rows contain every smaller batch's rows
            oracle.linear(d["x"], d["w"], d["b"])
            flops += 2.0 * d["x"].shape[0] * d["w"].shape[0] * d["w"].shape[1]
        passes += 1
    t = time.perf_counter() - t0
    log(f"cpu oracle: {flops / 1e9:.1f} GFLOP in {t:.1f}s on {threads} threads ({passes} passes)")
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{passes} passes of the float64 oracle linear on the M=256 batch (x 256x4096, bias) "
                      "for N=4096 and N=14336, i.e. every row of the GEMM sweep once per pass; "
                      "attention not included",
            "seconds": round(t, 2)}


# ---------------------------------------------------------------- profiling helpers
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


def summarize_stats(args):
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
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
