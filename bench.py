#!/usr/bin/env python3
"""Benchmark: sliding-window attention forward + backward on one MI355X.

A step is one pass of the whole path: attn_fwd (O, LSE) and the backward's two
launches (dQ, which also forms D = rowsum(dO * O); dK/dV) over the 32,768-token
workload (batch 1, 32 query / 8 KV heads, head_dim 128, causal window 1,024,
bf16), inputs resident in HBM.

value = in-window FLOPs / time: 14 * head_dim FLOPs per visible (query, key)
pair summed over query heads (forward Q K^T and P V; backward Q K^T, dO V^T,
P^T dO, dS^T Q, dS K), counted cell-exact; the recompute a split backward does
is not counted.

Prints one JSON line. With --gpus N > 1 it exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_DENSE_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
HBM_PEAK_GBS = 8000.0             # MI355X HBM3E (published)
SRC_FILES = ["sliding_window_flash_amd/csrc/attn_kernels.hip",
             "sliding_window_flash_amd/csrc/kernel_common.hpp",
             "sliding_window_flash_amd/csrc/sched.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_bf16_n32768_w1024.json")


def in_window_pairs(w) -> int:
    """Visible (query, key) cells summed over query heads, cell-exact."""
    total = 0
    for lq, lk in zip(w.lengths_q, w.lengths_k):
        delta = lk - lq
        if not w.causal:
            total += lq * lk
            continue
        # query i sees min(i + delta + 1, window) keys
        c = [min(i + delta + 1, w.window) for i in range(lq)]
        total += sum(c)
    return total * w.heads_q


def document_pairs(w, docs) -> int:
    """Visible cells of a causal window over one sequence packed from
    documents (a query sees the keys of its own document only), summed over
    query heads: the query at offset p of its document sees min(p + 1, w)."""
    assert w.batch == 1 and w.causal and w.lengths_q == w.lengths_k
    return w.heads_q * sum(sum(min(p + 1, w.window) for p in range(n)) for n in docs)


def source_hash() -> str:
    h = hashlib.sha256()
    for f in SRC_FILES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None if absent, taken on different kernel sources or on another workload."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except OSError:
        return None
    if t.get("source_hash") != source_hash() or t.get("workload") != workload:
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


KERNEL_NAMES = {"fwd_kernel": "fwd", "bwd_delta_kernel": "bwd_delta", "bwd_dq_kernel": "bwd_dq",
                "bwd_dkdv_kernel": "bwd_dkdv", "bwd_dkdv4_kernel": "bwd_dkdv"}


def write_traffic(fetch_csv: str, write_csv: str, copy_mib: int, commands: list, workload: str) -> dict:
    """Turn two rocprofv3 --pmc CSVs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)
    of a run made with --copy-calibration-mib into HBM bytes per launch of each
    kernel. The counters' scale is taken from the calibration copy, a kernel
    that reads and writes copy_mib MiB once: factor = known bytes / counted."""
    import csv
    import re
    from collections import defaultdict

    def read(path, counter):
        out = []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    out.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
        return out

    fetch, write = read(fetch_csv, "FETCH_SIZE"), read(write_csv, "WRITE_SIZE")
    known = copy_mib << 20
    # the calibration copy: the runtime's copy kernel (torch's device copy_)
    # that reads the most, else the non-attention dispatch that reads the most
    # (a fill writes as much but reads nothing); then the same kernel's write
    copies = [r for r in fetch if "copyBuffer" in r[0]]
    cf = max(copies or [r for r in fetch if "swa" not in r[0]], key=lambda r: r[2])
    cw = max((r for r in write if r[0] == cf[0] and r[1] == cf[1]), key=lambda r: r[2])
    f_fetch, f_write = known / (cf[2] * 1024), known / (cw[2] * 1024)

    def per_kernel(rows, factor):
        acc = defaultdict(list)
        for name, _, kib in rows:
            m = re.search(r"swa\d+(bwd_dkdv4_kernel|bwd_dkdv_kernel|bwd_delta_kernel|bwd_dq_kernel|fwd_kernel)",
                          name)
            if m and "Lb1E" not in name:  # the masked instantiations are another workload
                acc[KERNEL_NAMES[m.group(1)]].append(kib * 1024 * factor)
        return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}

    pf, pw = per_kernel(fetch, f_fetch), per_kernel(write, f_write)
    kernels = {k: {"fetch_bytes_per_launch": round(pf[k][0]), "write_bytes_per_launch": round(pw[k][0]),
                   "hbm_bytes_per_launch": round(pf[k][0] + pw[k][0]), "dispatches": pf[k][1]}
               for k in pf if k in pw}
    return {"source_hash": source_hash(), "workload": workload,
            "commands": commands,
            "calibration": {"kernel": cw[0], "bytes_read_and_written": known,
                            "fetch_kib": cf[2], "write_kib": cw[2],
                            "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4)},
            "kernels": kernels}


def cpu_baseline(w, x, rows: int):
    """The fp64 oracle, untuned, on a bounded sample of the same workload:
    query head 0, query rows [0, rows) of each sequence, full forward + backward."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import dense

    t0 = time.perf_counter()
    dense.sdpa_reference(x["q"], x["k"], x["v"], x["do"], x["cu_q"], x["cu_k"], w.scale, w.window,
                         w.causal, heads=[0], query_rows=(0, rows))
    dt = time.perf_counter() - t0
    pairs = 0
    for lq, lk in zip(w.lengths_q, w.lengths_k):
        delta = lk - lq
        pairs += sum(min(i + delta + 1, w.window) for i in range(min(rows, lq)))
    flops = 14 * w.head_dim * pairs
    info = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in info] + [1])
    blas = ", ".join(sorted({f"{p.get('internal_api', '?')} {p.get('version', '')}".strip()
                             for p in info if p.get("user_api") == "blas"})) or "unknown"
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model, "blas": blas,
            "sample": f"query head 0, query rows [0, {rows}) of each sequence; fp64 numpy dense "
                      f"masked score panels, forward + backward; {dt:.1f} s",
            "seconds": round(dt, 2)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="bf16_n32768_w1024_32q8kv_d128")
    ap.add_argument("--cpu-rows", type=int, default=32768,
                    help="query rows per sequence in the oracle's timing sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-memory-sweep", action="store_true")
    ap.add_argument("--no-gemma", action="store_true",
                    help="skip the head_dim-256 memory-probe shape (timing and peak-bytes sweep)")
    ap.add_argument("--gemma-steps", type=int, default=10)
    ap.add_argument("--no-masked", action="store_true",
                    help="skip the document-mask leg (the workload's tokens packed from documents)")
    ap.add_argument("--masked-steps", type=int, default=10)
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads' timing (2K windowed, 8K causal, ragged batch)")
    ap.add_argument("--config-steps", type=int, default=10)
    ap.add_argument("--no-ce", action="store_true",
                    help="skip the linear cross-entropy leg (the second workload)")
    ap.add_argument("--ce-steps", type=int, default=5)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (a known-size kernel for "
                         "scaling hardware byte counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: write the HBM traffic summary from two rocprofv3 --pmc CSVs "
                         "of a run with --copy-calibration-mib, then exit")
    ap.add_argument("--traffic-command", action="append", default=[],
                    help="the rocprofv3 command lines that made the CSVs (recorded in the summary)")
    args = ap.parse_args()

    if args.traffic_from:
        if args.copy_calibration_mib <= 0:
            print("--traffic-from needs the --copy-calibration-mib of the profiled run", file=sys.stderr)
            return 2
        t = write_traffic(*args.traffic_from, args.copy_calibration_mib, args.traffic_command, args.workload)
        with open(TRAFFIC_FILE, "w") as fh:
            json.dump(t, fh, indent=1)
            fh.write("\n")
        print(json.dumps(t["kernels"]))
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported by this build "
              "(the path runs on a single MI355X).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import sliding_window_flash_amd as swa
    from sliding_window_flash_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    swa.lib()  # fails loudly if the HIP library is missing
    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    x = W.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v, do = (torch.from_numpy(x[n]).to(dt).to(dev) for n in ("q", "k", "v", "do"))
    cu_q = torch.from_numpy(x["cu_q"]).to(dev)
    cu_k = torch.from_numpy(x["cu_k"]).to(dev)
    kw = dict(max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k, window=w.window,
              causal=w.causal, scale=w.scale)
    p = swa.params_for(q, k, cu_q, cu_k, **kw)
    o = torch.empty_like(q)
    lse = torch.empty((w.heads_q, w.total_q), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(swa.workspace_bytes(p), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    # the backward is two launches: dQ (which also forms D = rowsum(dO * O) and
    # LSE * log2 e for dK/dV) and dK/dV
    names = ["fwd", "bwd_dq", "bwd_dkdv"]
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        swa.fwd(q, k, v, cu_q, cu_k, out=o, lse=lse, **kw)
        if evs is not None:
            evs[1].record(stream)
        for n, stage in enumerate((swa.BWD_DQ, swa.BWD_DKDV)):
            swa.bwd(q, k, v, o, lse, do, cu_q, cu_k, dq=dq, dk=dk, dv=dv, workspace=ws,
                    stages=stage, **kw)
            if evs is not None:
                evs[2 + n].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    kern_ms = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(names)}

    d = w.head_dim
    pairs = in_window_pairs(w)
    flops_counted = 14 * d * pairs
    value = flops_counted / (ms_per_step * 1e-3) / 1e12
    # Work of each launch per visible (query, key) pair, in head_dim units d:
    # counted = the metric's in-window FLOPs (forward Q K^T and P V: 4d;
    # backward 10d, of which dQ's launch does dS K: 2d, and dK/dV's launch
    # Q K^T, dO V^T, P^T dO, dS^T Q: 8d); executed = what the launch runs
    # (dQ also recomputes S and dP: 6d). D = rowsum(dO * O), formed in dQ's
    # prologue, adds no contraction. At head_dim 256 the dK/dV launch forms S
    # twice (a dV pass, then a dK pass: 10d); at 512 the forward and dQ run
    # four passes of 128 output columns, each recomputing S (and dP), and the
    # dK/dV passes run four times each (forward 10d, dQ 18d, dK/dV 28d).
    fwd_x, dq_x, dkdv_x = (4, 6, 8) if d <= 128 else ((4, 6, 10) if d == 256 else (10, 18, 28))
    algo = {"fwd": (4, fwd_x), "bwd_dq": (2, dq_x), "bwd_dkdv": (8, dkdv_x)}
    kernels = {}
    for n in names:
        counted, executed = algo[n]
        sec = kern_ms[n] * 1e-3
        ach = counted * d * pairs / sec / 1e12
        ach_x = executed * d * pairs / sec / 1e12
        kernels[n] = {"ms": round(kern_ms[n], 4), "bound": "mfma", "achieved": round(ach, 2),
                      "peak": BF16_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(ach / BF16_DENSE_PEAK_TFLOPS, 4),
                      "flop_per_pair_counted": counted * d, "flop_per_pair_executed": executed * d,
                      "achieved_executed": round(ach_x, 2),
                      "frac_executed": round(ach_x / BF16_DENSE_PEAK_TFLOPS, 4)}
    # The stage API's separate D pass (D and LSE * log2 e, for callers that run
    # dK/dV without dQ): not part of the step, HBM-bound. Algorithmic bytes:
    # O and dO read once, LSE read, the two fp32 [Hq, T] outputs written.
    dev_ = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in dev_:
        e[0].record(stream)
        swa.bwd(q, k, v, o, lse, do, cu_q, cu_k, dq=dq, dk=dk, dv=dv, workspace=ws, stages=swa.BWD_DELTA, **kw)
        e[1].record(stream)
    torch.cuda.synchronize()
    delta_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in dev_]))
    delta_bytes = 2 * q.numel() * q.element_size() + 3 * lse.numel() * 4
    delta_gbs = delta_bytes / (delta_ms * 1e-3) / 1e9
    kernels_other = {"bwd_delta": {"ms": round(delta_ms, 4), "bound": "hbm", "achieved": round(delta_gbs, 1),
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(delta_gbs / HBM_PEAK_GBS, 4),
                                   "bytes_per_launch": delta_bytes,
                                   "note": "stage API only; attn_bwd forms D inside dQ"}}
    dom = max(("fwd", "bwd_dq", "bwd_dkdv"), key=lambda n: kern_ms[n])
    traffic = load_traffic(dom, w.name)
    roofline = {k: v for k, v in kernels[dom].items() if k in ("bound", "achieved", "peak", "unit", "frac")}
    roofline["kernel"] = dom
    roofline["traffic"] = traffic

    # synthetic device inputs of a workload (N(0,1); dO scaled like the workloads)
    def device_inputs(wl, seed=0):
        g = torch.Generator(device=dev).manual_seed(seed)
        t = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        dh = wl.head_dim
        qq = torch.randn((wl.total_q, wl.heads_q, dh), generator=g, device=dev).to(t)
        kk = torch.randn((wl.total_k, wl.heads_kv, dh), generator=g, device=dev).to(t)
        vv = torch.randn((wl.total_k, wl.heads_kv, dh), generator=g, device=dev).to(t)
        dd = (torch.randn((wl.total_q, wl.heads_q, dh), generator=g, device=dev) * wl.do_scale).to(t)
        cq = torch.tensor(wl.cu_seqlens_q(), device=dev)
        ck = torch.tensor(wl.cu_seqlens_k(), device=dev)
        kw_ = dict(max_seqlen_q=wl.max_seqlen_q, max_seqlen_k=wl.max_seqlen_k, window=wl.window,
                   causal=wl.causal, scale=wl.scale)
        return (qq, kk, vv, dd, cq, ck), kw_

    # peak device memory of one fwd + bwd (all buffers come from torch)
    def peak_for(wl, xin=None):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        (qq, kk, vv, dd, cq, ck), kk_ = device_inputs(wl)
        torch.cuda.synchronize()
        inputs = torch.cuda.memory_allocated() - base
        torch.cuda.reset_peak_memory_stats()
        oo, ll = swa.fwd(qq, kk, vv, cq, ck, **kk_)
        swa.bwd(qq, kk, vv, oo, ll, dd, cq, ck, **kk_)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        del qq, kk, vv, dd, oo, ll
        return peak, inputs

    del_list = [o, lse, dq, dk, dv, ws]
    peak, inputs = peak_for(w)
    mem = {"peak_gb": round(peak / 1e9, 4), "peak_above_inputs_gb": round((peak - inputs) / 1e9, 4)}
    if not args.no_memory_sweep and w.batch == 1 and w.causal:
        sweep = {}
        for n in (8192, 16384, 32768):
            wl = w.replace(lengths_q=(n,), lengths_k=(n,))
            pk, inp = peak_for(wl)
            sweep[str(n)] = round((pk - inp) / 1e9, 4)
        mem["peak_above_inputs_gb_by_tokens"] = sweep
        mem["peak_ratio_per_doubling"] = [round(sweep["16384"] / sweep["8192"], 3),
                                          round(sweep["32768"] / sweep["16384"], 3)]
    del del_list

    # The memory-probe shape (head_dim 256, 32 query / 16 KV heads, w 1024):
    # fwd + bwd throughput at 32K tokens and peak bytes above inputs at 8K,
    # 16K and 32K tokens.
    gemma = None
    if not args.no_gemma:
        gw = W.GEMMA_32K
        (qq, kk, vv, dd, cq, ck), gkw = device_inputs(gw)
        oo, ll = torch.empty_like(qq), torch.empty((gw.heads_q, gw.total_q), dtype=torch.float32, device=dev)
        dq2, dk2, dv2 = torch.empty_like(qq), torch.empty_like(kk), torch.empty_like(vv)
        ws2 = torch.empty(swa.workspace_bytes(swa.params_for(qq, kk, cq, ck, **gkw)), dtype=torch.uint8,
                          device=dev)

        def gstep():
            swa.fwd(qq, kk, vv, cq, ck, out=oo, lse=ll, **gkw)
            swa.bwd(qq, kk, vv, oo, ll, dd, cq, ck, dq=dq2, dk=dk2, dv=dv2, workspace=ws2, **gkw)

        for _ in range(3):
            gstep()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.gemma_steps):
            gstep()
        e1.record(stream)
        torch.cuda.synchronize()
        g_ms = e0.elapsed_time(e1) / args.gemma_steps
        g_flops = 14 * gw.head_dim * in_window_pairs(gw)
        del qq, kk, vv, dd, oo, ll, dq2, dk2, dv2, ws2
        gsweep = {}
        for n in (8192, 16384, 32768):
            pk, inp = peak_for(gw.replace(lengths_q=(n,), lengths_k=(n,)))
            gsweep[str(n)] = round((pk - inp) / 1e9, 4)
        gemma = {"workload": gw.name, "ms_per_step": round(g_ms, 4), "steps": args.gemma_steps,
                 "tflops": round(g_flops / (g_ms * 1e-3) / 1e12, 2),
                 "pct_bf16_peak": round(100 * g_flops / (g_ms * 1e-3) / 1e12 / BF16_DENSE_PEAK_TFLOPS, 2),
                 "peak_above_inputs_gb_by_tokens": gsweep,
                 "peak_ratio_per_doubling": [round(gsweep["16384"] / gsweep["8192"], 3),
                                             round(gsweep["32768"] / gsweep["16384"], 3)]}

    # The other bf16 workloads (parity configurations, not the headline): the
    # 2K windowed case, the 8K full-causal case with forward and backward
    # timed separately (the mlx-train-perf README times its flash op at this
    # shape on an M1 Max: 0.186 s forward, 0.576 s backward; another machine
    # and stack, quoted as context) and the ragged packed batch.
    configs = None
    if not args.no_configs:
        configs = {}
        for name in ("bf16_n2048_w1024_32q8kv_d128", "bf16_n8192_causal_32q8kv_d128",
                     "bf16_varlen4_w1024_32q8kv_d128"):
            cw = W.WORKLOADS[name]
            # two input and output sets, used in turn: the 2K and 8K workloads
            # (40 and 160 MB) would otherwise stay in the 256 MB last-level
            # cache from one step to the next
            sets = []
            for seed in (0, 1):
                (qq, kk, vv, dd, cq, ck), ckw = device_inputs(cw, seed)
                oo = torch.empty_like(qq)
                ll = torch.empty((cw.heads_q, cw.total_q), dtype=torch.float32, device=dev)
                dq4, dk4, dv4 = torch.empty_like(qq), torch.empty_like(kk), torch.empty_like(vv)
                ws4 = torch.empty(swa.workspace_bytes(swa.params_for(qq, kk, cq, ck, **ckw)), dtype=torch.uint8,
                                  device=dev)
                sets.append((qq, kk, vv, dd, cq, ck, oo, ll, dq4, dk4, dv4, ws4))
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.config_steps)]

            def cstep(n, e=None):
                qq, kk, vv, dd, cq, ck, oo, ll, dq4, dk4, dv4, ws4 = sets[n % 2]
                if e is not None:
                    e[0].record(stream)
                swa.fwd(qq, kk, vv, cq, ck, out=oo, lse=ll, **ckw)
                if e is not None:
                    e[1].record(stream)
                swa.bwd(qq, kk, vv, oo, ll, dd, cq, ck, dq=dq4, dk=dk4, dv=dv4, workspace=ws4, **ckw)
                if e is not None:
                    e[2].record(stream)

            for n in range(4):
                cstep(n)
            torch.cuda.synchronize()
            for n, e in enumerate(ev):
                cstep(n, e)
            torch.cuda.synchronize()
            f_ms = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
            b_ms = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
            cp = in_window_pairs(cw)
            d_ = cw.head_dim
            configs[name] = {
                "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
                "fwd_tflops": round(4 * d_ * cp / (f_ms * 1e-3) / 1e12, 2),
                "bwd_tflops": round(10 * d_ * cp / (b_ms * 1e-3) / 1e12, 2),
                "tflops": round(14 * d_ * cp / ((f_ms + b_ms) * 1e-3) / 1e12, 2),
                "in_window_pairs": cp, "steps": args.config_steps, "input_sets": 2}
            if name == "bf16_n8192_causal_32q8kv_d128":
                configs[name]["pages_m1_max_s"] = {"fwd": 0.186, "bwd": 0.576}
            del sets

    # The workload with an arbitrary mask combined with the window: its tokens
    # packed from corpus-like documents (block-diagonal mask, bit-packed rows).
    # Counted FLOPs are 14d per cell that both the window and the mask show.
    masked = None
    if not args.no_masked and w.batch == 1 and w.causal and w.lengths_q == w.lengths_k:
        o2, l2 = torch.empty_like(q), torch.empty((w.heads_q, w.total_q), dtype=torch.float32, device=dev)
        dq3, dk3, dv3 = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws3 = torch.empty(swa.workspace_bytes(p), dtype=torch.uint8, device=dev)

        def time_masked(mt, rng=None):
            def mstep():
                swa.fwd(q, k, v, cu_q, cu_k, out=o2, lse=l2, mask=mt, mask_ranges=rng, **kw)
                swa.bwd(q, k, v, o2, l2, do, cu_q, cu_k, dq=dq3, dk=dk3, dv=dv3, workspace=ws3, mask=mt,
                        mask_ranges=rng, **kw)
            for _ in range(3):
                mstep()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(args.masked_steps):
                mstep()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.masked_steps

        def leg(name, docs):
            """One document-packed workload, timed without and with the mask's
            ranges (attn_mask_ranges, computed once beside the timed region
            and also timed alone). Counted FLOPs are 14d per cell that both the
            window and the mask show."""
            mt = torch.from_numpy(W.document_mask_bits(w, [docs]).view(np.int32)).to(dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            rng = swa.mask_ranges(q, k, cu_q, cu_k, mt, **kw)
            torch.cuda.synchronize()
            e0.record(stream)
            rng = swa.mask_ranges(q, k, cu_q, cu_k, mt, out=rng, **kw)
            e1.record(stream)
            torch.cuda.synchronize()
            r_ms = e0.elapsed_time(e1)
            plain_ms = time_masked(mt)
            skip_ms = time_masked(mt, rng)
            m_pairs = document_pairs(w, docs)
            m_tf = 14 * d * m_pairs / (skip_ms * 1e-3) / 1e12
            out = {"workload": w.name + " " + name, "documents": len(docs), "longest_document": max(docs),
                   "mask_bytes": int(mt.numel() * 4), "ms_per_step": round(skip_ms, 4),
                   "ms_per_step_without_ranges": round(plain_ms, 4), "mask_ranges_ms": round(r_ms, 4),
                   "steps": args.masked_steps, "visible_pairs": m_pairs,
                   "visible_over_window_pairs": round(m_pairs / pairs, 4), "tflops": round(m_tf, 2),
                   "pct_bf16_peak": round(100 * m_tf / BF16_DENSE_PEAK_TFLOPS, 2),
                   "time_vs_unmasked": round(skip_ms / ms_per_step, 3),
                   "time_vs_unmasked_without_ranges": round(plain_ms / ms_per_step, 3)}
            del mt, rng
            return out

        docs = W.document_lengths(91, w.lengths_k[0])
        masked = leg("packed from documents", docs)
        masked["document_lengths"] = docs
        # documents of at most 512 tokens under the 1,024-token window: most
        # of each query tile's window belongs to other documents
        masked_short = leg("packed from documents of at most 512 tokens",
                           W.short_document_lengths(92, w.lengths_k[0], 512))
        masked["short_documents"] = masked_short
        del o2, l2, dq3, dk3, dv3, ws3

    # The second workload: the linear cross-entropy without the logits tensor
    # at the mlx-train-perf README's loss-layer shape. Forward 2 n V D FLOPs
    # (the logits), backward 4 n V D (the logits again and dH = dz W).
    ce_leg = None
    if not args.no_ce:
        cw = W.CE_BENCH
        g = torch.Generator(device=dev).manual_seed(cw.seed)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base_mem = torch.cuda.memory_allocated()
        ch = torch.randn((cw.n, cw.hidden), generator=g, device=dev).to(torch.bfloat16)
        cwh = (torch.randn((cw.vocab, cw.hidden), generator=g, device=dev) / math.sqrt(cw.hidden)).to(torch.bfloat16)
        ct = torch.randint(0, cw.vocab, (cw.n,), generator=g, device=dev, dtype=torch.int32)
        cg = torch.full((cw.n,), 1.0 / cw.n, device=dev)
        torch.cuda.synchronize()
        inputs_mem = torch.cuda.memory_allocated() - base_mem
        torch.cuda.reset_peak_memory_stats()
        nll_, lse_, tgt_ = swa.ce_fwd(ch, cwh, ct)
        dh_ = swa.ce_bwd(ch, cwh, ct, lse_, cg)
        torch.cuda.synchronize()
        ce_peak = torch.cuda.max_memory_allocated() - base_mem - inputs_mem
        fws = torch.empty(swa.lib().ce_fwd_workspace_bytes(ctypes.byref(swa.ce_params_for(ch, cwh))),
                          dtype=torch.uint8, device=dev)
        bws = torch.empty(swa.lib().ce_bwd_workspace_bytes(ctypes.byref(swa.ce_params_for(ch, cwh))),
                          dtype=torch.uint8, device=dev)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        fms, bms = [], []
        for it in range(args.ce_steps + 1):
            ev[0].record(stream)
            swa.ce_fwd(ch, cwh, ct, nll=nll_, lse=lse_, tgt=tgt_, workspace=fws)
            ev[1].record(stream)
            swa.ce_bwd(ch, cwh, ct, lse_, cg, dh=dh_, workspace=bws)
            ev[2].record(stream)
            torch.cuda.synchronize()
            if it:  # the first pass is a warmup
                fms.append(ev[0].elapsed_time(ev[1]))
                bms.append(ev[1].elapsed_time(ev[2]))
        f_ms, b_ms = float(np.mean(fms)), float(np.mean(bms))
        nvd = cw.n * cw.vocab * cw.hidden
        ce_leg = {"workload": cw.name, "tokens": cw.n, "vocab": cw.vocab, "hidden": cw.hidden, "dtype": cw.dtype,
                  "steps": args.ce_steps, "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
                  "fwd_tflops": round(2 * nvd / (f_ms * 1e-3) / 1e12, 2),
                  "bwd_tflops": round(4 * nvd / (b_ms * 1e-3) / 1e12, 2),
                  "fwd_pct_bf16_peak": round(100 * 2 * nvd / (f_ms * 1e-3) / 1e12 / BF16_DENSE_PEAK_TFLOPS, 2),
                  "bwd_pct_bf16_peak": round(100 * 4 * nvd / (b_ms * 1e-3) / 1e12 / BF16_DENSE_PEAK_TFLOPS, 2),
                  "peak_above_inputs_gb": round(ce_peak / 1e9, 4),
                  "logits_tensor_not_built_gb": round(cw.n * cw.vocab * 2 / 1e9, 3)}
        del ch, cwh, ct, cg, nll_, lse_, tgt_, dh_, fws, bws

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, x, args.cpu_rows)

    line = {
        "metric": "SWA fwd+bwd TFLOP/s (in-window) + % bf16 MFMA peak, N=32768 w=1024; peak GB",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "tokens": list(w.lengths_q),
                   "heads_q": w.heads_q, "heads_kv": w.heads_kv, "head_dim": d,
                   "window": w.window, "causal": w.causal, "in_window_pairs": pairs,
                   "flops_counted": flops_counted},
        "pct_bf16_peak": round(100 * value / BF16_DENSE_PEAK_TFLOPS, 2),
        "fwd_ms": round(kern_ms["fwd"], 4),
        "bwd_ms": round(kern_ms["bwd_dq"] + kern_ms["bwd_dkdv"], 4),
        "kernels": kernels,
        "kernels_other": kernels_other,
        "roofline": roofline,
        "memory": mem,
        "memory_probe_shape": gemma,
        "other_configs": configs,
        "masked_documents": masked,
        "linear_cross_entropy": ce_leg,
        "cpu_baseline": cpu,
        "source_hash": source_hash(),
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
