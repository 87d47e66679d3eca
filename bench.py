#!/usr/bin/env python3
"""Benchmark of the MoLE hot path on one MI355X.

Headline workload: the 1B-class stack -- 16 MoLE layers, each with its own
50304 x 16 x 2048 bf16 table (3.3 GB; 52.7 GB in all) and router, experts
2048 -> 8192 -> 2048 with GELU -- at a decode batch of T = 1024 Zipf(1.1)
token ids, a fresh hidden state per layer.

Before the timed region every layer's table is built by mole_build_lut from
seeded N(0, 0.02) weights (the reparameterisation; each build is event-timed
and reported as `roofline_build`, 4 V N D F flop per layer).  One *step* is
one decode step through the stack: the 16 mole_lookup_combine calls on one
stream.  `value` = T / step time (tokens/s through all 16 layers).
`roofline` is the combine kernel: its algorithmic bytes (gathered table rows
+ h + y + ids + W_r) over its mean event-timed launch duration, also on the
unique rows' bytes, with a distinct-id control.

The other rows of the hot path run on their own configurations after the
headline: the 410M-class layer (build timed separately; NF3 pack and the
NF3 combine in HBM and in pinned host memory; the bf16 combine at T = 256,
1024, 4096; the NF4/int8 tables and the device-grouped combine), the
160M-class decode batches (T = 1, 8, 64, 256), the 1B-class decode sweep
(T = 1, 16, 128, 1024, eager and as HIP-graph replays), and the extra
measurements of --probes.  The CPU oracle is timed on this host on a bounded
sample (`cpu_baseline`).  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "mixture_lookup_experts_amd", "csrc")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--tokens", type=int, default=1024, help="decode batch of the headline step")
    p.add_argument("--layers", type=int, default=16, help="layers of the 1B-class stack")
    p.add_argument("--ids", default="zipf", choices=("zipf", "uniform", "distinct"),
                   help="token-id law of the headline step (a distinct-id control is always measured)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="budget for the CPU-oracle baseline (0 disables it)")
    p.add_argument("--probes", default="sweep,host1b,410m,160m,host,disk,layer,train",
                   help="comma list of the measurements after the headline (or 'none'): sweep (1B-class "
                        "decode batches), host1b (the same with 1B-class NF3 tables in page-locked host "
                        "memory, read in place), 410m (build, NF3 pack, quantised, host-resident and grouped "
                        "combines), 160m (build and decode batches), host (16-layer host-resident NF3 stack), "
                        "disk (NF3 table file), layer (the MoLE block), train (training forward and backward); "
                        "opt-in: vendor_gemm (the vendor GEMM library on the build's shapes)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run one 256 MiB device-to-device copy first (the reference kernel "
                        "that scales FETCH_SIZE / WRITE_SIZE counters to bytes)")
    return p.parse_args()


def sources_sha(*names):
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(CSRC, n), "rb").read())
    return h.hexdigest()


COMBINE_SRCS = ("combine_dense.hip", "combine_common.hpp", "mole_device.hpp", "mole_tables.hpp")
BUILD_SRCS = ("build_lut.hip", "mole_device.hpp", "mole_tables.hpp")


def committed_traffic(fname: str, workload: str, srcs, **want):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel)
    from a committed counter summary, if it was taken on this workload with
    the current kernel sources (and the same launch parameters); else None."""
    try:
        kv = dict(l.split("=", 1) for l in open(os.path.join(ROOT, "profiles", fname)).read().split("\n")
                  if "=" in l and not l.startswith("#"))
    except OSError:
        return None
    if kv.get("workload", "").strip() != workload or kv.get("sources_sha256", "").strip() != sources_sha(*srcs):
        return None
    for k, v in want.items():
        if kv.get(k, "").strip() != str(v):
            return None
    return float(kv["hbm_bytes_per_launch"])


def ev(torch):
    return torch.cuda.Event(enable_timing=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build runs on a single MI355X and has no "
              "multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_lookup_experts_amd as mole
    from mixture_lookup_experts_amd import synth

    w = synth.WORKLOADS["1b"]
    V, D, N, F, L, T = w.V, w.D, w.N, w.F, args.layers, args.tokens
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)
    probes = set() if args.probes == "none" else set(args.probes.split(","))

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    torch.cuda.set_stream(stream)
    if args.copy_calibration:
        src_c = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst_c = torch.empty_like(src_c)
        dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c

    # ---------------- the stack's tables, built from weights (not timed as a step)
    stack = build_stack(torch, mole, synth, w, L, dev, stream, to_dev)
    luts, w_rs = stack["luts"], stack["w_rs"]
    build_ms = stack["build_ms"]
    build_flops = 4.0 * V * N * D * F

    # ---------------- headline: decode steps through the stack
    NB = 8
    g = torch.Generator(device=dev)
    g.manual_seed(synth.seed(w, 10))
    h_l = [[torch.randn((T, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(L)] for _ in range(NB)]
    y_l = [torch.empty((T, D), dtype=torch.float32, device=dev) for _ in range(L)]

    def run_steps(kind, steps, warmup):
        ids_host = [synth.make_ids(w, T, step=s, kind=kind) for s in range(NB)]
        ids_l = [to_dev(x) for x in ids_host]
        uniq = float(np.mean([np.unique(x).size for x in ids_host]))

        def step(b):
            for l in range(L):
                mole.mole_lookup_combine(ids_l[b], h_l[b][l], w_rs[l], luts[l], y_l[l], stream=stream)

        for k in range(warmup):
            step(k % NB)
        # One event pair per step, recorded on `stream` (the combines' stream):
        # a timing event between two launches costs the next launch several
        # microseconds here, so the per-launch figure is the step time over its
        # L launches (inter-launch gaps included).
        evs = [(ev(torch), ev(torch)) for _ in range(steps)]
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        for k in range(steps):
            evs[k][0].record(stream)
            step(k % NB)
            evs[k][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms_step = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        kern_us = ms_step * 1e3 / L
        return ms_step, kern_us, uniq, wall, step, ids_l

    with torch.cuda.stream(stream):
        ms_step, kern_us, uniq, wall, step_fn, ids_head = run_steps(args.ids, args.steps, args.warmup)
        d_ms, d_us, d_uniq, _, _, _ = run_steps("distinct", max(5, args.steps // 2), 2)
        # the same step captured as a HIP graph per input batch and replayed
        graphs = []
        for b in range(NB):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for l in range(L):
                    mole.mole_lookup_combine(ids_head[b], h_l[b][l], w_rs[l], luts[l], y_l[l],
                                             stream=torch.cuda.current_stream())
            graphs.append(gr)
        torch.cuda.synchronize()
    for b in range(NB):
        graphs[b].replay()
    torch.cuda.synchronize()
    e0, e1 = ev(torch), ev(torch)
    e0.record()
    for r in range(2 * NB):
        graphs[r % NB].replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / (2 * NB)
    del graphs

    per_gath = T * (N * D * 2 + D * 2 + 4 * D + 8) + N * D * 2   # bytes per launch, gathered rows
    per_uniq = per_gath - (T - uniq) * N * D * 2                  # the same with each distinct row once
    gbs = per_gath / (kern_us * 1e-6) / 1e9
    traffic = committed_traffic("traffic_combine_1b_T1024.txt", "1b-stack-T%d-%s" % (T, args.ids),
                                COMBINE_SRCS)
    d_gbs = per_gath / (d_us * 1e-6) / 1e9  # distinct ids: every row once
    build_mean = float(np.mean(build_ms))
    build_traffic = committed_traffic("traffic_build_lut_1b.txt", "1b-layer", BUILD_SRCS,
                                      build_workspace_bytes=stack["ws_bytes"])
    result = {
        "metric": "lookup-combine tokens/s + HBM GB/s (% peak); LUT-build TFLOP/s (% MFMA peak)",
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: tables built by mole_build_lut from seeded N(0,0.02) weights; h ~ N(0,1) "
                "fresh per layer; %s token ids" % {"zipf": "Zipf(1.1)", "uniform": "uniform",
                                                   "distinct": "distinct"}[args.ids],
        "config": {"workload": "1B-class stack: %d MoLE layers, V=%d D=%d N=%d experts of %d->%d->%d, "
                               "bf16 tables (%.1f GB), T=%d tokens per decode step; step = the %d "
                               "lookup-combines" % (L, V, D, N, D, F, D, L * V * N * D * 2 / 1e9, T, L),
                   "V": V, "D": D, "N": N, "F": F, "layers": L, "tokens": T, "parallelism": "single GPU"},
        "roofline": {"kernel": "lookup_combine_kernel (mole_lookup_combine), one launch per layer",
                     "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "us_per_launch": kern_us, "bytes_per_launch": per_gath,
                     "timing": "HIP events around each step on the launch stream; per launch = step / %d" % L,
                     "achieved_unique": per_uniq / (kern_us * 1e-6) / 1e9,
                     "frac_unique": per_uniq / (kern_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                     "mean_unique_ids": uniq},
        "distinct_id_control": {"ms_per_step": d_ms, "tokens_per_s": T / (d_ms * 1e-3), "us_per_launch": d_us,
                                "achieved": d_gbs, "frac": d_gbs / HBM_PEAK_GBS, "mean_unique_ids": d_uniq},
        "graph_replay": {"us_per_step": graph_us, "tokens_per_s": T / (graph_us * 1e-6),
                         "gbs": L * per_gath / (graph_us * 1e-6) / 1e9},
        "roofline_build": {"kernel": "mole_build_lut (gemm_nt_bf16 GELU + store per vocabulary block), "
                                     "one 1B-class layer", "bound": "mfma",
                           "achieved": build_flops / (build_mean * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": build_flops / (build_mean * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                           "traffic": build_traffic, "ms_per_build": build_mean, "builds": len(build_ms),
                           "flops_per_build": build_flops, "workspace_bytes": stack["ws_bytes"]},
        "wall_s_timed": wall,
    }
    del h_l, y_l
    torch.cuda.synchronize()

    if "sweep" in probes:
        result["decode_sweep_1b"] = decode_sweep(torch, mole, synth, w, luts, w_rs, dev, stream, to_dev)
    if "host1b" in probes:
        result["decode_sweep_1b_nf3_host"] = host_decode_sweep(torch, mole, synth, w, w_rs, dev, stream, to_dev)
    del luts, w_rs, stack
    torch.cuda.empty_cache()
    if "410m" in probes:
        result["layer_410m"] = layer410_probe(torch, mole, synth, dev, stream, to_dev)
    if "160m" in probes:
        result["layer_160m"] = layer160_probe(torch, mole, synth, dev, stream, to_dev)
    if "host" in probes:
        result["host_stack_nf3"] = host_stack_probe(torch, mole, synth, dev, stream)
    if "disk" in probes:
        result["disk_nf3"] = disk_probe(torch, mole, synth, dev, stream)
    if "layer" in probes:
        result["layer_block"] = layer_probe(torch, mole, synth, dev, stream)
    if "train" in probes:
        result["train"] = train_probe(torch, mole, synth, dev, stream)
    if "vendor_gemm" in probes:
        result["vendor_gemm"] = vendor_gemm_probe(torch, dev, stream)

    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(args, synth, L)

    print(json.dumps(result), flush=True)


def build_stack(torch, mole, synth, w, L, dev, stream, to_dev):
    """The L layers' tables, each built by mole_build_lut (bf16) from seeded
    weights drawn on the device (N(0, 0.02), one generator seed per layer and
    tensor), with the library's recommended workspace.  One shared embedding.
    Each build is event-timed on `stream`; layer 0 is built twice (the first
    build warms up the kernels) and only the second is kept."""
    V, D, N, F = w.V, w.D, w.N, w.F
    bf = torch.bfloat16
    with torch.cuda.stream(stream):
        g = torch.Generator(device=dev)
        g.manual_seed(synth.seed(w, 0))
        emb = (torch.randn((V, D), generator=g, device=dev) * 0.02).to(bf)
        _, ws_bytes = mole.mole_build_lut_workspace_size(V, D, F, N)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        luts, w_rs, ms = [], [], []
        for l in range(L):
            g.manual_seed(synth.seed(w, 1, l))
            w_up = (torch.randn((N, F, D), generator=g, device=dev) * 0.02).to(bf)
            g.manual_seed(synth.seed(w, 2, l))
            w_down = (torch.randn((N, D, F), generator=g, device=dev) * 0.02).to(bf)
            lut = torch.empty((V, N, D), dtype=bf, device=dev)
            for rep in range(2 if l == 0 else 1):
                e0, e1 = ev(torch), ev(torch)
                e0.record(stream)
                mole.mole_build_lut(emb, w_up, w_down, lut, workspace=ws, stream=stream)
                e1.record(stream)
                torch.cuda.synchronize()
                if rep == (1 if l == 0 else 0):
                    ms.append(e0.elapsed_time(e1))
            luts.append(lut)
            w_rs.append(to_dev(synth.make_router(w, l)))
            del w_up, w_down
        del ws, emb
    torch.cuda.empty_cache()
    return {"luts": luts, "w_rs": w_rs, "build_ms": ms, "ws_bytes": ws_bytes}


def time_launches(torch, stream, fn, reps, warm=5):
    """Mean event-timed microseconds of fn(i), i = 0..reps-1, on `stream`."""
    with torch.cuda.stream(stream):
        for i in range(warm):
            fn(i)
        e0, e1 = ev(torch), ev(torch)
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def decode_sweep(torch, mole, synth, w, luts, w_rs, dev, stream, to_dev):
    """Decode batches T = 1, 16, 128, 1024 through the built stack (Zipf ids,
    the same ids at every layer, fresh h per layer): one step = the L
    lookup-combines, eager on `stream` and as one HIP-graph replay."""
    V, D, N, L = w.V, w.D, w.N, len(luts)
    g = torch.Generator(device=dev)
    g.manual_seed(synth.seed(w, 70))
    out = {}
    for T in w.tokens:
        NB = 4
        ids_l = [to_dev(synth.make_ids(w, T, step=s)) for s in range(NB)]
        h_l = [[torch.randn((T, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(L)]
               for _ in range(NB)]
        y_l = [torch.empty((T, D), dtype=torch.float32, device=dev) for _ in range(L)]

        def stack(b, st):
            for l in range(L):
                mole.mole_lookup_combine(ids_l[b % NB], h_l[b % NB][l], w_rs[l], luts[l], y_l[l], stream=st)

        eager_us = time_launches(torch, stream, lambda i: stack(i, stream), 20, warm=3)
        with torch.cuda.stream(stream):
            graphs = []
            for b in range(NB):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    stack(b, torch.cuda.current_stream())
                graphs.append(gr)
        torch.cuda.synchronize()
        graph_us = time_launches(torch, torch.cuda.current_stream(), lambda i: graphs[i % NB].replay(), 20, warm=NB)
        per_layer = T * (N * D * 2 + D * 2 + 4 * D + 8) + D * N * 2
        best = min(eager_us, graph_us)
        out["T%d" % T] = {"eager_us_per_step": eager_us, "graph_us_per_step": graph_us,
                          "tokens_per_s": T / (best * 1e-6), "gbs": L * per_layer / (best * 1e-6) / 1e9,
                          "hbm_frac": L * per_layer / (best * 1e-6) / 1e9 / HBM_PEAK_GBS,
                          "bytes_per_step": L * per_layer}
        del graphs, h_l, y_l
    torch.cuda.empty_cache()
    return out


def host_decode_sweep(torch, mole, synth, w, w_rs, dev, stream, to_dev):
    """The same decode batches through a 16-layer stack of 1B-class NF3
    tables (V=50304 N=16 D=2048: 0.67 GB each, 10.7 GB in all) left in
    page-locked host memory and read in place by the combines
    (mole_lookup_combine_nf3_mapped): one step = the L combines, eager and
    as one HIP-graph replay.  The host tables hold zero codes and scales (the
    combine's cost does not depend on their values)."""
    V, D, N, L = w.V, w.D, w.N, len(w_rs)
    CB, SB = 3 * D // 8, D // 64
    codes_h = [torch.zeros((V, N, CB), dtype=torch.uint8, pin_memory=True) for _ in range(L)]
    scales_h = [torch.zeros((V, N, SB), dtype=torch.int16, pin_memory=True) for _ in range(L)]
    g = torch.Generator(device=dev)
    g.manual_seed(synth.seed(w, 71))
    out = {"workload": "16-layer stack of 1B-class NF3 tables (V=50304 N=16 D=2048) in page-locked host "
                       "memory, %.1f GB, read in place" % (L * V * N * (CB + 2 * SB) / 1e9)}
    row = N * (CB + 2 * SB)
    for T in w.tokens:
        NB = 4
        ids_l = [to_dev(synth.make_ids(w, T, step=s)) for s in range(NB)]
        h_l = [[torch.randn((T, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(L)]
               for _ in range(NB)]
        y_l = [torch.empty((T, D), dtype=torch.float32, device=dev) for _ in range(L)]

        def stack(b, st):
            for l in range(L):
                mole.mole_lookup_combine_nf3_mapped(ids_l[b % NB], h_l[b % NB][l], w_rs[l], codes_h[l],
                                                    scales_h[l], y_l[l], stream=st)

        eager_us = time_launches(torch, stream, lambda i: stack(i, stream), 20, warm=3)
        with torch.cuda.stream(stream):
            graphs = []
            for b in range(NB):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    stack(b, torch.cuda.current_stream())
                graphs.append(gr)
        torch.cuda.synchronize()
        graph_us = time_launches(torch, torch.cuda.current_stream(), lambda i: graphs[i % NB].replay(), 20, warm=NB)
        best = min(eager_us, graph_us)
        out["T%d" % T] = {"eager_us_per_step": eager_us, "graph_us_per_step": graph_us,
                          "tokens_per_s": T / (best * 1e-6), "pcie_bytes_requested_per_step": L * T * row,
                          "pcie_gbs_effective": L * T * row / (best * 1e-6) / 1e9}
        del graphs, h_l, y_l
    del codes_h, scales_h
    torch.cuda.empty_cache()
    return out


def build_layer(torch, mole, synth, w, dev, stream, reps=3):
    """One layer's table built by mole_build_lut from seeded device-drawn
    N(0, 0.02) weights; returns (lut, w_r, mean build ms over reps builds
    after one warm-up build)."""
    V, D, N, F = w.V, w.D, w.N, w.F
    bf = torch.bfloat16
    with torch.cuda.stream(stream):
        g = torch.Generator(device=dev)
        g.manual_seed(synth.seed(w, 0))
        emb = (torch.randn((V, D), generator=g, device=dev) * 0.02).to(bf)
        g.manual_seed(synth.seed(w, 1))
        w_up = (torch.randn((N, F, D), generator=g, device=dev) * 0.02).to(bf)
        g.manual_seed(synth.seed(w, 2))
        w_down = (torch.randn((N, D, F), generator=g, device=dev) * 0.02).to(bf)
        _, ws_bytes = mole.mole_build_lut_workspace_size(V, D, F, N)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        lut = torch.empty((V, N, D), dtype=bf, device=dev)
        ms = time_launches(torch, stream, lambda i: mole.mole_build_lut(emb, w_up, w_down, lut, workspace=ws,
                                                                       stream=stream), reps, warm=1) / 1e3
        del emb, w_up, w_down, ws
    return lut, ms


def combine_entry(T, us, row_bytes, D, N, bh=2):
    byts = T * (row_bytes + D * bh + 4 * D + 8) + D * N * bh
    return {"us": us, "tokens_per_s": T / (us * 1e-6), "gbs": byts / (us * 1e-6) / 1e9,
            "hbm_frac": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "bytes": byts}


def layer410_probe(torch, mole, synth, dev, stream, to_dev):
    """The 410M-class layer (V=50304 D=1024 N=16 F=4096) and its NF3 variant:
    the table built from weights (the build timed on its own), the NF3, NF4
    and int8 encoders over it, then at T = 256, 1024 and 4096 with Zipf(1.1)
    ids and a distinct-id control: the bf16 combine, the device-grouped bf16
    combine (index + combine, both launches timed), the NF3, NF4 and int8
    combines from HBM and the NF3 combine from pinned host memory (host
    dedupe and gather, one PCIe copy of the distinct rows, combine) and read in
    place by the kernel from page-locked host memory, as is the bf16 table.  50
    launches cycling 8 id batches per point; a 1 GiB device copy in the same
    run gives the measured HBM roofline, a 256 MiB pinned copy the PCIe one."""
    w = synth.WORKLOADS["410m"]
    V, D, N, F = w.V, w.D, w.N, w.F
    CB, SB = 3 * D // 8, D // 64
    lut, build_ms = build_layer(torch, mole, synth, w, dev, stream)
    flops = 4.0 * V * N * D * F
    out = {"workload": "410M-class layer V=50304 D=1024 N=16 F=4096 bf16 (table %.2f GB)" % (V * N * D * 2 / 1e9),
           "build": {"ms": build_ms, "tflops": flops / (build_ms * 1e-3) / 1e12,
                     "mfma_frac": flops / (build_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, "flops": flops}}
    with torch.cuda.stream(stream):
        w_r = to_dev(synth.make_router(w))
        codes = torch.empty((V, N, CB), dtype=torch.uint8, device=dev)
        scales = torch.empty((V, N, SB), dtype=torch.int16, device=dev)
        codes4 = torch.empty((V, N, D // 2), dtype=torch.uint8, device=dev)
        scales4 = torch.empty((V, N, SB), dtype=torch.int16, device=dev)
        codes8 = torch.empty((V, N, D), dtype=torch.int8, device=dev)
        scales8 = torch.empty((V, N), dtype=torch.float32, device=dev)
    packs = {}
    for name, fn, wbytes in (
            ("nf3", lambda i: mole.mole_pack_nf3(lut, codes, scales, stream=stream), V * N * (CB + 2 * SB)),
            ("nf4", lambda i: mole.mole_pack_nf4(lut, codes4, scales4, stream=stream), V * N * (D // 2 + 2 * SB)),
            ("int8", lambda i: mole.mole_pack_int8(lut, codes8, scales8, stream=stream), V * N * (D + 4))):
        us = time_launches(torch, stream, fn, 5, warm=1)
        byts = V * N * D * 2 + wbytes
        packs[name] = {"ms": us / 1e3, "gbs": byts / (us * 1e-6) / 1e9,
                       "hbm_frac": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    out["pack"] = packs
    with torch.cuda.stream(stream):
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    copy_us = time_launches(torch, stream, lambda i: dst.copy_(src), 5, warm=1)
    copy_gbs = 2 * (1 << 30) / (copy_us * 1e-6) / 1e9
    out["hbm_copy_gbs_measured"] = copy_gbs
    del src, dst
    with torch.cuda.stream(stream):
        psrc = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
        pdst = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    h2d_us = time_launches(torch, stream, lambda i: pdst.copy_(psrc, non_blocking=True), 3, warm=1)
    out["pcie_h2d_gbs_measured"] = (256 << 20) / (h2d_us * 1e-6) / 1e9
    del psrc, pdst
    # host-resident NF3 table: the packed table copied to pinned host memory
    codes_h = torch.empty((V, N, CB), dtype=torch.uint8, pin_memory=True)
    scales_h = torch.empty((V, N, SB), dtype=torch.int16, pin_memory=True)
    torch.cuda.synchronize()
    codes_h.copy_(codes.cpu())
    scales_h.copy_(scales.cpu())
    lut_h = lut.cpu().pin_memory()  # the bf16 table in page-locked host memory (1.65 GB)
    g = torch.Generator(device=dev)
    g.manual_seed(synth.seed(w, 60))
    nf3_row = N * (CB + 2 * SB)
    for T in (256, 1024, 4096):
        for kind in ("zipf", "distinct"):
            ids_host = [synth.make_ids(w, T, step=s, kind=kind) for s in range(8)]
            ids_l = [to_dev(x) for x in ids_host]
            ids_cpu = [torch.from_numpy(x) for x in ids_host]
            U = float(np.mean([np.unique(x).size for x in ids_host]))
            with torch.cuda.stream(stream):
                h_l = [torch.randn((T, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(8)]
                y = torch.empty((T, D), dtype=torch.float32, device=dev)
                gws = torch.empty(mole.mole_lookup_combine_grouped_workspace_size(T), dtype=torch.uint8, device=dev)
                nb = mole.mole_nf3_host_staging_size(T, N, D)
                st_h = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
                st_d = torch.empty(nb, dtype=torch.uint8, device=dev)
            res = {"mean_unique_ids": U}
            for name, fn, row in (
                    ("bf16", lambda i: mole.mole_lookup_combine(ids_l[i % 8], h_l[i % 8], w_r, lut, y,
                                                                stream=stream), N * D * 2),
                    ("bf16_grouped", lambda i: mole.mole_lookup_combine_grouped(ids_l[i % 8], h_l[i % 8], w_r,
                                                                                lut, y, gws, stream=stream),
                     N * D * 2),
                    ("nf3", lambda i: mole.mole_lookup_combine_nf3(ids_l[i % 8], h_l[i % 8], w_r, codes, scales, y,
                                                                   stream=stream), nf3_row),
                    ("nf4", lambda i: mole.mole_lookup_combine_nf4(ids_l[i % 8], h_l[i % 8], w_r, codes4, scales4,
                                                                   y, stream=stream), N * (D // 2 + 2 * SB)),
                    ("int8", lambda i: mole.mole_lookup_combine_int8(ids_l[i % 8], h_l[i % 8], w_r, codes8,
                                                                     scales8, y, stream=stream), N * (D + 4))):
                e = combine_entry(T, time_launches(torch, stream, fn, 50), row, D, N)
                e["hbm_frac_measured"] = e["gbs"] / copy_gbs
                e["gbs_unique"] = (e["bytes"] - (T - U) * row) / (e["us"] * 1e-6) / 1e9
                res[name] = e
            # host-resident NF3: the call waits for its previous copy, so time wall clock per call too
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            us = time_launches(torch, stream, lambda i: mole.mole_lookup_combine_nf3_host(
                ids_cpu[i % 8], h_l[i % 8], w_r, codes_h, scales_h, st_h, st_d, y, stream=stream), 20)
            pcie = U * nf3_row + 8 * T
            res["nf3_host"] = {"us": us, "tokens_per_s": T / (us * 1e-6), "pcie_bytes": pcie,
                               "pcie_gbs_effective": pcie / (us * 1e-6) / 1e9,
                               "wall_s": time.perf_counter() - t0}
            # the same tables read in place by the kernel (every token reads its own rows over PCIe)
            us = time_launches(torch, stream, lambda i: mole.mole_lookup_combine_nf3_mapped(
                ids_l[i % 8], h_l[i % 8], w_r, codes_h, scales_h, y, stream=stream), 20)
            res["nf3_mapped"] = {"us": us, "tokens_per_s": T / (us * 1e-6), "pcie_bytes_requested": T * nf3_row,
                                 "pcie_gbs_effective": T * nf3_row / (us * 1e-6) / 1e9}
            us = time_launches(torch, stream, lambda i: mole.mole_lookup_combine_mapped(
                ids_l[i % 8], h_l[i % 8], w_r, lut_h, y, stream=stream), 10, warm=2)
            res["bf16_mapped"] = {"us": us, "tokens_per_s": T / (us * 1e-6),
                                  "pcie_bytes_requested": T * N * D * 2,
                                  "pcie_gbs_effective": T * N * D * 2 / (us * 1e-6) / 1e9}
            us = time_launches(torch, stream, lambda i: mole.mole_lookup_combine_nf3_grouped_mapped(
                ids_l[i % 8], h_l[i % 8], w_r, codes_h, scales_h, y, gws, stream=stream), 20)
            res["nf3_grouped_mapped"] = {"us": us, "tokens_per_s": T / (us * 1e-6),
                                         "pcie_bytes_distinct_rows": U * nf3_row,
                                         "pcie_gbs_effective_distinct": U * nf3_row / (us * 1e-6) / 1e9}
            # grouped by id on the device: each run of equal ids reads its slab over PCIe once
            us = time_launches(torch, stream, lambda i: mole.mole_lookup_combine_grouped_mapped(
                ids_l[i % 8], h_l[i % 8], w_r, lut_h, y, gws, stream=stream), 10, warm=2)
            res["bf16_grouped_mapped"] = {"us": us, "tokens_per_s": T / (us * 1e-6),
                                          "pcie_bytes_distinct_rows": U * N * D * 2,
                                          "pcie_gbs_effective_distinct": U * N * D * 2 / (us * 1e-6) / 1e9}
            out["T%d_%s" % (T, kind)] = res
            del h_l, y, gws, st_h, st_d
    del lut, codes, scales, codes4, scales4, codes8, scales8, codes_h, scales_h, lut_h
    torch.cuda.empty_cache()
    return out


def layer160_probe(torch, mole, synth, dev, stream, to_dev):
    """The 160M-class layer (V=50304 D=768 N=4 F=3072): the build timed on
    its own, the NF3 pack, and the bf16 and NF3 combines at its decode
    batches T = 1, 8, 64, 256 (Zipf ids; 50 launches cycling 8 batches),
    both also with their tables in page-locked host memory read in place.
    Every launch here moves under 3 MB: latency-bound."""
    w = synth.WORKLOADS["160m"]
    V, D, N, F = w.V, w.D, w.N, w.F
    CB, SB = 3 * D // 8, D // 64
    lut, build_ms = build_layer(torch, mole, synth, w, dev, stream, reps=5)
    flops = 4.0 * V * N * D * F
    out = {"build": {"ms": build_ms, "tflops": flops / (build_ms * 1e-3) / 1e12,
                     "mfma_frac": flops / (build_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}}
    with torch.cuda.stream(stream):
        w_r = to_dev(synth.make_router(w))
        codes = torch.empty((V, N, CB), dtype=torch.uint8, device=dev)
        scales = torch.empty((V, N, SB), dtype=torch.int16, device=dev)
    us = time_launches(torch, stream, lambda i: mole.mole_pack_nf3(lut, codes, scales, stream=stream), 5, warm=1)
    byts = V * N * D * 2 + V * N * (CB + 2 * SB)
    out["pack_nf3"] = {"ms": us / 1e3, "gbs": byts / (us * 1e-6) / 1e9,
                       "hbm_frac": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    # the NF3 table in page-locked host memory, read in place at decode sizes
    torch.cuda.synchronize()
    codes_h = codes.cpu().pin_memory()
    scales_h = scales.cpu().pin_memory()
    lut_h = lut.cpu().pin_memory()
    nf3_row = N * (CB + 2 * SB)
    for T in w.tokens:
        ids_l = [to_dev(synth.make_ids(w, T, step=s)) for s in range(8)]
        h_l = [to_dev(synth.make_hidden(w, T, step=s)) for s in range(8)]
        y = torch.empty((T, D), dtype=torch.float32, device=dev)
        us_m = time_launches(torch, stream, lambda i: mole.mole_lookup_combine_nf3_mapped(
            ids_l[i % 8], h_l[i % 8], w_r, codes_h, scales_h, y, stream=stream), 50)
        us_b = time_launches(torch, stream, lambda i: mole.mole_lookup_combine_mapped(
            ids_l[i % 8], h_l[i % 8], w_r, lut_h, y, stream=stream), 50)
        out["T%d" % T] = {
            "bf16": combine_entry(T, time_launches(torch, stream, lambda i: mole.mole_lookup_combine(
                ids_l[i % 8], h_l[i % 8], w_r, lut, y, stream=stream), 50), N * D * 2, D, N),
            "nf3": combine_entry(T, time_launches(torch, stream, lambda i: mole.mole_lookup_combine_nf3(
                ids_l[i % 8], h_l[i % 8], w_r, codes, scales, y, stream=stream), 50), nf3_row, D, N),
            "nf3_mapped": {"us": us_m, "tokens_per_s": T / (us_m * 1e-6), "pcie_bytes_requested": T * nf3_row,
                           "pcie_gbs_effective": T * nf3_row / (us_m * 1e-6) / 1e9},
            "bf16_mapped": {"us": us_b, "tokens_per_s": T / (us_b * 1e-6), "pcie_bytes_requested": T * N * D * 2,
                            "pcie_gbs_effective": T * N * D * 2 / (us_b * 1e-6) / 1e9}}
    del lut, codes, scales, codes_h, scales_h, lut_h
    torch.cuda.empty_cache()
    return out


def layer_probe(torch, mole, synth, dev, stream):
    """The full MoLE block at inference, x += shared FFN(h) + lookup(ids, h),
    for the three bf16 configurations, with a shared expert of the routed
    experts' size (D -> F -> D).  Per (configuration, T): event-timed block
    time on `stream`, and the roofline it is held to -- the larger of its
    bf16 FLOPs (4 T D F) at the MFMA peak and its algorithmic HBM bytes
    (shared weights 4 D F, gathered table rows T N D 2, h, residual read and
    write, ids, router) at the HBM peak.  Blocks of up to 128 tokens are also
    timed as HIP-graph replays (graph_us)."""
    out = {"peaks": {"bf16_tflops": BF16_PEAK_TFLOPS, "hbm_gbs": HBM_PEAK_GBS}}
    ctx = torch.cuda.stream(stream)
    ctx.__enter__()
    for name, Ts in (("160m", (1, 64, 256)), ("410m", (256, 1024, 4096)), ("1b", (1, 128, 1024))):
        w = synth.WORKLOADS[name]
        V, D, N, F = w.V, w.D, w.N, w.F
        g = torch.Generator(device=dev)
        g.manual_seed(synth.seed(w, 80))
        lut = (torch.randn((V, N, D), generator=g, device=dev) * 0.02).to(torch.bfloat16)
        w_r = (torch.randn((N, D), generator=g, device=dev) * 0.02).to(torch.bfloat16)
        wu = (torch.randn((F, D), generator=g, device=dev) * 0.02).to(torch.bfloat16)
        wd = (torch.randn((D, F), generator=g, device=dev) * 0.02).to(torch.bfloat16)
        perm = synth.rank_permutation(w)
        for T in Ts:
            NB = 4
            ids_l = [torch.from_numpy(synth.make_ids(w, T, step=s, perm=perm)).to(dev) for s in range(NB)]
            h_l = [torch.randn((T, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(NB)]
            x = torch.zeros((T, D), dtype=torch.float32, device=dev)
            ws = torch.empty(mole.mole_layer_workspace_size(T, D, F), dtype=torch.uint8, device=dev)

            def block(i):
                mole.mole_layer_forward(ids_l[i % NB], h_l[i % NB], w_r, lut, wu, wd, x, ws, stream=stream)

            for i in range(5):
                block(i)
            reps = 50 if T <= 256 else 20
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(reps):
                block(i)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            graph_us = None
            if T <= 128:
                # decode-sized blocks as a decode loop would run them: eight
                # consecutive blocks (different batches) captured once and
                # replayed, so launch overhead is off the critical path
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    cur = torch.cuda.current_stream()
                    for i in range(8):
                        mole.mole_layer_forward(ids_l[i % NB], h_l[i % NB], w_r, lut, wu, wd, x, ws, stream=cur)
                gr.replay()
                torch.cuda.synchronize()
                e0.record(stream)
                for _ in range(10):
                    gr.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                graph_us = e0.elapsed_time(e1) * 1e3 / 80
                del gr
            flops = 4.0 * T * D * F
            byts = 4.0 * D * F + T * (N * D * 2 + D * 2 + 8 * D + 8) + N * D * 2
            roof_us = max(flops / (BF16_PEAK_TFLOPS * 1e12), byts / (HBM_PEAK_GBS * 1e9)) * 1e6
            out["%s_T%d" % (name, T)] = {
                "us": us, "tokens_per_s": T / (us * 1e-6), "tflops": flops / (us * 1e-6) / 1e12,
                "gbs": byts / (us * 1e-6) / 1e9, "roofline_us": roof_us,
                "bound": "mfma" if flops / (BF16_PEAK_TFLOPS * 1e12) > byts / (HBM_PEAK_GBS * 1e9) else "hbm",
                "roofline_frac": roof_us / us, "flops": flops, "bytes": byts, "graph_us": graph_us,
                "config": "V=%d D=%d N=%d F=%d (shared FFN D->F->D), Zipf(1.1) ids" % (V, D, N, F)}
            del ws, x, h_l, ids_l
        del lut, w_r, wu, wd
        torch.cuda.empty_cache()
    torch.cuda.synchronize()
    ctx.__exit__(None, None, None)
    return out


def train_probe(torch, mole, synth, dev, stream):
    """Training mode of the routed experts: forward (every expert on the
    batch's distinct embedding rows, dense gates) and backward (router,
    hidden-state, embedding-row and expert-weight gradients), event-timed on
    `stream` for the 160M-class layer at T = 256, the 410M-class layer at
    T = 1024 and 4096 and the 1B-class layer at T = 1024 (Zipf ids, weights
    N(0, 0.02)).  Roofline: the MFMA peak on the algorithmic flops, 4 U N D F
    forward and 8 U N D F backward (U = distinct ids)."""
    out = {}
    with torch.cuda.stream(stream):
        for name, T in (("160m", 256), ("410m", 1024), ("410m", 4096), ("1b", 1024)):
            w = synth.WORKLOADS[name]
            V, D, N, F = w.V, w.D, w.N, w.F
            g = torch.Generator(device=dev)
            g.manual_seed(synth.seed(w, 90))
            bf = lambda *shape: (torch.randn(shape, generator=g, device=dev) * 0.02).to(torch.bfloat16)
            emb, w_up, w_down, w_r = bf(V, D), bf(N, F, D), bf(N, D, F), bf(N, D)
            h = torch.randn((T, D), generator=g, device=dev).to(torch.bfloat16)
            dy = torch.randn((T, D), generator=g, device=dev)
            ids = torch.from_numpy(synth.make_ids(w, T))
            uniq, remap, row_ptr, tok = mole.mole_train_index(ids, V)
            U = uniq.numel()
            uniq, remap, row_ptr, tok = (x.to(dev) for x in (uniq, remap, row_ptr, tok))
            fb, bb = mole.mole_train_workspace_size(T, U, D, F, N)
            fws = torch.empty(fb, dtype=torch.uint8, device=dev)
            bws = torch.empty(bb, dtype=torch.uint8, device=dev)
            y = torch.empty((T, D), dtype=torch.float32, device=dev)
            grads = [torch.empty(s, dtype=torch.float32, device=dev)
                     for s in ((N, F, D), (N, D, F), (N, D), (T, D), (U, D))]

            def fwd():
                mole.mole_train_forward(uniq, remap, emb, w_up, w_down, h, w_r, y, fws, stream=stream)

            def bwd():
                mole.mole_train_backward(remap, row_ptr, tok, U, V, w_up, w_down, h, w_r, dy, fws, bws, *grads,
                                         stream=stream)

            res = {"tokens": T, "distinct_ids": U, "config": "V=%d D=%d N=%d F=%d" % (V, D, N, F)}
            for lab, fn, fl in (("forward", fwd, 4.0 * U * N * D * F), ("backward", bwd, 8.0 * U * N * D * F)):
                fwd()
                for _ in range(2):
                    fn()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                reps = 10
                e0.record(stream)
                for _ in range(reps):
                    fn()
                e1.record(stream)
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / reps
                res[lab] = {"ms": ms, "tflops": fl / (ms * 1e-3) / 1e12,
                            "mfma_frac": fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
            res["tokens_per_s_fwd_bwd"] = T / ((res["forward"]["ms"] + res["backward"]["ms"]) * 1e-3)
            out["%s_T%d" % (name, T)] = res
            del emb, w_up, w_down, w_r, h, dy, fws, bws, y, grads
            torch.cuda.empty_cache()
    return out


def vendor_gemm_probe(torch, dev, stream):
    """Reference point, not part of the hot path: bf16 GEMMs through the vendor
    library (torch.matmul on 2-D contiguous operands, which dispatches to
    hipBLASLt) on the build's GEMM shapes (one expert for GEMM-2) and on two
    square shapes, event-timed on `stream`.  It bounds what a tuned library
    reaches on this part at these shapes."""
    out = {}
    with torch.cuda.stream(stream):
        for name, M, N, K in (("square_8192", 8192, 8192, 8192), ("16384x16384x4096", 16384, 16384, 4096),
                              ("160m_gemm1", 50304, 12288, 768), ("160m_gemm2_one_expert", 50304, 768, 3072),
                              ("410m_gemm2_one_expert", 50304, 1024, 4096)):
            g = torch.Generator(device=dev)
            g.manual_seed(7)
            A = (torch.randn((M, K), generator=g, device=dev) * 0.05).to(torch.bfloat16)
            B = (torch.randn((K, N), generator=g, device=dev) * 0.05).to(torch.bfloat16)
            for _ in range(3):
                torch.matmul(A, B)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 10
            e0.record(stream)
            for _ in range(reps):
                torch.matmul(A, B)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            out[name] = {"ms": ms, "tflops": tf, "mfma_frac": tf / BF16_PEAK_TFLOPS}
            del A, B
            torch.cuda.empty_cache()
    return out


def host_stack_probe(torch, mole, synth, dev, stream):
    """A 16-layer stack of 410M-class NF3 tables (V=50304 N=16 D=1024,
    0.33 GB each, 5.3 GB in all) in pinned host memory.  One decode step
    = the 16 layers' lookup-combines, run two ways: (a) per layer, the
    host-resident call (gather + copy + combine, 16 transfers); (b) one
    step-start prefetch of every layer's rows in a single transfer, then 16
    device combines on the staged rows.  Then (c) the prefetch hidden behind
    device work: the 16 layers' shared-expert FFNs (F = 4096, through
    mole_layer_forward with a one-row zero table, so its own routed pass
    reads one cached row) are enqueued on the compute stream first, the
    prefetch's host gather and copy run meanwhile (the copy on a second
    stream), and the 16 NF3 combines wait for the copy; against the same
    work in order on one stream.  And (d) the 16 combines reading each
    layer's host table in place (mole_lookup_combine_nf3_mapped: every token
    reads its own rows over PCIe, no gather or staging).  Also a pinned host->device copy of 256
    MiB, the PCIe roofline measured in the same run.  The host tables are
    left as allocated (zero pages): the combine's cost does not depend on the
    code values."""
    w = synth.WORKLOADS["410m-nf3"]
    V, D, N, L = w.V, w.D, w.N, 16
    CB, SB = 3 * D // 8, D // 64
    ctx = torch.cuda.stream(stream)
    ctx.__enter__()
    codes_h = [torch.zeros((V, N, CB), dtype=torch.uint8, pin_memory=True) for _ in range(L)]
    scales_h = [torch.zeros((V, N, SB), dtype=torch.int16, pin_memory=True) for _ in range(L)]
    g = torch.Generator(device=dev)
    g.manual_seed(synth.seed(w, 80))
    w_rs = [(torch.randn((N, D), generator=g, device=dev) * 0.02).to(torch.bfloat16) for _ in range(L)]
    w_up = [(torch.randn((4 * D, D), generator=g, device=dev) * 0.02).to(torch.bfloat16) for _ in range(L)]
    w_down = [(torch.randn((D, 4 * D), generator=g, device=dev) * 0.02).to(torch.bfloat16) for _ in range(L)]
    copy_stream = torch.cuda.Stream(device=dev)
    # PCIe roofline: one pinned 256 MiB host->device copy
    src = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        dst.copy_(src, non_blocking=True)
    e1.record(stream)
    torch.cuda.synchronize()
    h2d_gbs = 3 * (256 << 20) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    out = {"workload": "16-layer stack of 410M-class NF3 tables (V=50304 N=16 D=1024) in pinned host "
                       "memory, %.1f GB" % (L * V * N * (CB + 2 * SB) / 1e9),
           "pcie_h2d_gbs_measured": h2d_gbs}
    perm = synth.rank_permutation(w)
    for T in (256, 1024, 4096):
        NB = 3
        ids_l = [torch.from_numpy(synth.make_ids(w, T, step=s, perm=perm)) for s in range(NB)]
        h_l = [[torch.randn((T, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(L)]
               for _ in range(NB)]
        y_l = [torch.empty((T, D), dtype=torch.float32, device=dev) for _ in range(L)]
        one = mole.mole_nf3_host_staging_size(T, N, D)
        st1_h = torch.empty(one, dtype=torch.uint8, pin_memory=True)
        st1_d = torch.empty(one, dtype=torch.uint8, device=dev)
        allb = mole.mole_nf3_host_stack_staging_size(T, L, N, D)
        stL_h = torch.empty(allb, dtype=torch.uint8, pin_memory=True)
        stL_d = torch.empty(allb, dtype=torch.uint8, device=dev)
        uniq = []

        def per_layer(b):
            for l in range(L):
                uniq.append(mole.mole_lookup_combine_nf3_host(ids_l[b], h_l[b][l], w_rs[l], codes_h[l],
                                                              scales_h[l], st1_h, st1_d, y_l[l],
                                                              stream=stream))

        def prefetched(b):
            remap, layers = mole.mole_prefetch_nf3_host_stack(ids_l[b], codes_h, scales_h, stL_h, stL_d,
                                                              stream=stream)
            for l in range(L):
                mole.mole_lookup_combine_nf3(remap, h_l[b][l], w_rs[l], layers[l][0], layers[l][1], y_l[l],
                                             stream=stream)

        # (c) the shared experts' FFNs of the same 16 layers on the compute stream
        F = 4 * D
        ids0 = torch.zeros(T, dtype=torch.int64, device=dev)
        lut0 = torch.zeros((1, N, D), dtype=torch.bfloat16, device=dev)
        x_l = [torch.zeros((T, D), dtype=torch.float32, device=dev) for _ in range(L)]
        ws_l = torch.empty(mole.mole_layer_workspace_size(T, D, F), dtype=torch.uint8, device=dev)

        def ffns(b):
            for l in range(L):
                mole.mole_layer_forward(ids0, h_l[b][l], w_rs[l], lut0, w_up[l], w_down[l], x_l[l], ws_l,
                                        stream=stream)

        ids_dl = [x.to(dev) for x in ids_l]

        def mapped(b):
            # (d) each layer's table read in place by its combine: no gather, copy or staging
            for l in range(L):
                mole.mole_lookup_combine_nf3_mapped(ids_dl[b], h_l[b][l], w_rs[l], codes_h[l], scales_h[l],
                                                    y_l[l], stream=stream)

        def serial(b):
            ffns(b)
            prefetched(b)

        done = [torch.cuda.Event()]  # the previous step's combines, the last readers of stL_d
        done[0].record(stream)

        def overlapped(b):
            ffns(b)
            copy_stream.wait_event(done[0])  # the copy overwrites stL_d only after they end
            remap, layers = mole.mole_prefetch_nf3_host_stack(ids_l[b], codes_h, scales_h, stL_h, stL_d,
                                                              stream=copy_stream)
            ev = torch.cuda.Event()
            ev.record(copy_stream)
            stream.wait_event(ev)
            for l in range(L):
                mole.mole_lookup_combine_nf3(remap, h_l[b][l], w_rs[l], layers[l][0], layers[l][1], y_l[l],
                                             stream=stream)
            done[0] = torch.cuda.Event()
            done[0].record(stream)

        res = {}
        for name, fn in (("per_layer", per_layer), ("prefetched", prefetched), ("mapped", mapped),
                         ("ffn_only", ffns), ("ffn_then_prefetched", serial),
                         ("ffn_overlapped_prefetch", overlapped)):
            for b in range(2):
                fn(b % NB)
            torch.cuda.synchronize()
            # each step timed on its own (a host-bound step varies with the host's load): the median
            reps, ev_us, wall_us = 7, [], []
            for r in range(reps):
                t0 = time.perf_counter()
                e0.record(stream)
                fn(r % NB)
                e1.record(stream)
                torch.cuda.synchronize()
                wall_us.append((time.perf_counter() - t0) * 1e6)
                ev_us.append(e0.elapsed_time(e1) * 1e3)
            res[name + "_us_per_step"] = float(np.median(ev_us))
            res[name + "_wall_us_per_step"] = float(np.median(wall_us))
        # hidden: FFNs and prefetched step run one after the other, minus the overlapped step
        res["prefetch_hidden_us"] = (res["ffn_only_us_per_step"] + res["prefetched_us_per_step"]
                                     - res["ffn_overlapped_prefetch_us_per_step"])
        del x_l, ws_l
        U = float(np.mean(uniq)) if uniq else 0.0
        pcie = L * U * N * (CB + 2 * SB) + 8 * T
        best = min(res["per_layer_us_per_step"], res["prefetched_us_per_step"], res["mapped_us_per_step"])
        res.update({"mean_unique_ids": U, "pcie_bytes_per_step": pcie,
                    "pcie_gbs_effective_prefetched": pcie / (res["prefetched_us_per_step"] * 1e-6) / 1e9,
                    "tokens_per_s": T / (best * 1e-6)})
        out["T%d" % T] = res
        del st1_h, st1_d, stL_h, stL_d, h_l, y_l, ids_dl
    torch.cuda.synchronize()
    ctx.__exit__(None, None, None)
    del codes_h, scales_h, w_rs, w_up, w_down
    torch.cuda.empty_cache()
    return out


def _mount_of(path):
    """(mount point, filesystem type) holding `path`, from /proc/mounts."""
    best = ("/", "unknown")
    try:
        for line in open("/proc/mounts"):
            parts = line.split()
            mp, fs = parts[1], parts[2]
            if (path == mp or path.startswith(mp.rstrip("/") + "/")) and len(mp) >= len(best[0]):
                best = (mp, fs)
    except OSError:
        pass
    return best


def disk_probe(torch, mole, synth, dev, stream):
    """The disk tier: one 410M-class NF3 table (V=50304 N=16 D=1024,
    0.33 GB) written as a table file to the temporary directory, then
    mole_lookup_combine_nf3_file at T = 256, 1024 and 4096 Zipf ids: the
    distinct rows are read from the file (one positioned read each) into
    pinned staging, copied to the device in one transfer and combined.
    Timed per call (wall clock to the end of the combine) with the file in
    the page cache, and after dropping the file's cached pages
    (posix_fadvise DONTNEED) so the rows come from the device behind the
    filesystem -- on a RAM-backed filesystem (tmpfs) the two are the same.
    The table's code values do not change the cost."""
    import tempfile
    w = synth.WORKLOADS["410m-nf3"]
    V, D, N = w.V, w.D, w.N
    CB, SB = 3 * D // 8, D // 64
    d = tempfile.mkdtemp(prefix="mole_disk_")
    path = os.path.join(d, "table.molt")
    out = {}
    try:
        t0 = time.perf_counter()
        mole.mole_nf3_file_write(path, torch.zeros((V, N, CB), dtype=torch.uint8),
                                 torch.zeros((V, N, SB), dtype=torch.int16))
        mp, fs = _mount_of(os.path.realpath(d))
        rec = N * (CB + 2 * SB)
        out["workload"] = ("410M-class NF3 table file (V=50304 N=16 D=1024, %.2f GB, %d-byte records), %s "
                           "filesystem at %s" % ((64 + V * rec) / 1e9, rec, fs, mp))
        out["file_write_s"] = time.perf_counter() - t0
        fd = os.open(path, os.O_RDONLY)
        os.fsync(fd)  # written pages reach the device, so dropping them later works
        g = torch.Generator(device=dev)
        g.manual_seed(synth.seed(w, 85))
        w_r = (torch.randn((N, D), generator=g, device=dev) * 0.02).to(torch.bfloat16)
        perm = synth.rank_permutation(w)
        with torch.cuda.stream(stream):
            for T in (256, 1024, 4096):
                NB = 4
                ids_l = [torch.from_numpy(synth.make_ids(w, T, step=s, perm=perm)) for s in range(NB)]
                h = torch.randn((T, D), generator=g, device=dev).to(torch.bfloat16)
                y = torch.empty((T, D), dtype=torch.float32, device=dev)
                nb = mole.mole_nf3_host_staging_size(T, N, D)
                st_h = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
                st_d = torch.empty(nb, dtype=torch.uint8, device=dev)
                res = {}
                for mode in ("page_cache", "dropped"):
                    times, uniq = [], []
                    for r in range(2 + 6):
                        if mode == "dropped":
                            os.posix_fadvise(fd, 0, 0, os.POSIX_FADV_DONTNEED)
                        torch.cuda.synchronize()
                        t1 = time.perf_counter()
                        U = mole.mole_lookup_combine_nf3_file(fd, ids_l[r % NB], h, w_r, V, st_h, st_d, y,
                                                              stream=stream)
                        torch.cuda.synchronize()
                        if r >= 2:
                            times.append(time.perf_counter() - t1)
                            uniq.append(U)
                    us = float(np.median(times)) * 1e6
                    U = float(np.mean(uniq))
                    res[mode] = {"us_per_call": us, "mean_unique_ids": U, "bytes_read": U * rec,
                                 "read_gbs_effective": U * rec / (us * 1e-6) / 1e9, "tokens_per_s": T / (us * 1e-6)}
                out["T%d" % T] = res
                del st_h, st_d, h, y
        os.close(fd)
    finally:
        try:
            os.remove(path)
            os.rmdir(d)
        except OSError:
            pass
    return out


def cpu_baseline(args, synth, L):
    """The CPU oracle (plain fp64 C, OpenMP over tokens or rows) on this
    host's cores, on the headline configuration: the lookup-combine of one
    1B-class layer at the headline batch (Zipf ids), warmed up once, then
    repeated for about 40 % of the budget; the median call scaled to the
    L-layer step gives `value` (tokens/s through the stack).  The table is
    zero except the rows the batch reads: the oracle touches only those rows
    and its time does not depend on the values.  Also the build of one layer
    on a sample of vocabulary rows (extrapolated linearly to V) and the
    combine at every batch size of the 160M-, 410M- and 1B-class workloads
    (per_config, all cores and one core)."""
    import oracle

    w = synth.WORKLOADS["1b"]
    V, D, N, F, T = w.V, w.D, w.N, w.F, args.tokens
    cores = len(os.sched_getaffinity(0))
    budget = args.cpu_seconds
    t_start = time.perf_counter()
    ids = synth.make_ids(w, T, kind=args.ids)
    h = synth.make_hidden(w, T)
    w_r = synth.make_router(w)
    table = np.zeros((V, N, D), dtype=np.uint16)
    rows = np.unique(ids)
    rng = np.random.Generator(np.random.PCG64(20259998))
    table[rows] = synth.f32_to_bf16_bits(rng.standard_normal((rows.size, N, D), dtype=np.float32) * np.float32(0.02))
    oracle.lookup_combine(ids, h, w_r, table, nthreads=cores)  # warm-up (page faults, thread pool)
    times = []
    t1 = time.perf_counter()
    while time.perf_counter() - t1 < 0.4 * budget or len(times) < 3:
        t2 = time.perf_counter()
        oracle.lookup_combine(ids, h, w_r, table, nthreads=cores)
        times.append(time.perf_counter() - t2)
    comb_s = float(np.median(times))
    del table
    # build: sampled vocabulary rows of one layer (smaller weights are not
    # representative: the cost per row is 4 N D F flop)
    layer = synth.make_layer(w)
    nrow, build_s = 8, None
    t1 = time.perf_counter()
    while True:
        sel = np.arange(nrow, dtype=np.int64) * (V // nrow)
        t2 = time.perf_counter()
        oracle.build_lut_rows(layer.emb, layer.w_up, layer.w_down, rows=sel, nthreads=cores)
        dt = time.perf_counter() - t2
        build_s = dt * V / nrow
        if dt > 0.1 * budget or time.perf_counter() - t1 > 0.3 * budget or nrow >= V:
            break
        nrow *= 2
    del layer
    per_config = oracle_sweep(oracle, synth, cores)
    return {"value": T / (L * comb_s), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "lookup-combine of one 1B-class layer (V=%d N=%d D=%d) at T=%d %s ids, median of %d calls "
                      "after a warm-up call, scaled to the %d-layer step; build of one layer on %d sampled "
                      "vocabulary rows, extrapolated linearly to V" % (V, N, D, T, args.ids, len(times), L, nrow),
            "combine_s_per_layer_median": comb_s, "combine_calls": len(times),
            "combine_tokens_per_s_per_layer": T / comb_s,
            "build_s_per_layer_extrapolated": build_s, "build_rows_sampled": nrow,
            "per_config": per_config, "measured_s": time.perf_counter() - t_start}


def oracle_sweep(oracle, synth, cores):
    """The oracle's combine (and NF3 combine on the NF3 workload) at every
    batch size of the 160M-, 410M- and 1B-class workloads (one layer), on all
    host cores and on one core, Zipf ids; each point warmed once, then the
    median of the calls made in about 0.1 s."""
    out = {}
    for key in ("160m", "410m", "1b", "410m-nf3"):
        w = synth.WORKLOADS[key]
        V, D, N = w.V, w.D, w.N
        rng = np.random.Generator(np.random.PCG64(20259999))
        w_r = synth.make_router(w)
        if w.nf3:
            codes = np.zeros((V, N, 3 * D // 8), dtype=np.uint8)
            scales = np.zeros((V, N, D // 64), dtype=np.uint16)
        else:
            table = np.zeros((V, N, D), dtype=np.uint16)
        res = {}
        for T in sorted(w.tokens):
            ids = synth.make_ids(w, T)
            h = synth.make_hidden(w, T)
            rows = np.unique(ids)
            if w.nf3:
                codes[rows] = rng.integers(0, 256, size=(rows.size, N, 3 * D // 8), dtype=np.uint8)
                scales[rows] = 0x2000  # fp16 2^-7
                fn = lambda nt: oracle.lookup_combine_nf3(ids, h, w_r, codes, scales, nthreads=nt)
            else:
                table[rows] = synth.f32_to_bf16_bits(
                    rng.standard_normal(size=(rows.size, N, D), dtype=np.float32) * np.float32(0.02))
                fn = lambda nt: oracle.lookup_combine(ids, h, w_r, table, nthreads=nt)
            r = {}
            for label, nt in (("all_cores", cores), ("one_core", 1)):
                fn(nt)
                times, t1 = [], time.perf_counter()
                while time.perf_counter() - t1 < 0.1 or len(times) < 3:
                    t2 = time.perf_counter()
                    fn(nt)
                    times.append(time.perf_counter() - t2)
                r[label + "_tokens_per_s"] = T / float(np.median(times))
            res["T%d" % T] = r
        out[key] = res
    return out


if __name__ == "__main__":
    main()
