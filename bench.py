#!/usr/bin/env python3
"""Benchmark of the MoLE hot path on one MI355X.

One *step* is one pass of every row of the hot path over one batch of
synthetic input, in the order a deployment runs them:

  1. mole_build_lut            reparameterise the N routed experts into the
                               token-id table LUT[V][N][D] (bf16 MFMA GEMMs);
  2. mole_pack_nf3             compress the table to 3-bit NF3 codes + scales;
  3. mole_lookup_combine       router softmax + gather + combine of T tokens
                               from the bf16 table in HBM;
  4. mole_lookup_combine_nf3   the same from the NF3 table in HBM;
  5. mole_lookup_combine_nf3_host  the same with the NF3 table in pinned host
                               memory: host dedupe/gather, PCIe copy of the
                               distinct rows, combine.

Default workload: the 160M-class layer (V=50304, D=768, N=4 experts of
768->3072->768, bf16) with a batch of T=256 Zipf(1.1) token ids.  All inputs
are seeded synthetic arrays already resident in HBM (or pinned host memory
for row 5) before the timed region; 8 pre-drawn (ids, h) batches are cycled.

Printed: ONE JSON line.  `value` is whole-step throughput (T tokens per
step / measured step time); per-row figures (build TFLOP/s, combine
tokens/s and GB/s, ...) are in `rows`; `roofline` describes the dominant
kernel of the step (the LUT build) and `roofline_combine` the combine.
The CPU oracle is timed on a bounded sample on this host (`cpu_baseline`).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="160m", help="160m | 410m | 1b | tiny")
    p.add_argument("--tokens", type=int, default=256)
    p.add_argument("--ids", default=None, choices=("zipf", "uniform", "distinct"),
                   help="token-id law (default: the workload's own; 'distinct' = no repeats, "
                        "so gathered bytes = unique bytes)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="budget for the CPU-oracle baseline (0 disables it)")
    p.add_argument("--probes", default="scale,decode,host,disk,layer,train",
                   help="comma list of the extra measurements to run: scale (combine on the 410M-class "
                        "table), decode (1B-class 16-layer stack), host (host-resident NF3 stack), "
                        "disk (NF3 table file, rows read per call), layer (the full MoLE block: shared FFN + lookup + residual), train (training-mode "
                        "forward and backward of the routed experts); not in the default "
                        "list: vendor_gemm (the vendor GEMM library, via torch.matmul, on the build's GEMM "
                        "shapes and two square ones, as a practical MFMA ceiling)")
    p.add_argument("--no-scale-probe", action="store_true",
                   help="skip the 410M-class combine measurement at T=1024/4096")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run one 256 MiB device-to-device copy first (the reference kernel "
                        "that scales FETCH_SIZE / WRITE_SIZE counters to bytes)")
    return p.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_build_lut_160m.txt")
BUILD_SRC = os.path.join(ROOT, "mixture_lookup_experts_amd", "csrc", "build_lut.hip")


def measured_traffic(workload: str, ws_bytes: int):
    """HBM bytes per build call from the committed counter summary, if it
    was taken on this workload, with the current build kernel source and the
    same build workspace (which sets the vocabulary blocks, hence the launches)."""
    import hashlib
    try:
        kv = dict(l.split("=", 1) for l in open(TRAFFIC_FILE).read().split("\n")
                  if "=" in l and not l.startswith("#"))
        src = hashlib.sha256(open(BUILD_SRC, "rb").read()).hexdigest()
    except OSError:
        return None
    if kv.get("workload", "").strip() != workload or kv.get("build_lut_sha256", "").strip() != src:
        return None
    if kv.get("build_workspace_bytes", "").strip() != str(ws_bytes):
        return None
    return float(kv["bytes_per_build"])


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build runs on a single MI355X and has no "
              "multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_lookup_experts_amd as mole
    from mixture_lookup_experts_amd import synth

    w = synth.WORKLOADS[args.workload]
    V, D, N, F, T = w.V, w.D, w.N, w.F, args.tokens
    bf16 = w.dtype == "bf16"
    tdt = torch.bfloat16 if bf16 else torch.float32
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    # ---------------- inputs (host draws -> HBM), outside the timed region,
    # produced on `stream` (the stream every kernel below runs on)
    torch.cuda.set_stream(stream)
    layer = synth.make_layer(w)
    emb, w_up, w_down, w_r = (to_dev(x) for x in (layer.emb, layer.w_up, layer.w_down, layer.w_r))
    perm = synth.rank_permutation(w)
    NB = 8
    ids_h = [synth.make_ids(w, T, step=s, kind=args.ids, perm=perm) for s in range(NB)]
    batches = [(to_dev(ids_h[s]), to_dev(synth.make_hidden(w, T, step=s))) for s in range(NB)]
    uniq = [np.unique(x).size for x in ids_h]

    lut = torch.empty((V, N, D), dtype=tdt, device=dev)
    ws = None
    if bf16:
        # the library's recommended workspace: vocabulary blocks whose hidden
        # activations (about 256 MB) fit the last-level cache; timed the same
        # as one block over all of V in this step, at a fifth of the memory
        _, ws_bytes = mole.mole_build_lut_workspace_size(V, D, F, N)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    nf3 = D % 64 == 0
    CB, SB = 3 * D // 8, D // 64
    codes = torch.empty((V, N, CB), dtype=torch.uint8, device=dev)
    scales = torch.empty((V, N, SB), dtype=torch.int16, device=dev)
    y = torch.empty((T, D), dtype=torch.float32, device=dev)
    y3 = torch.empty((T, D), dtype=torch.float32, device=dev)
    y5 = torch.empty((T, D), dtype=torch.float32, device=dev)
    # host-resident NF3 table (filled from the first pack, before timing)
    codes_h = torch.empty((V, N, CB), dtype=torch.uint8, pin_memory=True)
    scales_h = torch.empty((V, N, SB), dtype=torch.int16, pin_memory=True)
    st_bytes = mole.mole_nf3_host_staging_size(T, N, D) if nf3 else 16
    stage_h = torch.empty(st_bytes, dtype=torch.uint8, pin_memory=True)
    stage_d = torch.empty(st_bytes, dtype=torch.uint8, device=dev)
    ids_cpu = [torch.from_numpy(x) for x in ids_h]

    ROWS = ["build", "pack_nf3", "combine", "combine_nf3", "combine_nf3_host"]
    n_unique_host = []

    def step(k, evs=None):
        ids, h = batches[k % NB]
        rec = (lambda i: evs[i].record(stream)) if evs is not None else (lambda i: None)
        rec(0)
        mole.mole_build_lut(emb, w_up, w_down, lut, workspace=ws, stream=stream)
        rec(1)
        if nf3:
            mole.mole_pack_nf3(lut, codes, scales, stream=stream)
        rec(2)
        mole.mole_lookup_combine(ids, h, w_r, lut, y, stream=stream)
        rec(3)
        if nf3:
            mole.mole_lookup_combine_nf3(ids, h, w_r, codes, scales, y3, stream=stream)
        rec(4)
        if nf3:
            n_unique_host.append(mole.mole_lookup_combine_nf3_host(
                ids_cpu[k % NB], h, w_r, codes_h, scales_h, stage_h, stage_d, y5, stream=stream))
        rec(5)

    with torch.cuda.stream(stream):
        if args.copy_calibration:
            src_c = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
            dst_c = torch.empty_like(src_c)
            dst_c.copy_(src_c)
            torch.cuda.synchronize()
            del src_c, dst_c
        # fill the host-resident table once
        mole.mole_build_lut(emb, w_up, w_down, lut, workspace=ws, stream=stream)
        if nf3:
            mole.mole_pack_nf3(lut, codes, scales, stream=stream)
            stream.synchronize()
            codes_h.copy_(codes.cpu())
            scales_h.copy_(scales.cpu())
        for k in range(args.warmup):
            step(k)
        torch.cuda.synchronize()

        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t_start.record(stream)
        for k in range(args.steps):
            step(k, evs[k])
        t_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0

    ms_step = t_start.elapsed_time(t_end) / args.steps
    row_ms = {name: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))
              for i, name in enumerate(ROWS)}
    sweep = batch_sweep(torch, mole, synth, w, perm, to_dev, lut, codes if nf3 else None,
                        scales if nf3 else None, w_r, stream)

    # ---------------- per-row algorithmic work
    bL = 2 if bf16 else 4
    bh = bL
    mean_u = float(np.mean(uniq))
    build_flops = 4.0 * V * N * D * F
    pack_bytes = V * N * D * bL + V * N * (CB + 2 * SB)
    comb_bytes = T * (N * D * bL + D * bh + 4 * D + 8) + D * N * bh
    comb_uniq = comb_bytes - (T - mean_u) * N * D * bL
    nf3_row = N * (CB + 2 * SB)
    nf3_bytes = T * (nf3_row + D * bh + 4 * D + 8) + D * N * bh
    host_pcie = float(np.mean(n_unique_host)) * nf3_row + 8 * T if n_unique_host else 0.0

    def rate(bytes_, ms):
        return bytes_ / (ms * 1e-3) / 1e9

    rows = {
        "build": {"ms": row_ms["build"], "tflops": build_flops / (row_ms["build"] * 1e-3) / 1e12,
                  "mfma_frac": build_flops / (row_ms["build"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                  "flops": build_flops},
        "pack_nf3": {"ms": row_ms["pack_nf3"], "gbs": rate(pack_bytes, row_ms["pack_nf3"]),
                     "hbm_frac": rate(pack_bytes, row_ms["pack_nf3"]) / HBM_PEAK_GBS},
        "combine": {"us": row_ms["combine"] * 1e3, "tokens_per_s": T / (row_ms["combine"] * 1e-3),
                    "gbs": rate(comb_bytes, row_ms["combine"]),
                    "hbm_frac": rate(comb_bytes, row_ms["combine"]) / HBM_PEAK_GBS,
                    "gbs_unique": rate(comb_uniq, row_ms["combine"]), "bytes": comb_bytes,
                    "mean_unique_ids": mean_u},
        "combine_nf3": {"us": row_ms["combine_nf3"] * 1e3,
                        "tokens_per_s": T / (row_ms["combine_nf3"] * 1e-3),
                        "gbs": rate(nf3_bytes, row_ms["combine_nf3"]),
                        "hbm_frac": rate(nf3_bytes, row_ms["combine_nf3"]) / HBM_PEAK_GBS},
        "combine_nf3_host": {"us": row_ms["combine_nf3_host"] * 1e3,
                             "tokens_per_s": T / (row_ms["combine_nf3_host"] * 1e-3),
                             "pcie_bytes": host_pcie,
                             "pcie_gbs_effective": rate(host_pcie, row_ms["combine_nf3_host"])
                             if host_pcie else 0.0},
    }

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
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) h, %s ids)"
                % {"zipf": "Zipf(1.1)", "uniform": "uniform", "distinct": "distinct"}[
                    args.ids or ("zipf" if w.zipf else "uniform")],
        "config": {"workload": "%s-class MoLE layer V=%d D=%d N=%d F=%d, T=%d %s ids; step = "
                               "build + NF3 pack + combine + NF3 combine + host-resident NF3 combine"
                               % (w.name, V, D, N, F, T, args.ids or ("Zipf(1.1)" if w.zipf else "uniform")),
                   "V": V, "D": D, "N": N, "F": F, "tokens": T, "parallelism": "single GPU"},
        "rows": rows,
        "roofline": {"kernel": "mole_build_lut (gemm_nt_bf16 GELU + store per vocabulary block)",
                     "bound": "mfma", "achieved": rows["build"]["tflops"], "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": rows["build"]["mfma_frac"],
                     "traffic": measured_traffic(args.workload, ws_bytes) if T == 256 and bf16 else None},
        "roofline_combine": {"kernel": "lookup_combine_kernel", "bound": "hbm",
                             "achieved": rows["combine"]["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": rows["combine"]["hbm_frac"], "traffic": None},
        "wall_s_timed": wall,
        "batch_sweep": sweep,
    }

    probes = set() if args.no_scale_probe or not bf16 else set(args.probes.split(","))
    if probes:
        torch.cuda.synchronize()
    if "scale" in probes:
        result["combine_at_scale"] = scale_probe(torch, mole, synth, dev, stream)
    if "decode" in probes:
        result["decode_stack_1b"] = decode_stack_probe(torch, mole, synth, dev, stream)
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
        result["cpu_baseline"] = cpu_baseline(args, w, layer, ids_h[0], synth, T)

    print(json.dumps(result), flush=True)


def batch_sweep(torch, mole, synth, w, perm, to_dev, lut, codes, scales, w_r, stream):
    """The combine and the NF3 combine on this workload's table at each of
    its batch sizes (Zipf ids): event-timed over 50 launches that cycle
    through 8 id batches, after 5 warm-up launches.  Bytes per launch as for
    the headline combine (gathered rows + h + y + ids + W_r)."""
    V, D, N = w.V, w.D, w.N
    bL = 2 if w.dtype == "bf16" else 4
    out = {}
    for T in sorted(w.tokens):
        ids_l = [to_dev(synth.make_ids(w, T, step=s, perm=perm)) for s in range(8)]
        h_l = [to_dev(synth.make_hidden(w, T, step=s)) for s in range(8)]
        y = torch.empty((T, D), dtype=torch.float32, device=lut.device)
        res = {}
        runs = [("bf16" if bL == 2 else "f32",
                 lambda i: mole.mole_lookup_combine(ids_l[i % 8], h_l[i % 8], w_r, lut, y, stream=stream),
                 N * D * bL)]
        if codes is not None:
            runs.append(("nf3", lambda i: mole.mole_lookup_combine_nf3(ids_l[i % 8], h_l[i % 8], w_r, codes,
                                                                       scales, y, stream=stream),
                         N * (3 * D // 8 + D // 32)))
        for name, fn, row in runs:
            with torch.cuda.stream(stream):
                for i in range(5):
                    fn(i)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                reps = 50
                e0.record(stream)
                for i in range(reps):
                    fn(i)
                e1.record(stream)
                torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            byts = T * (row + D * bL + 4 * D + 8) + D * N * bL
            res[name] = {"us": us, "tokens_per_s": T / (us * 1e-6), "gbs": byts / (us * 1e-6) / 1e9,
                         "hbm_frac": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "bytes": byts}
        out["T%d" % T] = res
    return out


def scale_probe(torch, mole, synth, dev, stream):
    """Combine throughput where one launch moves tens of MB: the 410M-class
    table (50304 x 16 x 1024 bf16 and its NF3, NF4 and int8 forms) at
    T = 1024 and 4096, Zipf ids and a distinct-id control (gathered bytes =
    unique bytes); the bf16 combine also in its grouped form (tokens grouped
    by distinct id on the host, each slab read once per run; the index time
    is reported, outside the timed region); plus the NF4 and int8 encoders
    over the whole table.  Fractions against the nominal 8 TB/s and against a
    device-to-device copy measured in the same run."""
    w = synth.WORKLOADS["410m"]
    V, D, N = w.V, w.D, w.N
    # every input is produced on `stream`, the stream the kernels run on
    ctx = torch.cuda.stream(stream)
    ctx.__enter__()
    g = torch.Generator(device=dev)
    g.manual_seed(synth.seed(w, 60))
    lut = (torch.randn((V, N, D), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    codes = torch.empty((V, N, 3 * D // 8), dtype=torch.uint8, device=dev)
    scales = torch.empty((V, N, D // 64), dtype=torch.int16, device=dev)
    w_r = (torch.randn((N, D), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    mole.mole_pack_nf3(lut, codes, scales, stream=stream)
    # the 4- and 8-bit formats of the same table
    codes4 = torch.empty((V, N, D // 2), dtype=torch.uint8, device=dev)
    scales4 = torch.empty((V, N, D // 64), dtype=torch.int16, device=dev)
    codes8 = torch.empty((V, N, D), dtype=torch.int8, device=dev)
    scales8 = torch.empty((V, N), dtype=torch.float32, device=dev)
    out = {"workload": "410M-class table V=50304 D=1024 N=16 (bf16 %.2f GB, NF3 %.2f GB, NF4 %.2f GB, "
           "int8 %.2f GB)" % (V * N * D * 2 / 1e9, V * N * (3 * D // 8 + D // 32) / 1e9,
                              V * N * (D // 2 + D // 32) / 1e9, V * N * (D + 4) / 1e9)}
    packs = {}
    for name, fn, wbytes in (
            ("nf4", lambda: mole.mole_pack_nf4(lut, codes4, scales4, stream=stream), V * N * (D // 2 + D // 32)),
            ("int8", lambda: mole.mole_pack_int8(lut, codes8, scales8, stream=stream), V * N * (D + 4))):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        byts = V * N * D * 2 + wbytes
        packs[name] = {"ms": ms, "gbs": byts / (ms * 1e-3) / 1e9, "hbm_frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    out["pack"] = packs
    # Measured HBM peak of this part in this run: a 1 GiB device-to-device
    # copy (read + write bytes over its event time), the second roofline the
    # combines are reported against.
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    out["hbm_copy_gbs_measured"] = copy_gbs
    del src, dst
    perm = synth.rank_permutation(w)
    for T in (256, 1024, 4096):
        for kind in ("zipf", "distinct"):
            ids_host = [torch.from_numpy(synth.make_ids(w, T, step=s, kind=kind, perm=perm)) for s in range(8)]
            ids_l = [x.to(dev) for x in ids_host]
            # the grouped form's host index (tokens grouped by distinct id), built before the timed region
            t_idx = time.perf_counter()
            idx = [mole.mole_grouped_index(x, V) for x in ids_host]
            index_us = (time.perf_counter() - t_idx) / len(ids_host) * 1e6
            grp = [(r.to(dev), tk.to(dev)) for (r, tk) in idx]
            h_l = [torch.randn((T, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(8)]
            y = torch.empty((T, D), dtype=torch.float32, device=dev)
            torch.cuda.synchronize()
            res = {}
            for name, fn, row in (
                    ("bf16_grouped", lambda i: mole.mole_lookup_combine_grouped(*grp[i % 8], h_l[i % 8], w_r, lut, y,
                                                                                stream=stream), N * D * 2),
                    ("bf16", lambda i: mole.mole_lookup_combine(ids_l[i % 8], h_l[i % 8], w_r, lut, y,
                                                                stream=stream), N * D * 2),
                    ("nf3", lambda i: mole.mole_lookup_combine_nf3(ids_l[i % 8], h_l[i % 8], w_r, codes,
                                                                   scales, y, stream=stream),
                     N * (3 * D // 8 + D // 32)),
                    ("nf4", lambda i: mole.mole_lookup_combine_nf4(ids_l[i % 8], h_l[i % 8], w_r, codes4,
                                                                   scales4, y, stream=stream),
                     N * (D // 2 + D // 32)),
                    ("int8", lambda i: mole.mole_lookup_combine_int8(ids_l[i % 8], h_l[i % 8], w_r, codes8,
                                                                     scales8, y, stream=stream),
                     N * (D + 4))):
                with torch.cuda.stream(stream):
                    for i in range(5):
                        fn(i)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    reps = 50
                    e0.record(stream)
                    for i in range(reps):
                        fn(i)
                    e1.record(stream)
                    torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / reps
                byts = T * (row + D * 2 + 4 * D + 8) + D * N * 2
                res[name] = {"us": us, "tokens_per_s": T / (us * 1e-6), "gbs": byts / (us * 1e-6) / 1e9,
                             "hbm_frac": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                             "hbm_frac_measured": byts / (us * 1e-6) / 1e9 / copy_gbs, "bytes": byts}
            res["bf16_grouped"]["host_index_us"] = index_us
            res["bf16_grouped"]["mean_unique_ids"] = float(np.mean([torch.unique(r).numel() for (r, _) in idx]))
            out["T%d_%s" % (T, kind)] = res
    torch.cuda.synchronize()
    ctx.__exit__(None, None, None)
    del lut, codes, scales
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


def decode_stack_probe(torch, mole, synth, dev, stream):
    """Decode through the 1B-class stack: 16 layers, each with its own
    50304 x 16 x 2048 bf16 table (3.3 GB, 52.7 GB in all) and router, the
    same token ids at every layer and a fresh hidden state per layer.  One
    step = the 16 lookup-combines; timed eagerly and as one HIP graph
    replay, at T = 1, 16, 128 and 1024 Zipf(1.1) ids."""
    w = synth.WORKLOADS["1b"]
    V, D, N, L = w.V, w.D, w.N, w.layers
    ctx = torch.cuda.stream(stream)
    ctx.__enter__()
    g = torch.Generator(device=dev)
    g.manual_seed(synth.seed(w, 70))
    luts, w_rs = [], []
    for _ in range(L):
        luts.append((torch.randn((V, N, D), generator=g, device=dev) * 0.02).to(torch.bfloat16))
        w_rs.append((torch.randn((N, D), generator=g, device=dev) * 0.02).to(torch.bfloat16))
    perm = synth.rank_permutation(w)
    out = {"workload": "1B-class stack: %d layers x table V=%d N=%d D=%d bf16 (%.1f GB in all)"
           % (L, V, N, D, L * V * N * D * 2 / 1e9)}
    for T in w.tokens:
        NB = 4
        ids_l = [torch.from_numpy(synth.make_ids(w, T, step=s, perm=perm)).to(dev) for s in range(NB)]
        h_l = [[torch.randn((T, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(L)]
               for _ in range(NB)]
        y_l = [torch.empty((T, D), dtype=torch.float32, device=dev) for _ in range(L)]

        def stack(b, st):
            for l in range(L):
                mole.mole_lookup_combine(ids_l[b], h_l[b][l], w_rs[l], luts[l], y_l[l], stream=st)

        torch.cuda.synchronize()
        for b in range(3):
            stack(b % NB, stream)
        reps = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for r in range(reps):
            stack(r % NB, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        eager_us = e0.elapsed_time(e1) * 1e3 / reps
        # the same 16 launches captured once per input batch, replayed
        graphs = []
        for b in range(NB):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                stack(b, torch.cuda.current_stream())
            graphs.append(gr)
        torch.cuda.synchronize()
        for b in range(NB):
            graphs[b].replay()
        torch.cuda.synchronize()
        e0.record()
        for r in range(reps):
            graphs[r % NB].replay()
        e1.record()
        torch.cuda.synchronize()
        graph_us = e0.elapsed_time(e1) * 1e3 / reps
        per_layer = T * (N * D * 2 + D * 2 + 4 * D + 8) + D * N * 2
        best = min(eager_us, graph_us)
        out["T%d" % T] = {"eager_us_per_step": eager_us, "graph_us_per_step": graph_us,
                          "tokens_per_s": T / (best * 1e-6),
                          "gbs": L * per_layer / (best * 1e-6) / 1e9,
                          "hbm_frac": L * per_layer / (best * 1e-6) / 1e9 / HBM_PEAK_GBS,
                          "bytes_per_step": L * per_layer}
        del graphs
    torch.cuda.synchronize()
    ctx.__exit__(None, None, None)
    del luts, w_rs
    torch.cuda.empty_cache()
    return out


def host_stack_probe(torch, mole, synth, dev, stream):
    """A 16-layer stack of 410M-class NF3 tables (V=50304 N=16 D=1024,
    0.33 GB each, 5.3 GB in all) in pinned host memory.  One decode step
    = the 16 layers' lookup-combines, run two ways: (a) per layer, the
    host-resident call (gather + copy + combine, 16 transfers); (b) one
    step-start prefetch of every layer's rows in a single transfer, then 16
    device combines on the staged rows.  Also a pinned host->device copy of
    256 MiB, the PCIe roofline measured in the same run.  The host tables are
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

        res = {}
        for name, fn in (("per_layer", per_layer), ("prefetched", prefetched)):
            for b in range(2):
                fn(b % NB)
            torch.cuda.synchronize()
            reps = 5
            t0 = time.perf_counter()
            e0.record(stream)
            for r in range(reps):
                fn(r % NB)
            e1.record(stream)
            torch.cuda.synchronize()
            wall = (time.perf_counter() - t0) / reps
            res[name + "_us_per_step"] = e0.elapsed_time(e1) * 1e3 / reps
            res[name + "_wall_us_per_step"] = wall * 1e6
        U = float(np.mean(uniq)) if uniq else 0.0
        pcie = L * U * N * (CB + 2 * SB) + 8 * T
        best = min(res["per_layer_us_per_step"], res["prefetched_us_per_step"])
        res.update({"mean_unique_ids": U, "pcie_bytes_per_step": pcie,
                    "pcie_gbs_effective_prefetched": pcie / (res["prefetched_us_per_step"] * 1e-6) / 1e9,
                    "tokens_per_s": T / (best * 1e-6)})
        out["T%d" % T] = res
        del st1_h, st1_d, stL_h, stL_d, h_l, y_l
    torch.cuda.synchronize()
    ctx.__exit__(None, None, None)
    del codes_h, scales_h, w_rs
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


def cpu_baseline(args, w, layer, ids, synth, T):
    """The CPU oracle (plain fp64 C, OpenMP) on this host: the build on a
    sample of vocabulary rows and the NF3 encoder on a sample of table rows,
    both extrapolated linearly to the whole vocabulary, plus the two
    combines on the whole batch.  value = T / (extrapolated step time)."""
    import oracle

    cores = len(os.sched_getaffinity(0))
    budget = args.cpu_seconds
    h = synth.make_hidden(w, T)
    t0 = time.perf_counter()
    nrow = 1
    while True:
        rows = np.arange(nrow, dtype=np.int64) * (w.V // nrow)
        t1 = time.perf_counter()
        lut_rows = oracle.build_lut_rows(layer.emb, layer.w_up, layer.w_down, rows=rows, nthreads=cores)
        dt = time.perf_counter() - t1
        if dt > 0.4 * budget or nrow >= w.V or time.perf_counter() - t0 > 0.6 * budget:
            break
        nrow = min(w.V, nrow * 4)
    build_s = dt * w.V / nrow
    table = synth.f32_to_bf16_bits(lut_rows.astype(np.float32)) if w.dtype == "bf16" else lut_rows.astype(np.float32)
    t1 = time.perf_counter()
    reps = 0
    while True:
        codes, scales, _ = oracle.pack_nf3(table, nthreads=cores) if w.D % 64 == 0 else (None, None, 0)
        reps += 1
        if time.perf_counter() - t1 > 0.5 or reps >= 50:
            break
    pack_s = (time.perf_counter() - t1) / reps * w.V / nrow
    # combine on the whole batch: ids remapped into the sampled rows (same work per token)
    ids_s = (np.asarray(ids) % nrow).astype(np.int64)
    t1 = time.perf_counter()
    oracle.lookup_combine(ids_s, h, layer.w_r, table, nthreads=cores)
    comb_s = time.perf_counter() - t1
    nf3_s = 0.0
    if codes is not None:
        t1 = time.perf_counter()
        oracle.lookup_combine_nf3(ids_s, h, layer.w_r, codes, scales, nthreads=cores)
        nf3_s = time.perf_counter() - t1
    step_s = build_s + pack_s + comb_s + 2 * nf3_s
    per_config = oracle_sweep(oracle, synth, cores)
    return {"value": T / step_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "build on %d of %d vocabulary rows and NF3 pack of those rows, extrapolated "
                      "linearly to V; combine and NF3 combine (counted twice, device and host "
                      "table) on the full batch of %d tokens" % (nrow, w.V, T),
            "build_s_extrapolated": build_s, "pack_s_extrapolated": pack_s,
            "combine_tokens_per_s": T / comb_s, "combine_nf3_tokens_per_s": T / nf3_s if nf3_s else None,
            "per_config": per_config,
            "measured_s": time.perf_counter() - t0}


def oracle_sweep(oracle, synth, cores):
    """The oracle's combine (and NF3 combine on the NF3 workload) at every
    batch size of the 160M-, 410M- and 1B-class workloads (one layer), on all
    host cores and on one core, Zipf ids.  The tables are zero except the
    rows the batch reads (random values there): the oracle touches only
    those rows, and its time does not depend on the values."""
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
                reps, t1 = 0, time.perf_counter()
                while True:
                    fn(nt)
                    reps += 1
                    if time.perf_counter() - t1 > 0.05:
                        break
                r[label + "_tokens_per_s"] = T * reps / (time.perf_counter() - t1)
            res["T%d" % T] = r
        out[key] = res
    return out


if __name__ == "__main__":
    main()
