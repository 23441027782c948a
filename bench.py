#!/usr/bin/env python3
"""Benchmark of the FluxBin LUT GEMV on one MI355X.

One step = one fluxbin_gemv call (the whole hot path: VCM gather of x[S],
scale-fused table build, sign-pattern lookups over every global and salient
basis, row scaling, reduction, fp16 store) over one synthetic activation
vector, on the LLaMA-2-7B q_proj shape (K = N = 4096, two global bases, one
salient basis on 256 columns, g = 4, batch 1).

To measure HBM and not the 256 MB Infinity Cache, R distinct weight sets
(R * 4.37 MB > 1 GiB) are resident in HBM and step i uses set i mod R.  The
R calls are captured once in a HIP graph (torch.cuda.CUDAGraph) and the graph
is replayed; the timed region is bracketed by torch.cuda.synchronize() and
HIP events recorded on the replay stream.

--format blockwise measures the same shape in the pages' block-wise row-scale
storage instead (one fp16 row scale per row per basis per 128-column group,
two global and two salient bases, --sal-group salient columns per group:
about 2.63 bits per weight at 8, 2.75 at 16; FluxBin summary, appendix C.2).

Prints one JSON line.  --out FILE also writes the extra figures (per-call timings, plan) as JSON.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, decimal GB/s
WORKLOAD_ID = 2
PAGES_A100_US = 41.0    # FluxBin summary, appendix E.4: isolated 4096x4096 2-bit GEMV on A100


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in ["binary_basis_lut_amd/csrc/common.hpp", "binary_basis_lut_amd/csrc/gemv_kernel.hpp",
              "binary_basis_lut_amd/csrc/fluxbin.hip"]:
        h.update((ROOT / p).read_bytes())
    return h.hexdigest()[:16]


def measured_traffic(name: str):
    """HBM bytes per launch from the committed counter summary `name`, if it was taken on this kernel source."""
    f = ROOT / "profiles" / name
    if not f.exists():
        return None, "no counter summary for this workload"
    try:
        d = json.loads(f.read_text())
    except Exception:
        return None, None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None, "counters were taken on another kernel source"
    return d.get("hbm_bytes_per_launch"), d.get("note")


def cpu_baseline(layer, x, budget_s: float, wb: int):
    """Time the fp64 oracle (as it is) on the host cores: whole q_proj GEMVs of one weight set
    (wb = the call's weight-side bytes)."""
    from oracle import oracle as O
    threads = len(os.sched_getaffinity(0))
    O.gemv_dense(layer, x, nthreads=threads)  # warm caches and thread pool
    calls, t0 = 0, time.perf_counter()
    while True:
        O.gemv_dense(layer, x, nthreads=threads)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per_call = el / calls
    fmt = "block-wise row scales" if getattr(layer, "row_group", 0) else "per-row scales"
    return {
        "value": round(wb / per_call / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{calls} full 4096x4096 q_proj GEMVs ({layer.kb} global + {layer.ks} salient bases, {fmt}, fp64 dense "
                  f"reconstruction row by row, OpenMP over rows), {el:.1f} s; {per_call * 1e3:.2f} ms per call",
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4096)
    ap.add_argument("--warmup", type=int, default=512)
    ap.add_argument("--sets", type=int, default=256, help="distinct resident weight sets (cache busting)")
    ap.add_argument("--chunks-per-block", type=int, default=0)
    ap.add_argument("--no-graph", action="store_true", help="launch every call from Python instead")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--format", choices=["per-row", "blockwise"], default="per-row",
                    help="row-scale storage: per row per basis (default), or per row per 128-column group")
    ap.add_argument("--sal-group", type=int, default=8, choices=[8, 16],
                    help="blockwise: salient columns per 128-column group")
    ap.add_argument("--out", default=None, help="also write the extra figures to this JSON file")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(one GPU's share of a layer is measured; the path would shard by output rows).", file=sys.stderr)
        return 2

    import torch
    from binary_basis_lut_amd import accounting as A
    from binary_basis_lut_amd import fluxbin as F
    from binary_basis_lut_amd import inputs as I

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    wl = I.WORKLOADS[WORKLOAD_ID]
    sh = wl.shapes[0]
    blockwise = args.format == "blockwise"
    kb, ks = (2, 2) if blockwise else (wl.kb, wl.ks)

    def make(i):
        if blockwise:
            lay = I.make_grouped_layer(sh.n, sh.k, kb, ks, wl.g, 128, args.sal_group, outlier_frac=wl.outlier_frac,
                                       seed=(WORKLOAD_ID, i, 100 + args.sal_group))
            return lay, I.make_x(lay, 1, seed=(WORKLOAD_ID, i, 100 + args.sal_group))
        lay = I.workload_layer(WORKLOAD_ID, 0, i)
        return lay, I.workload_x(WORKLOAD_ID, lay, 1, 0, i)

    R = max(1, args.sets)
    steps = max(R, int(math.ceil(args.steps / R)) * R)
    warm = max(R, int(math.ceil(args.warmup / R)) * R)

    t_gen = time.perf_counter()
    layers, dls, xs, ys = [], [], [], []
    for i in range(R):
        lay, x_np = make(i)
        dl = F.DeviceLayer(lay, max_batch=1, chunks_per_block=args.chunks_per_block)
        dls.append(dl)
        xs.append(torch.from_numpy(x_np.view(np.int16)).cuda())
        ys.append(torch.empty((1, sh.n), dtype=torch.int16, device="cuda"))
        if i == 0:
            layers.append((lay, x_np))
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    plan = dls[0].plan
    lay0, x0 = layers[0]
    bytes_per_gemv = (A.grouped_weight_bytes(sh.n, sh.k, kb, ks, 128, args.sal_group) if blockwise
                      else A.weight_bytes(sh.n, sh.k, lay0.s, wl.kb, wl.ks))
    act_bytes = A.activation_bytes(sh.n, sh.k, 1)

    # parity spot check of the timed configuration (set 0) against the oracle
    from oracle import oracle as O
    dls[0].gemv(xs[0], ys[0])
    torch.cuda.synchronize()
    y16 = ys[0].cpu().numpy().view(np.uint16)
    rows = np.arange(0, sh.n, 7)
    y_ref, mag = O.gemv_dense(lay0, x0, rows=rows)
    err = np.abs(O.half_to_double(y16[:, rows]) - y_ref)
    parity_ok = bool(np.all(err <= 1e-3 * mag))
    parity_ratio = float((err / (1e-3 * mag)).max())

    stream = torch.cuda.Stream()
    use_graph = not args.no_graph
    graph = None
    if use_graph:
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            for i in range(R):  # one eager pass before capture
                dls[i].gemv(xs[i], ys[i], stream=stream)
        stream.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                for i in range(R):
                    dls[i].gemv(xs[i], ys[i], stream=stream)
        torch.cuda.synchronize()

    def run(n_steps):
        if use_graph:
            for _ in range(n_steps // R):
                graph.replay()
        else:
            with torch.cuda.stream(stream):
                for s in range(n_steps):
                    dls[s % R].gemv(xs[s % R], ys[s % R], stream=stream)

    with torch.cuda.stream(stream):
        run(warm)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        run(steps)
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1)
    us_per_gemv = ms * 1e3 / steps
    gbs = bytes_per_gemv / (us_per_gemv * 1e-6) / 1e9

    # dense fp16 context kernel on the same shape (R distinct matrices would need 8.6 GB; 32 are 1 GiB)
    Rd = 32
    wd = [torch.randn(sh.n, sh.k, device="cuda").to(torch.float16).view(torch.int16) for _ in range(Rd)]
    yd = torch.empty((1, sh.n), dtype=torch.int16, device="cuda")
    with torch.cuda.stream(stream):
        for i in range(Rd):
            F.fluxbin_dense_gemv_f16(wd[i], sh.n, sh.k, xs[0], yd, 1, stream=stream)
        stream.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for rep in range(8):
            for i in range(Rd):
                F.fluxbin_dense_gemv_f16(wd[i], sh.n, sh.k, xs[0], yd, 1, stream=stream)
        d1.record(stream)
    torch.cuda.synchronize()
    dense_us = d0.elapsed_time(d1) * 1e3 / (8 * Rd)
    del wd

    traffic, traffic_note = measured_traffic(f"lut_gemv_q_proj_4096_blockwise_s{args.sal_group}_counters.json"
                                             if blockwise else "lut_gemv_q_proj_4096_counters.json")
    cpu = None if args.no_cpu else cpu_baseline(lay0, x0, args.cpu_seconds, bytes_per_gemv)

    line = {
        "metric": "packed-weight GB/s (LUT GEMV, weight-side bytes per call / time per call)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(ms / steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"llama2_7b_q_proj_4096x4096_kb2_ks2_g128_s{args.sal_group}_g4" if blockwise else wl.name),
            "row_scales": "per 128-column group" if blockwise else "per row",
            "k": sh.k, "n": sh.n, "kb": kb, "ks": ks, "s": lay0.s, "g": wl.g, "batch": 1,
            "weight_sets_resident": R,
            "bytes_per_gemv": bytes_per_gemv,
            "us_per_gemv": round(us_per_gemv, 4),
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "launch": "hip graph of %d calls" % R if use_graph else "python loop",
            "plan": plan,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)

    detail = dict(line)
    detail.update({
        "wall_s_timed": wall, "gen_s": t_gen, "parity_ok_set0": parity_ok, "parity_worst_ratio_set0": parity_ratio,
        "activation_bytes_per_gemv": act_bytes,
        "dense_f16_context": {"us_per_gemv": dense_us, "bytes": A.dense_f16_bytes(sh.n, sh.k),
                              "gbs": A.dense_f16_bytes(sh.n, sh.k) / (dense_us * 1e-6) / 1e9},
        "pages_a100_context_us": PAGES_A100_US,
        "traffic_note": traffic_note,
        "kernel_source_hash": kernel_source_hash(),
    })
    if args.out:
        Path(args.out).parent.mkdir(parents=True, exist_ok=True)
        Path(args.out).write_text(json.dumps(detail, indent=1))
    for d in dls:
        d.close()
    return 0 if parity_ok else 3


if __name__ == "__main__":
    sys.exit(main())
