"""Profiling driver: replay one workload shape through fluxbin_gemv, or run a plain device copy.

Used under rocprofv3 to produce the kernel-trace and counter summaries kept in
profiles/ (each summary names the exact command).  Two modes:

  python3 -m binary_basis_lut_amd.profile_workload gemv --workload 2 --shape 0 --sets 256 --reps 2
      builds `sets` distinct weight sets of the shape (resident in HBM, more
      than the 256 MB Infinity Cache for the q_proj shape), captures one call
      per set in a HIP graph and replays it `reps` times, and prints the time
      per call (HIP events around the replays);  --format blockwise draws the
      shape in the block-wise row-scale storage instead (--kb global and --ks
      salient bases, --sal-group salient columns per 128-column group);

  python3 -m binary_basis_lut_amd.profile_workload decompose --n 4096 --k 4096 --kb 2 --iters 5 --reps 3
      the offline decomposition of one synthetic fp16 matrix (HIP events
      around fluxbin_decompose; no error trace), time per call and per
      iteration;

  python3 -m binary_basis_lut_amd.profile_workload dense --n 11008 --k 4096 --batch 128 --sets 8 --reps 20
      the dense fp16 product y = x W^T of the same shape with torch.matmul
      (the platform GEMM library) over `sets` distinct resident matrices, and,
      for batch <= 16, the library's own dense fp16 GEMV kernel: time per call;

  python3 -m binary_basis_lut_amd.profile_workload copy --bytes 1073741824 --reps 4
      a plain device-to-device copy of known size (torch's copy kernel): the
      reference that scales the FETCH_SIZE / WRITE_SIZE counters to bytes;

  python3 -m binary_basis_lut_amd.profile_workload stream --bytes 1073741824 --reps 10
      the HBM read rate of the GEMV's access pattern (fluxbin_probe_stream_read:
      1 KiB per wave load, non-temporal, each wave a contiguous span) over a
      buffer larger than the 256 MB Infinity Cache, at every in-flight depth and
      a few grid sizes: GB/s per configuration and the best one;

  python3 -m binary_basis_lut_amd.profile_workload empty --workgroups 528 --threads 256 --nodes 256 --reps 20
      the launch floor: a HIP graph of `nodes` empty kernels of the given grid,
      microseconds per node;

  python3 -m binary_basis_lut_amd.profile_workload lookup --iters 2000 --reps 5
      the table-lookup rate alone (fluxbin_probe_lds_lookup) for g = 4 at 1, 2,
      4, 8, 16 batch rows and g = 8 at 1, 2, 4, and of the g = 8 bank-private
      tables (fluxbin_probe_lds_lookup_banked) over 2- and 4-chunk regions:
      lookups per second, per CU per clock (2.4 GHz), and the packed-weight
      GB/s that rate would sustain (one lookup per g bits of one row's
      weights, divided by the batch rows that share them).
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def run_gemv(args) -> None:
    import numpy as np
    import torch

    from binary_basis_lut_amd import accounting as A
    from binary_basis_lut_amd import fluxbin as F
    from binary_basis_lut_amd import inputs as I

    wl = I.WORKLOADS[args.workload]
    sh = wl.shapes[args.shape]
    blockwise = args.format == "blockwise"
    dls, xs, ys = [], [], []
    for i in range(args.sets):
        if blockwise:
            seed = (args.workload, i, 100 + args.sal_group + 1000 * args.shape)
            lay = I.make_grouped_layer(sh.n, sh.k, args.kb, args.ks, wl.g, 128, args.sal_group,
                                       outlier_frac=wl.outlier_frac, seed=seed)
            x = I.make_x(lay, args.batch, seed=seed)
        else:
            lay = I.workload_layer(args.workload, args.shape, i)
            x = I.workload_x(args.workload, lay, args.batch, args.shape, i)
        if args.g:
            lay.g = args.g  # table width is a kernel choice: the packed sign bits do not depend on it
        dls.append(F.DeviceLayer(lay, max_batch=args.batch, chunks_per_block=args.chunks_per_block,
                                 waves_per_block=args.waves_per_block, table_precision=args.table_precision))
        xs.append(torch.from_numpy(x.view(np.int16)).cuda())
        ys.append(torch.empty((args.batch, lay.n), dtype=torch.int16, device="cuda"))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for i in range(args.sets):
            dls[i].gemv(xs[i], ys[i], stream=stream)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            for i in range(args.sets):
                dls[i].gemv(xs[i], ys[i], stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(args.reps):
            graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (args.reps * args.sets)
    lay = dls[0].layer
    wb = (A.grouped_weight_bytes(lay.n, lay.k, lay.kb, lay.ks, 128, args.sal_group) if blockwise
          else A.weight_bytes(lay.n, lay.k, lay.s, lay.kb, lay.ks))
    tables = "fp16 tables" if args.table_precision else "fp32 tables"
    print(f"gemv workload {args.workload} shape {args.shape} ({sh.name} {sh.k}->{sh.n}, {args.format}, {tables}, "
          f"batch {args.batch}): "
          f"{args.sets} sets x {args.reps} replays, {us:.3f} us per call, {wb / us / 1e3:.1f} GB/s of "
          f"{wb} weight-side bytes, plan {dls[0].plan}", flush=True)
    for d in dls:
        d.close()


def run_decompose(args) -> None:
    import numpy as np
    import torch

    from binary_basis_lut_amd import fluxbin as F
    from binary_basis_lut_amd import inputs as I

    n, k, kb, iters = args.n, args.k, args.kb, args.iters
    w = torch.from_numpy(I.decomp_matrix(n, k, seed=(7, n, k)).view(np.int16)).cuda()
    nbytes = F.fluxbin_decomp_workspace_size(n, k, kb)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    wpr = (k + 31) // 32
    bits = torch.empty(kb * n * wpr, dtype=torch.int32, device="cuda")
    r16 = torch.empty(kb * n, dtype=torch.int16, device="cuda")
    c16 = torch.empty(kb * k, dtype=torch.int16, device="cuda")
    r64 = torch.empty(kb * n, dtype=torch.float64, device="cuda")
    c64 = torch.empty(kb * k, dtype=torch.float64, device="cuda")
    trace = torch.empty(2 + iters * (2 * kb + 1), dtype=torch.float64, device="cuda")

    def call(with_trace):
        F.fluxbin_decompose(w, n, k, kb, iters, None, bits, r16, c16, r64, c64, trace if with_trace else None, ws,
                            nbytes)

    call(True)  # warm-up, and the error trace of this matrix
    torch.cuda.synchronize()
    tr = trace.cpu().numpy()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.reps):
        call(False)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.reps
    norm = float((w.view(torch.float16).double() ** 2).sum())
    print(f"decompose {n}x{k} kb={kb} iters={iters}: {ms:.3f} ms per call ({n * k / (ms * 1e-3) / 1e9:.2f} G "
          f"weights/s); relative error init {tr[0] / norm:.5f} -> final {tr[-1] / norm:.5f}", flush=True)


def run_dense(args) -> None:
    import torch

    from binary_basis_lut_amd import fluxbin as F

    n, k, b = args.n, args.k, args.batch
    ws = [torch.randn(n, k, device="cuda").mul_(0.02).half() for _ in range(args.sets)]
    x = torch.randn(b, k, device="cuda").half()
    y = torch.empty(b, n, device="cuda", dtype=torch.float16)

    def time_it(fn):
        for i in range(args.sets):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.reps):
            for i in range(args.sets):
                fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (args.reps * args.sets)

    us_lib = time_it(lambda i: torch.matmul(x, ws[i].t(), out=y))
    line = (f"dense {k}->{n} batch {b}: torch matmul {us_lib:.3f} us per call "
            f"({2 * n * k * b / us_lib / 1e6:.1f} TFLOP/s, {2 * n * k / us_lib / 1e3:.0f} GB/s of weights)")
    if b <= 16:
        xi, yi = x.view(torch.int16), y.view(torch.int16)
        us_own = time_it(lambda i: F.fluxbin_dense_gemv_f16(ws[i].view(torch.int16), n, k, xi, yi, b))
        line += f"; fluxbin_dense_gemv_f16 {us_own:.3f} us per call"
    print(line, flush=True)


def run_copy(args) -> None:
    import torch

    n = args.bytes // 4
    src = torch.ones(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy: {args.reps} x {n * 4} bytes read and written", flush=True)


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def run_stream(args) -> None:
    import torch

    from binary_basis_lut_amd import fluxbin as F

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    buf = torch.ones(args.bytes // 4, dtype=torch.int32, device="cuda")
    best = (0.0, None)
    for wg_per_cu in (4, 8, 16):
        wgs = cus * wg_per_cu
        sink = torch.zeros(wgs * 256, dtype=torch.int32, device="cuda")
        for depth in (1, 2, 4, 8, 16):
            F.fluxbin_probe_stream_read(buf, args.bytes, depth, wgs, 0x9E3779B9, sink)
            torch.cuda.synchronize()
            e0, e1 = _events()
            e0.record()
            for _ in range(args.reps):
                F.fluxbin_probe_stream_read(buf, args.bytes, depth, wgs, 0x9E3779B9, sink)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / args.reps
            gbs = args.bytes / us / 1e3
            print(f"stream read {args.bytes} B, {wgs} workgroups x 4 waves, depth {depth}: {us:.1f} us, "
                  f"{gbs:.0f} GB/s", flush=True)
            if gbs > best[0]:
                best = (gbs, (wgs, depth))
    print(f"stream read best: {best[0]:.0f} GB/s at {best[1][0]} workgroups, depth {best[1][1]} "
          f"({cus} CUs)", flush=True)


def run_empty(args) -> None:
    import torch

    from binary_basis_lut_amd import fluxbin as F

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        F.fluxbin_probe_empty(args.workgroups, args.threads, stream=stream)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            for _ in range(args.nodes):
                F.fluxbin_probe_empty(args.workgroups, args.threads, stream=stream)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = _events()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(args.reps):
            graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (args.reps * args.nodes)
    print(f"empty kernel {args.workgroups} x {args.threads} threads: {us:.3f} us per graph node "
          f"({args.nodes} nodes x {args.reps} replays)", flush=True)


def run_lookup(args) -> None:
    import torch

    from binary_basis_lut_amd import fluxbin as F

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = cus * 8  # 32 waves per CU
    sink = torch.zeros(wgs * 256, dtype=torch.float32, device="cuda")
    for g, nb in ((4, 1), (4, 2), (4, 4), (4, 8), (4, 16), (8, 1), (8, 2), (8, 4)):
        F.fluxbin_probe_lds_lookup(g, nb, wgs, args.iters, -1.0, sink)
        torch.cuda.synchronize()
        e0, e1 = _events()
        e0.record()
        for _ in range(args.reps):
            F.fluxbin_probe_lds_lookup(g, nb, wgs, args.iters, -1.0, sink)
        e1.record()
        torch.cuda.synchronize()
        s = e0.elapsed_time(e1) * 1e-3 / args.reps
        lookups = wgs * 256 * args.iters * nb * 128 // g
        rate = lookups / s
        per_cu_clk = rate / cus / 2.4e9
        # at b = nb the weights of one lookup-set are g bits per row: bytes/s = rate / nb * g / 8
        gbs = rate / nb * g / 8 / 1e9
        print(f"lookups g={g} batch rows={nb}: {rate / 1e12:.3f} T lookups/s, {per_cu_clk:.2f} per CU per clock, "
              f"weight stream it sustains {gbs:.0f} GB/s", flush=True)
    # the g = 8 bank-private tables (one batch row), 8 waves per workgroup, as many workgroups per CU as
    # the GEMV runs (4 with 2-chunk regions, 2 with 4-chunk ones)
    for region, per_cu in ((2, 4), (4, 2)):
        wgs_b = cus * per_cu * 2
        sink_b = torch.zeros(wgs_b * 512, dtype=torch.float32, device="cuda")
        F.fluxbin_probe_lds_lookup_banked(region, wgs_b, args.iters, -1.0, sink_b)
        torch.cuda.synchronize()
        e0, e1 = _events()
        e0.record()
        for _ in range(args.reps):
            F.fluxbin_probe_lds_lookup_banked(region, wgs_b, args.iters, -1.0, sink_b)
        e1.record()
        torch.cuda.synchronize()
        s = e0.elapsed_time(e1) * 1e-3 / args.reps
        rate = wgs_b * 512 * args.iters * 16 * region / s
        print(f"lookups g=8 banked tables, {region}-chunk regions: {rate / 1e12:.3f} T lookups/s, "
              f"{rate / cus / 2.4e9:.2f} per CU per clock, weight stream it sustains {rate / 1e9:.0f} GB/s", flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="mode", required=True)
    g = sub.add_parser("gemv")
    g.add_argument("--workload", type=int, default=2)
    g.add_argument("--shape", type=int, default=0)
    g.add_argument("--sets", type=int, default=256)
    g.add_argument("--reps", type=int, default=2)
    g.add_argument("--batch", type=int, default=1)
    g.add_argument("--chunks-per-block", type=int, default=0)
    g.add_argument("--waves-per-block", type=int, default=0)
    g.add_argument("--table-precision", type=int, default=0, choices=[0, 1], help="0: fp32 tables, 1: fp16")
    g.add_argument("--format", choices=["per-row", "blockwise"], default="per-row")
    g.add_argument("--kb", type=int, default=2, help="blockwise: global bases")
    g.add_argument("--ks", type=int, default=2, help="blockwise: salient bases")
    g.add_argument("--sal-group", type=int, default=8, choices=[8, 16])
    g.add_argument("--g", type=int, default=0, choices=[0, 4, 8], help="table width (0: the workload's)")
    dp = sub.add_parser("decompose")
    dp.add_argument("--n", type=int, default=4096)
    dp.add_argument("--k", type=int, default=4096)
    dp.add_argument("--kb", type=int, default=2)
    dp.add_argument("--iters", type=int, default=5)
    dp.add_argument("--reps", type=int, default=3)
    dn = sub.add_parser("dense")
    dn.add_argument("--n", type=int, default=11008)
    dn.add_argument("--k", type=int, default=4096)
    dn.add_argument("--batch", type=int, default=1)
    dn.add_argument("--sets", type=int, default=8)
    dn.add_argument("--reps", type=int, default=20)
    c = sub.add_parser("copy")
    c.add_argument("--bytes", type=int, default=1 << 30)
    c.add_argument("--reps", type=int, default=4)
    st = sub.add_parser("stream")
    st.add_argument("--bytes", type=int, default=1 << 30)
    st.add_argument("--reps", type=int, default=10)
    em = sub.add_parser("empty")
    em.add_argument("--workgroups", type=int, default=528)
    em.add_argument("--threads", type=int, default=256)
    em.add_argument("--nodes", type=int, default=256)
    em.add_argument("--reps", type=int, default=20)
    lk = sub.add_parser("lookup")
    lk.add_argument("--iters", type=int, default=2000)
    lk.add_argument("--reps", type=int, default=5)
    args = ap.parse_args()
    {"gemv": run_gemv, "decompose": run_decompose, "dense": run_dense, "copy": run_copy, "stream": run_stream,
     "empty": run_empty, "lookup": run_lookup}[args.mode](args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
