#!/usr/bin/env python3
"""Benchmark of the FluxBin LUT GEMV on one MI355X.

Headline: the LLaMA-2-70B decode stream.  One step = one decoder layer's four
GEMVs at batch 1 (qkv 8192->10240, o 8192->8192, gate+up 8192->57344, down
28672->8192; two global bases, one salient basis on 3 % of the columns, g = 4)
through fluxbin_gemv, on that layer's own weights: the whole hot path (VCM
gather of x[S], scale-fused table build, sign-pattern lookups over every
global and salient basis, row scaling, split reduction, fp16 store) four times.
All 80 layers' packed weights (17.4 GB) are resident in HBM, so every call
streams from HBM, not from the 256 MB Infinity Cache.  The 80 layers are
captured once as a HIP graph (torch.cuda.CUDAGraph); K steps replay it
floor(K / 80) times plus a graph of the first K mod 80 layers.  The timed
region is bracketed by torch.cuda.synchronize() and HIP events on the replay
stream.  `value` = weight-side bytes of the K layers / time.

Layer 0 of every shape is drawn on the host by binary_basis_lut_amd.inputs
(the seeded recipe) and checked against the fp64 oracle in the cpu_baseline
leg; layers 1..79 are timing-only sets of the same shapes and structure whose
sign words and scales are drawn on the device (uniform random words,
fp16(|N(0, 0.02)| + 1e-3) scales, layer 0's salient index).

In the same run, after the timed region: the mean kernel duration of every
GEMV of the stream, from start/stop events that fluxbin_gemv_timed records
at each kernel's own start and end, over an eager pass of the 80 layers (the
gate+up projection is the dominant kernel of the roofline object); the HBM read rate of the GEMV's access pattern
(fluxbin_probe_stream_read, the measured peak); the table-lookup rate
(fluxbin_probe_lds_lookup) that bounds the batch path; the LLaMA-2-7B q_proj
call on 256 resident sets; the LLaMA-2-7B 32-layer g = 8 stream, each GEMV
against the banked lookup rate (fluxbin_probe_lds_lookup_banked); the
4096->11008 / 11008->4096 batch sweep (fp32 tables, and fp16 tables from 4
batch rows); the hand-written dense fp16 GEMV on the 70B shapes; and the fp64
oracle on the host cores (cpu_baseline).

Prints one JSON line.  --out FILE also writes the detail as JSON.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

from binary_basis_lut_amd import rocprof_summary as RS  # noqa: E402  (host-only helpers: hashes, no GPU)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, decimal GB/s
HEADLINE = 5            # LLaMA-2-70B decode layers
N_LAYERS = 80
STREAM_7B = 3           # LLaMA-2-7B layers at g = 8
N_LAYERS_7B = 32
PAGES_A100_US = 41.0    # FluxBin summary, appendix E.4: isolated 4096x4096 2-bit GEMV on A100


def measured_traffic(name: str):
    """HBM bytes per launch from the committed counter summary `name`, if it was taken on this kernel source."""
    f = ROOT / "profiles" / name
    if not f.exists():
        return None, "no counter summary for this kernel"
    try:
        d = json.loads(f.read_text())
    except Exception:
        return None, "unreadable counter summary"
    if d.get("kernel_source_hash") != RS.kernel_source_hash():
        return None, "counters were taken on another kernel source"
    return d.get("hbm_bytes_per_launch"), d.get("note")


class Model:
    """Handles of a streamed model: n_layers x the workload's shapes, every (layer, shape) its own weights."""

    def __init__(self, wid: int, n_layers: int, torch, F, I, A, gen, max_batch: int = 1, shapes=None,
                 table_precision: int = 0):
        self.wl = I.WORKLOADS[wid]
        self.wid = wid
        self.n_layers = n_layers
        self.shape_ids = list(range(len(self.wl.shapes))) if shapes is None else list(shapes)
        self.max_batch = max_batch
        self.table_precision = table_precision
        self.layer0 = [I.workload_layer(wid, si, 0) for si in self.shape_ids]
        self.x0 = [I.workload_x(wid, lay, max_batch, si, 0) for si, lay in zip(self.shape_ids, self.layer0)]
        self.bytes = [A.weight_bytes(l.n, l.k, l.s, l.kb, l.ks) for l in self.layer0]
        self.xs = [torch.from_numpy(x.view(np.int16)).cuda() for x in self.x0]
        self.ys = [torch.empty((max_batch, l.n), dtype=torch.int16, device="cuda") for l in self.layer0]
        self.handles = []   # [layer][shape] -> fluxbin handle
        self.keep = []      # tensors and DeviceLayers the handles point into
        for li in range(n_layers):
            row = []
            for si, lay in enumerate(self.layer0):
                if li == 0:
                    dl = F.DeviceLayer(lay, max_batch=max_batch, table_precision=table_precision)
                    self.keep.append(dl)
                    row.append(dl.handle)
                else:
                    row.append(self._device_filled(torch, F, lay, gen))
            self.handles.append(row)
        torch.cuda.synchronize()

    def _device_filled(self, torch, F, lay, gen):
        """A handle over device-drawn weights of lay's shape and structure (timing only)."""
        def words(count):
            return torch.randint(-2 ** 31, 2 ** 31, (max(count, 4),), dtype=torch.int32, device="cuda",
                                 generator=gen)

        def scales(count):
            v = torch.randn(count, device="cuda", generator=gen).abs_().mul_(0.02).add_(1e-3)
            return v.half().view(torch.int16)

        t = {"bits_g": words(lay.kb * F.fluxbin_tiled_words(lay.n, lay.k)),
             "r_g": scales(lay.kb * lay.n), "c_g": scales(lay.kb * lay.k)}
        if lay.ks:
            t.update(bits_s=words(lay.ks * F.fluxbin_tiled_words(lay.n, lay.s)), r_s=scales(lay.ks * lay.n),
                     c_s=scales(lay.ks * lay.s), idx=torch.from_numpy(lay.sal_idx).cuda())
        d = F.LayerDesc()
        d.abi_version = F.ABI_VERSION
        d.g, d.kb, d.ks = lay.g, lay.kb, lay.ks
        d.n, d.k, d.s, d.max_batch = lay.n, lay.k, lay.s, self.max_batch
        d.layout = F.LAYOUT_TILED
        d.table_precision = self.table_precision
        d.bits_global, d.r_global, d.c_global = (t["bits_g"].data_ptr(), t["r_g"].data_ptr(), t["c_g"].data_ptr())
        if lay.ks:
            d.bits_sal, d.r_sal, d.c_sal, d.sal_idx = (t["bits_s"].data_ptr(), t["r_s"].data_ptr(),
                                                       t["c_s"].data_ptr(), t["idx"].data_ptr())
        ws = F.fluxbin_workspace_size(d)
        if ws:
            t["ws"] = torch.empty(ws, dtype=torch.uint8, device="cuda")
            d.workspace, d.workspace_bytes = t["ws"].data_ptr(), ws
        torch.cuda.synchronize()
        h = F.fluxbin_create(d)
        self.keep.append(t)
        return h

    def launch(self, F, li, si, stream):
        F.fluxbin_gemv(self.handles[li][si], self.xs[si], self.ys[si], self.max_batch, stream=stream)

    def capture(self, torch, F, stream, layers):
        """One graph of `layers` consecutive layers (all shapes)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for li in range(layers):
                    for si in range(len(self.layer0)):
                        self.launch(F, li, si, stream)
        torch.cuda.synchronize()
        return g

    def close(self, F):
        for row in self.handles[1:]:
            for h in row:
                F.fluxbin_destroy(h)
        for k in self.keep:
            if hasattr(k, "close"):
                k.close()


def run_steps(torch, graphs, stream, steps, n_layers):
    """Replay whole-model graphs and one partial graph: exactly `steps` layers."""
    full, part = graphs
    with torch.cuda.stream(stream):
        for _ in range(steps // n_layers):
            full.replay()
        if steps % n_layers:
            part.replay()


def timed(torch, stream, fn):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3  # seconds


def per_gemv_durations(torch, F, model, stream, reps=2):
    """Mean kernel duration of every shape's GEMV over the model's layers: an eager pass over all layers in
    stream order, each call through fluxbin_gemv_timed (HIP events recorded by the kernel launch itself at
    its start and end), `reps` times.  Returns ({shape name: us}, how)."""
    L, S = model.n_layers, len(model.layer0)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(S)]
          for _ in range(L)]
    with torch.cuda.stream(stream):
        for row in ev:
            for e0, e1 in row:
                e0.record(stream)
                e1.record(stream)
    torch.cuda.synchronize()
    acc = np.zeros(S)
    for _ in range(reps):
        with torch.cuda.stream(stream):
            for li in range(L):
                for si in range(S):
                    F.fluxbin_gemv_timed(model.handles[li][si], model.xs[si], model.ys[si], model.max_batch,
                                         ev[li][si][0], ev[li][si][1], stream=stream)
        torch.cuda.synchronize()
        for si in range(S):
            acc[si] += sum(ev[li][si][0].elapsed_time(ev[li][si][1]) for li in range(L)) * 1e3 / L
    how = (f"fluxbin_gemv_timed (start/stop events recorded by the launch itself) on every GEMV of the {L} layers, "
           f"eager, stream order, mean of {reps} passes")
    return {model.wl.shapes[model.shape_ids[si]].name: float(acc[si] / reps) for si in range(S)}, how


def stream_probe(torch, F, nbytes=1 << 30, reps=5):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    best = (0.0, None)
    for wg_per_cu in (8, 16):
        wgs = cus * wg_per_cu
        sink = torch.zeros(wgs * 256, dtype=torch.int32, device="cuda")
        for depth in (4, 8, 16):
            F.fluxbin_probe_stream_read(buf, nbytes, depth, wgs, 0x9E3779B9, sink)
            sec = timed(torch, torch.cuda.current_stream(),
                        lambda: [F.fluxbin_probe_stream_read(buf, nbytes, depth, wgs, 0x9E3779B9, sink)
                                 for _ in range(reps)])
            gbs = nbytes * reps / sec / 1e9
            if gbs > best[0]:
                best = (gbs, {"workgroups": wgs, "depth": depth})
    del buf
    return {"gbs": round(best[0], 1), "bytes": nbytes, **best[1], "cus": cus}


def lookup_probe(torch, F, configs, iters=400, reps=3):
    """Table lookups per second (the GEMV's address, LDS-read and add instructions, weights in registers)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = cus * 8
    sink = torch.zeros(wgs * 256, dtype=torch.float32, device="cuda")
    out = {}
    for g, nb in configs:
        F.fluxbin_probe_lds_lookup(g, nb, wgs, iters, -1.0, sink)
        sec = timed(torch, torch.cuda.current_stream(),
                    lambda: [F.fluxbin_probe_lds_lookup(g, nb, wgs, iters, -1.0, sink) for _ in range(reps)])
        out[(g, nb)] = wgs * 256 * iters * nb * (128 // g) * reps / sec
    return out


def banked_lookup_rate(torch, F, region, iters=400, reps=3):
    """Lookups per second of the g = 8 bank-private tables (the banked GEMV's lookup instructions)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = cus * (4 if region == 2 else 2) * 2
    sink = torch.zeros(wgs * 512, dtype=torch.float32, device="cuda")
    F.fluxbin_probe_lds_lookup_banked(region, wgs, iters, -1.0, sink)
    sec = timed(torch, torch.cuda.current_stream(),
                lambda: [F.fluxbin_probe_lds_lookup_banked(region, wgs, iters, -1.0, sink) for _ in range(reps)])
    return wgs * 512 * iters * 16 * region * reps / sec


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(O, model, ys_gpu, budget_s: float):
    """The fp64 oracle, as it is, on the host cores: layer 0's four GEMVs, repeated for ~budget_s.

    The same calls check the GPU's layer-0 outputs (every 7th row of each shape, the 1e-3 contract)."""
    threads = len(os.sched_getaffinity(0))
    worst, ok = 0.0, True
    for si, (lay, x) in enumerate(zip(model.layer0, model.x0)):
        rows = np.arange(0, lay.n, 7)
        y_ref, mag = O.gemv_dense(lay, x, rows=rows, nthreads=threads)
        err = np.abs(O.half_to_double(ys_gpu[si][:, rows]) - y_ref)
        ok &= bool(np.all(err <= 1e-3 * mag))
        worst = max(worst, float((err / (1e-3 * mag)).max()))
    calls, t0 = 0, time.perf_counter()
    while True:
        for lay, x in zip(model.layer0, model.x0):
            O.gemv_dense(lay, x, nthreads=threads)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per_layer = el / calls
    wb = sum(model.bytes)
    # one thread, for the scaling: one call of the smallest shape (the o projection)
    so = min(range(len(model.layer0)), key=lambda i: model.bytes[i])
    t1 = time.perf_counter()
    O.gemv_dense(model.layer0[so], model.x0[so], nthreads=1)
    t1 = time.perf_counter() - t1
    lo = model.layer0[so]
    return {
        "value": round(wb / per_layer / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{calls} x the four layer-0 GEMVs of the 70B stream (qkv, o, gate+up, down at batch 1; 2 global + "
                  f"1 salient bases; fp64 dense reconstruction row by row, OpenMP over rows), {el:.1f} s: "
                  f"{per_layer * 1e3:.0f} ms per layer; the 80-layer stream would take {80 * per_layer:.0f} s "
                  f"(x80 extrapolated)",
        "cpu_model": cpu_model(),
        "single_thread": {"value": round(model.bytes[so] / t1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                          "sample": f"one {lo.k}->{lo.n} GEMV of layer 0 on one thread, {t1 * 1e3:.0f} ms"},
    }, {"parity_layer0_ok": ok, "parity_layer0_worst_err_over_tol": worst, "rows": "every 7th row of each shape"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=160, help="decoder layers timed (one step = one layer)")
    ap.add_argument("--warmup", type=int, default=80)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle leg (and with it the layer-0 check)")
    ap.add_argument("--headline-only", action="store_true", help="skip the extra measurements")
    ap.add_argument("--out", default=None, help="also write the detail to this JSON file")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported here (the path would shard by "
              "output rows, one GPU's share measured at full shape).", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch
    from binary_basis_lut_amd import accounting as A
    from binary_basis_lut_amd import fluxbin as F
    from binary_basis_lut_amd import inputs as I

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261203)
    detail = {}

    # ---------------------------------------------------------------- headline: the 70B stream
    t_gen = time.perf_counter()
    m70 = Model(HEADLINE, N_LAYERS, torch, F, I, A, gen)
    t_gen = time.perf_counter() - t_gen
    with torch.cuda.stream(stream):  # one eager pass over the stream, then layer 0 again for the oracle check
        for li in list(range(N_LAYERS)) + [0]:
            for si in range(4):
                m70.launch(F, li, si, stream)
    torch.cuda.synchronize()
    ys0 = [y.cpu().numpy().view(np.uint16).copy() for y in m70.ys]
    full = m70.capture(torch, F, stream, N_LAYERS)
    parts = {n: m70.capture(torch, F, stream, n) for n in {args.steps % N_LAYERS, args.warmup % N_LAYERS} - {0}}
    run_steps(torch, (full, parts.get(args.warmup % N_LAYERS)), stream, args.warmup, N_LAYERS)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    sec = timed(torch, stream, lambda: run_steps(torch, (full, parts.get(args.steps % N_LAYERS)), stream,
                                                 args.steps, N_LAYERS))
    wall = time.perf_counter() - wall0
    bytes_per_layer = sum(m70.bytes)
    us_per_layer = sec * 1e6 / args.steps
    value = bytes_per_layer * args.steps / sec / 1e9

    per, how = per_gemv_durations(torch, F, m70, stream)
    names = [s.name for s in m70.wl.shapes]
    per_gemv = {nm: {"us": round(per[nm], 3), "bytes": m70.bytes[i],
                     "gbs": round(m70.bytes[i] / per[nm] / 1e3, 1),
                     "pct_hbm_peak": round(100 * m70.bytes[i] / per[nm] / 1e3 / HBM_PEAK_GBS, 2),
                     "plan": F.fluxbin_get_plan(m70.handles[0][i])} for i, nm in enumerate(names)}
    dom = "gate_up"
    achieved = m70.bytes[names.index(dom)] / per[dom] / 1e3
    peak = stream_probe(torch, F)
    traffic, traffic_note = measured_traffic("lut_gemv_70b_gate_up_counters.json")
    detail["per_gemv_timing"] = how
    detail["stream_probe"] = peak
    detail["generation_s"] = t_gen
    detail["wall_s_timed"] = wall

    # ---------------------------------------------------------------- extra measurements
    extra = {}
    if not args.headline_only:
        # dense fp16 context on the 70B shapes (2 distinct matrices per shape, the larger ones exceed the cache)
        dense = {}
        for i, lay in enumerate(m70.layer0):
            ws = [torch.randn(lay.n, lay.k, device="cuda").mul_(0.02).half().view(torch.int16) for _ in range(2)]
            yd = torch.empty((1, lay.n), dtype=torch.int16, device="cuda")
            xd = m70.xs[i]
            with torch.cuda.stream(stream):
                F.fluxbin_dense_gemv_f16(ws[0], lay.n, lay.k, xd, yd, 1, stream=stream)
            s_ = timed(torch, stream, lambda: [F.fluxbin_dense_gemv_f16(ws[r % 2], lay.n, lay.k, xd, yd, 1,
                                                                        stream=stream) for r in range(8)])
            us = s_ * 1e6 / 8
            dense[names[i]] = {"us": round(us, 2), "bytes": 2 * lay.n * lay.k,
                               "gbs": round(2 * lay.n * lay.k / us / 1e3, 1)}
            del ws
        extra["dense_f16_gemv_70b"] = dense
    if not args.headline_only:
        # LLaMA-2-7B 32-layer stream at g = 8
        m7 = Model(STREAM_7B, N_LAYERS_7B, torch, F, I, A, gen)
        g7 = m7.capture(torch, F, stream, N_LAYERS_7B)
        with torch.cuda.stream(stream):
            g7.replay()
        reps = 10
        s7 = timed(torch, stream, lambda: [g7.replay() for _ in range(reps)])
        per7, _ = per_gemv_durations(torch, F, m7, stream)
        b7 = sum(m7.bytes)
        plans7 = [F.fluxbin_get_plan(m7.handles[0][i]) for i in range(len(m7.wl.shapes))]
        brates = {r: banked_lookup_rate(torch, F, r) for r in sorted({p["banked_tables"] for p in plans7}) if r}

        def lookup_floor_us(i):
            lay, r = m7.layer0[i], plans7[i]["banked_tables"]
            return A.lookups(lay.n, lay.k, lay.s, lay.kb, lay.ks, lay.g, 1) / brates[r] * 1e6 if r else None
        extra["llama2_7b_g8_stream"] = {
            "workload": m7.wl.name, "layers": N_LAYERS_7B, "bytes_per_layer": b7,
            "us_per_layer": round(s7 * 1e6 / (reps * N_LAYERS_7B), 3),
            "gbs": round(b7 * reps * N_LAYERS_7B / s7 / 1e9, 1),
            "pct_hbm_peak": round(100 * b7 * reps * N_LAYERS_7B / s7 / 1e9 / HBM_PEAK_GBS, 2),
            "per_gemv": {s.name: {"us": round(per7[s.name], 3), "gbs": round(m7.bytes[i] / per7[s.name] / 1e3, 1),
                                  "lookup_roofline_us": round(lookup_floor_us(i), 3),
                                  "frac_of_lookup_roofline": round(lookup_floor_us(i) / per7[s.name], 4),
                                  "plan": plans7[i]}
                         for i, s in enumerate(m7.wl.shapes)},
            "banked_lookup_rate_per_s": {f"region{r}": v for r, v in brates.items()},
        }
        m7.close(F)
        del m7, g7
        # LLaMA-2-7B q_proj, 256 resident sets (the isolated-kernel shape of the pages' appendix E.4)
        mq = Model(2, 256, torch, F, I, A, gen)
        gq = mq.capture(torch, F, stream, 256)
        with torch.cuda.stream(stream):
            gq.replay()
        sq = timed(torch, stream, lambda: [gq.replay() for _ in range(4)])
        us_q = sq * 1e6 / (4 * 256)
        extra["llama2_7b_q_proj"] = {"workload": mq.wl.name, "sets": 256, "us_per_gemv": round(us_q, 3),
                                     "bytes": mq.bytes[0], "gbs": round(mq.bytes[0] / us_q / 1e3, 1),
                                     "pct_hbm_peak": round(100 * mq.bytes[0] / us_q / 1e3 / HBM_PEAK_GBS, 2),
                                     "plan": F.fluxbin_get_plan(mq.handles[0][0]),
                                     "pages_a100_context_us": PAGES_A100_US}
        mq.close(F)
        del mq, gq
        # batch sweep 4096 -> 11008 and 11008 -> 4096 against the lookup-rate roofline: 48 sets per call
        # (layer 0 drawn on the host, 47 device-drawn; 550 MB, beyond the Infinity Cache)
        rates = lookup_probe(torch, F, [(4, 1), (4, 4), (4, 8), (4, 16)])
        sweep = {}
        for si, sh in enumerate(I.WORKLOADS[4].shapes):
            for b in (1, 4, 8, 16):
                mb = Model(4, 48, torch, F, I, A, gen, max_batch=b, shapes=[si])
                g = mb.capture(torch, F, stream, 48)
                with torch.cuda.stream(stream):
                    g.replay()
                s_ = timed(torch, stream, lambda: [g.replay() for _ in range(4)])
                us = s_ * 1e6 / (4 * 48)
                lay, wb = mb.layer0[0], mb.bytes[0]
                lk = A.lookups(lay.n, lay.k, lay.s, lay.kb, lay.ks, lay.g, b)
                floor_us = lk / rates[(4, b)] * 1e6
                sweep[f"{sh.name}_b{b}"] = {"us": round(us, 3), "gbs": round(wb / us / 1e3, 1),
                                            "pct_hbm_peak": round(100 * wb / us / 1e3 / HBM_PEAK_GBS, 2),
                                            "lookups": lk, "lookup_roofline_us": round(floor_us, 3),
                                            "frac_of_lookup_roofline": round(floor_us / us, 4),
                                            "plan": F.fluxbin_get_plan(mb.handles[0][0])}
                mb.close(F)
                del mb, g
        # the same calls with fp16 tables (quantised entries, two batch rows per table dword)
        sweep16 = {}
        for si, sh in enumerate(I.WORKLOADS[4].shapes):
            for b in (4, 8, 16):
                mb = Model(4, 48, torch, F, I, A, gen, max_batch=b, shapes=[si], table_precision=F.TABLE_F16)
                g = mb.capture(torch, F, stream, 48)
                with torch.cuda.stream(stream):
                    g.replay()
                s_ = timed(torch, stream, lambda: [g.replay() for _ in range(4)])
                us = s_ * 1e6 / (4 * 48)
                sweep16[f"{sh.name}_b{b}"] = {"us": round(us, 3),
                                              "vs_fp32_tables": round(sweep[f"{sh.name}_b{b}"]["us"] / us, 3)}
                mb.close(F)
                del mb, g
        extra["batch_sweep_4096_11008"] = {"lookup_rate_per_s": {f"g{g}_b{nb}": r for (g, nb), r in rates.items()},
                                          "calls": sweep, "sets": 48, "fp16_tables": sweep16}

    cpu = None
    if not args.no_cpu:
        from oracle import oracle as O
        cpu, check = cpu_baseline(O, m70, ys0, args.cpu_seconds)
        detail.update(check)
    m70.close(F)

    line = {
        "metric": "packed-weight GB/s (LUT GEMV decode stream: weight-side bytes / time)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3 / args.steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{m70.wl.name}_stream_{N_LAYERS}_layers",
            "step": "one decoder layer: qkv, o, gate+up, down GEMVs at batch 1 on that layer's own packed weights",
            "layers_resident": N_LAYERS,
            "bytes_per_step": bytes_per_layer,
            "us_per_layer": round(us_per_layer, 3),
            "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "launch": f"hip graph of {N_LAYERS} layers (4 GEMV launches each) replayed {args.steps // N_LAYERS} times"
                      + (f", then a graph of the first {args.steps % N_LAYERS} layers" if args.steps % N_LAYERS else ""),
            "per_gemv": per_gemv,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "lut_gemv_kernel on the 70B gate+up projection (8192 -> 57344), the dominant kernel",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "measured_peak": peak["gbs"],
            "frac_of_measured_peak": round(achieved / peak["gbs"], 4),
        },
        "cpu_baseline": cpu,
    }
    if extra:
        line["config"]["extra"] = extra
    print(json.dumps(line), flush=True)
    detail.update(line)
    detail["traffic_note"] = traffic_note
    detail["kernel_source_hash"] = RS.kernel_source_hash()
    if args.out:
        Path(args.out).parent.mkdir(parents=True, exist_ok=True)
        Path(args.out).write_text(json.dumps(detail, indent=1, default=str))
    ok = detail.get("parity_layer0_ok", True)
    return 0 if ok else 3


if __name__ == "__main__":
    sys.exit(main())
