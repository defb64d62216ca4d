#!/usr/bin/env python3
"""Benchmark of the blockwise-scaled FP8 GEMM hot path on one MI355X.

Workload: the N = K = 4096 sweep over M in {1, 8, 9, 16, 24, 32, 64, 128, 160, 192, 224,
256, 512, 1024, 2048, 4096, 8192} (the M sweep of page "lmdeploy/pull/4830", section
"Performance"). Inputs are seeded synthetic data with the distributions of the vLLM
test on page "prhub.com.cn ... vllm/pull/49932": fp32 activations U(-448, 448) and
e4m3 weights (U(-448, 448) clamped and cast) with 128x128 float32 block scales
U(0, 1e-2).

One step = for every M of the sweep: quantize the activations per 1x128 group
(bfp8_quant_act) and run the blockwise GEMM (bfp8_gemm), i.e. one pass of the whole
hot path per M. `value` is the sweep's total GEMM FLOPs (2 M N K summed over M)
divided by the measured time per step (quantization included), in TFLOP/s.

Cold mode (default) rotates among copies of the weights totalling more than twice
the 256 MB last-level cache, so every GEMM reads its weights from HBM; warm mode
reuses one copy (the pages' "identical preallocated inputs").

Also reported (same JSON line):
  * roofline: the dominant kernel (the M = 8192 GEMM) against the dense FP8 matrix
    peak, timed with HIP events around its launches on the launch stream;
  * per_m: per-shape GEMM latency (p50 of 5 replays of a captured HIP graph of
    back-to-back launches, so host launch cost is excluded), TFLOP/s and the fraction
    of the HBM (M <= 256) or FP8 (M >= 512) roofline, plus the quantizer's GB/s;
  * cpu_baseline: the CPU oracle on a bounded sample of the same sweep;
  * per_m[...]["ue8m0"]: the same GEMM with power-of-two (UE8M0) scales, which the
    hardware-scaled MFMA applies (bfp8_gemm_ue8m0; not part of the step).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 matrix throughput
N = K = 4096
SWEEP_M = (1, 8, 9, 16, 24, 32, 64, 128, 160, 192, 224, 256, 512, 1024, 2048, 4096, 8192)
DOMINANT_M = 8192
LLC_BYTES = 256 * 2**20
KERNEL_SOURCES = ["gemm_tiled.hip", "device_common.h"]  # the dominant GEMM's device code (kernel and helpers)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def gemm_alg_bytes(m: int, n: int = N, k: int = K) -> int:
    """A + As + B + Bs + C, each touched once."""
    kb = k // 128
    return n * k + (-(-n // 128)) * kb * 4 + m * k + m * kb * 4 + 2 * m * n


def quant_alg_bytes(m: int, k: int = K, in_bytes: int = 4) -> int:
    return m * k * in_bytes + m * k + m * (k // 128) * 4


RIDGE_FLOP_PER_BYTE = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)


def roofline_entry(us: float, flops: float, alg_bytes: float) -> dict:
    """Time, rates and the fraction of the roofline that bounds this shape (HBM below the ridge)."""
    tflops = flops / (us * 1e-6) / 1e12
    gbs = alg_bytes / (us * 1e-6) / 1e9
    hbm = flops / alg_bytes < RIDGE_FLOP_PER_BYTE
    return {"us": round(us, 2), "tflops": round(tflops, 1), "alg_gbs": round(gbs, 1), "bound": "hbm" if hbm else "mfma",
            "frac": round(gbs / PEAK_HBM_GBS if hbm else tflops / PEAK_FP8_TFLOPS, 4)}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_scaled_fp8_bfp8_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(rows_cap: int = 8192):
    """The oracle on the sweep (every M, first min(M, rows_cap) rows; the default cap keeps all
    rows, about 10-15 s of float64 BLAS on 16 host threads)."""
    import numpy as np

    import workloads
    from oracle import gemm as ogemm
    from oracle import quant as oquant

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = os.cpu_count() or 1
    w = workloads.square_weight()
    bq, bs = w.q.numpy(), w.s.numpy()
    flops = 0.0
    t0 = time.perf_counter()
    for m in SWEEP_M:
        rows = min(m, rows_cap)
        x = workloads.square_act(m)[:rows].numpy()
        q, s = oquant.quant_act_ref(x)
        ogemm.gemm_ref(q, s, bq, bs)
        flops += 2.0 * rows * N * K
    dt = time.perf_counter() - t0
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"the whole N=K=4096 sweep" if rows_cap >= max(SWEEP_M) else
                   f"N=K=4096 sweep, every M with rows capped at {rows_cap}")
                  + f" ({flops / 1e9:.0f} GFLOP, quantization included), float64 numpy/BLAS, {dt:.1f} s",
        "cpu": platform.processor() or platform.machine(),
        "affinity_cores": len(os.sched_getaffinity(0)),
    }


def measure_ceilings(torch, np, dev, stream, graph_time_us) -> dict:
    """Ceilings measured on this device in this run (libbfp8_probes.so):
      * fp8_mfma_loop_tflops: 256 workgroups of 8 waves (the 256x256 GEMM's occupancy, 2 waves per SIMD)
        issuing independent 16x16x128 FP8 MFMAs from registers; fp8_mfma_promote_tflops: the same
        with the four promotion FMAs per MFMA of the float-scale method; fp8_mfma32_loop_tflops and
        fp8_mfma32_promote_tflops: the 32x32x64 MFMA (one 1x64 group) accumulating, or promoted
        with sixteen FMAs per MFMA as the 1x64 method does;
      * hbm_read_1gib_gbs: one launch streaming 1 GiB (4x the last-level cache);
      * hbm_read_16mib_cold_us: one launch streaming 16 MiB (the N = K = 4096 weight) that is not in
        the last-level cache (40 buffers read in turn), the floor of a small-M GEMM launch;
      * l2_to_lds_copy_gbs: 256 workgroups copying L2-resident rows into LDS with the direct-to-LDS
        loads the GEMMs stage their operands with (8 rows x 128 bytes per copy, 8 per wave in flight)."""
    from block_scaled_fp8_bfp8_amd import _native

    pr = _native.probes()
    wgs, iters = 256, 2000
    out = torch.empty(wgs * 512, dtype=torch.float32, device=dev)
    res = {}
    # each launch runs about half a millisecond: timed one by one with events on the launch stream
    for mode, key in ((0, "fp8_mfma_loop_tflops"), (1, "fp8_mfma_promote_tflops"), (2, "fp8_mfma_zero_c_tflops")):
        times = []
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if pr.bfp8_probe_mfma_loop(out.data_ptr(), wgs, iters, mode, stream.cuda_stream):
                raise RuntimeError("mfma probe launch failed")
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        us = float(np.median(times[1:]))
        res[key] = round(pr.bfp8_probe_mfma_loop_flops(wgs, iters) / (us * 1e-6) / 1e12, 1)
    for mode, key in ((0, "fp8_mfma32_loop_tflops"), (1, "fp8_mfma32_promote_tflops")):
        times = []
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if pr.bfp8_probe_mfma32_loop(out.data_ptr(), wgs, iters // 2, mode, stream.cuda_stream):
                raise RuntimeError("mfma32 probe launch failed")
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        us = float(np.median(times[1:]))
        res[key] = round(pr.bfp8_probe_mfma32_loop_flops(wgs, iters // 2) / (us * 1e-6) / 1e12, 1)
    sink = torch.empty(2048 * 512, dtype=torch.int32, device=dev)
    big = torch.zeros(2**30 // 4, dtype=torch.int32, device=dev)

    def read_big(n):
        for _ in range(n):
            if pr.bfp8_probe_stream_read(big.data_ptr(), 2**30, sink.data_ptr(), 2048,
                                         torch.cuda.current_stream(dev).cuda_stream):
                raise RuntimeError("read probe launch failed")
    res["hbm_read_1gib_gbs"] = round(2**30 / (graph_time_us(read_big, 2) * 1e-6) / 1e9, 1)
    del big
    small = [torch.zeros(2**24 // 4, dtype=torch.int32, device=dev) for _ in range(40)]

    def read_small(n):
        for j in range(n):
            if pr.bfp8_probe_stream_read(small[j % len(small)].data_ptr(), 2**24, sink.data_ptr(), 1024,
                                         torch.cuda.current_stream(dev).cuda_stream):
                raise RuntimeError("read probe launch failed")
    us16 = graph_time_us(read_small, 40)
    res["hbm_read_16mib_cold_us"] = round(us16, 2)
    res["hbm_read_16mib_cold_gbs"] = round(2**24 / (us16 * 1e-6) / 1e9, 1)
    del small
    # direct-to-LDS copies (the GEMMs' operand path) of 8 rows x 128 bytes, 8 per wave in flight,
    # from a 2 MiB window that stays in the L2 caches
    win = torch.zeros(2**21, dtype=torch.uint8, device=dev)
    times = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if pr.bfp8_probe_copy_lds(win.data_ptr(), 64, 1024, 8, 1, sink.data_ptr(), 256, stream.cuda_stream):
            raise RuntimeError("copy probe launch failed")
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    res["l2_to_lds_copy_gbs"] = round(256 * 8 * 1024 * 1024 / (float(np.median(times[1:])) * 1e-6) / 1e9, 1)
    del win
    torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--mode", choices=["cold", "warm"], default="cold")
    ap.add_argument("--no-table", action="store_true", help="skip the per-M latency table")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-m", type=int, default=0, help="profile helper: run only this M (steps of GEMM+quant)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the transformer-linear and MoE grouped-GEMM configurations")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 256 MiB device copy (for counter calibration under rocprofv3)")
    ap.add_argument("--only-config", choices=["transformer_linear", "moe_grouped", "moe_chain", "gemm_1x64"], default=None,
                    help="profile helper: run only this configuration (no sweep, no table)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured MFMA-loop and HBM-read ceilings")
    ap.add_argument("--ceilings-only", action="store_true", help="profile helper: only the ceiling probes")
    ap.add_argument("--schedule", choices=["auto", "small_m", "tiled", "persistent"], default="auto",
                    help="profile helper: force one GEMM schedule")
    args = ap.parse_args()

    if args.gpus != 1:
        log(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the library has no multi-GPU path; "
            "run with --gpus 1.")
        return 2
    if os.environ.get("WORLD_SIZE", "1") not in ("", "1"):
        log("bench.py runs as a single process on one GPU")
        return 2

    import numpy as np
    import torch

    import block_scaled_fp8_bfp8_amd as bfp8
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bfp8.set_schedule(args.schedule)
    stream = torch.cuda.current_stream(dev)
    sweep = (args.only_m,) if args.only_m else () if args.only_config or args.ceilings_only else SWEEP_M

    # ---- inputs, resident in HBM before any timing -------------------------------------
    w = workloads.square_weight()
    copies = 1 if args.mode == "warm" else max(2, -(-2 * LLC_BYTES // (N * K)) + 1)
    bq = [w.q.to(dev) for _ in range(copies)]
    bsc = [w.s.to(dev) for _ in range(copies)]
    xs = {m: workloads.square_act(m).to(dev) for m in sweep}
    qs = {m: torch.empty((m, K), dtype=torch.uint8, device=dev) for m in sweep}
    ss = {m: torch.empty((K // 128, m), dtype=torch.float32, device=dev).t() for m in sweep}
    cs = {m: torch.empty((m, N), dtype=torch.bfloat16, device=dev) for m in sweep}
    torch.cuda.synchronize()
    log(f"inputs ready: {copies} weight copies ({copies * N * K / 2**20:.0f} MiB), mode={args.mode}")

    rot = [0]

    if args.copy_calibration:
        src = torch.ones(256 * 2**20 // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 256 MiB device-to-device copy done")

    # One step: quantize + GEMM for every M of the sweep. Everything but the dominant GEMM is
    # replayed from a captured HIP graph (host launch cost would otherwise dominate the
    # microsecond-scale small-M kernels); the dominant GEMM is launched directly with HIP
    # events around it on the same stream, which times that kernel inside the timed region.
    def graph_part():
        for j, m in enumerate(sweep):
            bfp8.quant_act(xs[m], q=qs[m], scales=ss[m])
            if m != DOMINANT_M:
                i = j % copies
                bfp8.gemm(qs[m], ss[m], bq[i], bsc[i], out=cs[m])

    capture_stream = torch.cuda.Stream(dev)
    step_graph = torch.cuda.CUDAGraph()
    if sweep:
        with torch.cuda.stream(capture_stream):
            graph_part()
            capture_stream.synchronize()
            with torch.cuda.graph(step_graph, stream=capture_stream):
                graph_part()
    torch.cuda.synchronize()

    def step(dom_events=None):
        if sweep:
            step_graph.replay()
        if DOMINANT_M in sweep:
            i = rot[0] % copies
            rot[0] += 1
            if dom_events is not None:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                bfp8.gemm(qs[DOMINANT_M], ss[DOMINANT_M], bq[i], bsc[i], out=cs[DOMINANT_M])
                e1.record(stream)
                dom_events.append((e0, e1))
            else:
                bfp8.gemm(qs[DOMINANT_M], ss[DOMINANT_M], bq[i], bsc[i], out=cs[DOMINANT_M])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    dom_events = []
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        step(dom_events)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / max(args.steps, 1)
    flops_per_step = sum(2.0 * m * N * K for m in sweep)
    value = flops_per_step / (ms_per_step * 1e-3) / 1e12
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step, {value:.1f} TFLOP/s (quantization included)")

    roofline = None
    if dom_events:
        dom_ms = float(np.mean([a.elapsed_time(b) for a, b in dom_events]))
        achieved = 2.0 * DOMINANT_M * N * K / (dom_ms * 1e-3) / 1e12
        traffic = None
        if os.path.exists(TRAFFIC_FILE):
            with open(TRAFFIC_FILE) as f:
                tr = json.load(f)
            if tr.get("source_hash") == kernel_source_hash() and tr.get("m") == DOMINANT_M:
                traffic = tr.get("bytes_per_launch")
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
                    "kernel": f"bfp8_gemm M={DOMINANT_M} N={N} K={K} schedule={bfp8.schedule_for(DOMINANT_M, N, K)}",
                    "avg_launch_us": round(dom_ms * 1e3, 2), "launches": len(dom_events)}

    # ---- per-M table: back-to-back launches replayed from a captured HIP graph (so host-side
    # launch cost is not measured), p50 of 5 trials; cold mode cycles the weight copies ----
    graph_stream = torch.cuda.Stream(dev)

    def graph_time_us(fn, calls: int) -> float:
        """Median per-call time of `calls` back-to-back calls of fn, captured once and replayed."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(graph_stream):
            fn(calls)  # warm the code paths on the capture stream
            graph_stream.synchronize()
            with torch.cuda.graph(g, stream=graph_stream):
                fn(calls)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        trials = []
        for _ in range(5):
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            trials.append(e0.elapsed_time(e1) * 1e3 / calls)
        del g
        return float(np.median(trials))

    per_m = {}
    if not args.no_table and sweep:

        w8 = workloads.weight_ue8m0(N, K, seed=1)  # the same e4m3 codes as the sweep's weight
        if not torch.equal(w8.q, w.q):
            raise RuntimeError("the UE8M0 weight must share the sweep weight's codes")
        be8 = bfp8.ue8m0_scales(w8.s.to(dev))
        for m in sweep:
            q8, e8 = bfp8.quant_act_ue8m0(xs[m])
            c8 = torch.empty_like(cs[m])

            def gemm8_calls(n):
                for j in range(n):
                    bfp8.gemm_ue8m0(q8, e8, bq[j % copies], be8, out=c8)

            def gemm_calls(n):
                for j in range(n):
                    i = j % copies
                    bfp8.gemm(qs[m], ss[m], bq[i], bsc[i], out=cs[m])

            def quant_calls(n):
                for _ in range(n):
                    bfp8.quant_act(xs[m], q=qs[m], scales=ss[m])

            # back-to-back calls per replay (independent of the copies, so warm mode times
            # launches, not the replay of a one-call graph)
            calls = 33 if m <= 2048 else 8
            res = {"gemm": graph_time_us(gemm_calls, calls), "quant": graph_time_us(quant_calls, min(calls, 32)),
                   "gemm_ue8m0": graph_time_us(gemm8_calls, calls)}
            us = res["gemm"]
            tflops = 2.0 * m * N * K / (us * 1e-6) / 1e12
            gbs = gemm_alg_bytes(m) / (us * 1e-6) / 1e9
            hbm_bound = m <= 256
            frac = gbs / PEAK_HBM_GBS if hbm_bound else tflops / PEAK_FP8_TFLOPS
            qgbs = quant_alg_bytes(m) / (res["quant"] * 1e-6) / 1e9
            per_m[str(m)] = {"gemm_us": round(us, 2), "tflops": round(tflops, 1), "alg_gbs": round(gbs, 1),
                             "bound": "hbm" if hbm_bound else "mfma", "frac": round(frac, 4),
                             "schedule": bfp8.schedule_for(m, N, K), "quant_us": round(res["quant"], 2),
                             "quant_gbs": round(qgbs, 1),
                             "ue8m0": roofline_entry(res["gemm_ue8m0"], 2.0 * m * N * K,
                                                     gemm_alg_bytes(m) - m * (K // 128) * 3 - (N // 128) * (K // 128) * 3)}
            log(f"M={m:5d}  gemm {us:8.2f} us  {tflops:8.1f} TFLOP/s  {gbs:7.1f} GB/s  "
                f"{'HBM' if hbm_bound else 'FP8'} frac {frac:.3f}  [{per_m[str(m)]['schedule']}]   "
                f"quant {res['quant']:7.2f} us {qgbs:7.1f} GB/s   ue8m0 gemm {res['gemm_ue8m0']:8.2f} us")

    # ---- the other workload configurations (not part of the step): the FP8 linear layer on the
    # hidden-5120 transformer shapes, and the M-grouped contiguous MoE GEMM ----
    configs = {}
    want = ((lambda name: args.only_config in (None, name)) if not args.no_configs and not args.only_m and not args.ceilings_only
            else (lambda name: False))
    if want("transformer_linear") or want("moe_grouped") or want("moe_chain") or want("gemm_1x64"):
        del bq, bsc  # the sweep's weight copies
        torch.cuda.empty_cache()
    if want("transformer_linear"):
        lin = {}
        for layer, (n_l, k_l) in workloads.TRANSFORMER_LAYERS.items():
            wl = workloads.transformer_weight(layer)
            n_copies = max(1, min(6, -(-2 * LLC_BYTES // (n_l * k_l)) + 1))
            wq_l = [wl.q.to(dev) for _ in range(n_copies)]
            ws_l = [wl.s.to(dev) for _ in range(n_copies)]
            lin[layer] = {}
            for m in workloads.TRANSFORMER_M:
                x_l = workloads.transformer_act(layer, m).to(dev)
                o_l = torch.empty((m, n_l), dtype=torch.bfloat16, device=dev)
                wsp = torch.empty(bfp8.linear_workspace_bytes(m, n_l, k_l), dtype=torch.uint8, device=dev)

                def lin_calls(n, x_l=x_l, o_l=o_l, wsp=wsp, wq_l=wq_l, ws_l=ws_l):
                    for j in range(n):
                        bfp8.linear(x_l, wq_l[j % len(wq_l)], ws_l[j % len(wq_l)], out=o_l, workspace=wsp)

                us = graph_time_us(lin_calls, 2 * n_copies if m < 2048 else n_copies)
                kb_l = k_l // 128
                alg = 2 * m * k_l + n_l * k_l + (-(-n_l // 128)) * kb_l * 4 + 2 * m * n_l
                lin[layer][str(m)] = {"n": n_l, "k": k_l, "one_launch": bfp8.linear_fuses(m, n_l, k_l),
                                      **roofline_entry(us, 2.0 * m * n_l * k_l, alg)}
                log(f"linear {layer:8s} M={m:5d} N={n_l} K={k_l}: {us:8.2f} us  {lin[layer][str(m)]['tflops']:8.1f} "
                    f"TFLOP/s  {lin[layer][str(m)]['bound']} frac {lin[layer][str(m)]['frac']:.3f}")
            del wq_l, ws_l
            torch.cuda.empty_cache()
        configs["transformer_linear"] = {"what": "bfp8_linear (bf16 x quantized per 1x128 group, blockwise FP8 GEMM, "
                                                 "bf16 out), graph replay of back-to-back calls",
                                         "layers": lin}
    if want("moe_grouped"):
        case = workloads.moe_case()
        bq_g = torch.stack([w_.q for w_ in case.weights]).to(dev)
        bs_g = torch.stack([w_.s for w_ in case.weights]).to(dev)
        q_g, s_g = bfp8.quant_act(case.act.to(dev))
        lay_g = case.layout.to(dev)
        out_g = torch.empty((case.layout.numel(), workloads.MOE_N), dtype=torch.bfloat16, device=dev)

        def grouped_calls(n):
            for _ in range(n):
                bfp8.grouped_gemm_contiguous(q_g, s_g, bq_g, bs_g, lay_g, out=out_g)

        us = graph_time_us(grouped_calls, 4)
        m_real = int(case.counts.sum())
        m_pad = case.layout.numel()
        g_n, g_k, g_g = workloads.MOE_N, workloads.MOE_K, workloads.MOE_GROUPS
        alg = m_pad * g_k + m_pad * (g_k // 128) * 4 + g_g * (g_n * g_k + (g_n // 128) * (g_k // 128) * 4) + 2 * m_real * g_n
        configs["moe_grouped"] = {"groups": g_g, "n": g_n, "k": g_k, "tokens": m_real, "padded_rows": m_pad,
                                  "flops": "2 * tokens * N * K (padding rows not counted)",
                                  **roofline_entry(us, 2.0 * m_real * g_n * g_k, alg)}
        log(f"grouped MoE G={g_g} N={g_n} K={g_k} tokens={m_real} (padded {m_pad}): {us:8.2f} us  "
            f"{configs['moe_grouped']['tflops']:8.1f} TFLOP/s  {configs['moe_grouped']['bound']} "
            f"frac {configs['moe_grouped']['frac']:.3f}")
        del bq_g, bs_g
        torch.cuda.empty_cache()

    if want("gemm_1x64"):
        # 1x64 activation groups / 128x64 weight blocks on the sweep's N = K = 4096 (the same
        # weight codes with 128x64 scales), cold weights
        g64 = {}
        w64 = workloads.weight_1x64(N, K, seed=1)
        n_copies = max(2, -(-2 * LLC_BYTES // (N * K)) + 1)
        wq64 = [w64.q.to(dev) for _ in range(n_copies)]
        ws64 = [w64.s.to(dev) for _ in range(n_copies)]
        for m in (1, 16, 256, 2048, 8192):
            q64, s64 = bfp8.quant_act_1x64(workloads.square_act(m).to(dev))
            c64 = torch.empty((m, N), dtype=torch.bfloat16, device=dev)

            def g64_calls(n, q64=q64, s64=s64, c64=c64):
                for j in range(n):
                    bfp8.gemm_1x64(q64, s64, wq64[j % n_copies], ws64[j % n_copies], out=c64)

            us = graph_time_us(g64_calls, 33 if m <= 2048 else 8)
            alg = m * K + 4 * m * (K // 64) + N * K + 4 * (N // 128) * (K // 64) + 2 * m * N
            g64[str(m)] = roofline_entry(us, 2.0 * m * N * K, alg)
            log(f"gemm_1x64 M={m:5d}: {us:8.2f} us  {g64[str(m)]['tflops']:8.1f} TFLOP/s  {g64[str(m)]['bound']} "
                f"frac {g64[str(m)]['frac']:.3f}")
        configs["gemm_1x64"] = {"what": "bfp8_gemm_1x64 (1x64 activation groups, 128x64 weight blocks), N = K = 4096, "
                                        "graph replay of back-to-back calls, cold weights", "per_m": g64}
        del wq64, ws64
        torch.cuda.empty_cache()

    if want("moe_chain"):
        # MoE expert chain: 512 tokens, top-8 of 16 experts (4096 pairs, like the grouped
        # configuration), hidden 7168, intermediate 2048 (gate+up weights [16, 4096, 7168]).
        t_c, k_c, e_c, h_c, i_c = 512, 8, 16, 7168, 2048
        ids_c, w_c = workloads.moe_routing(t_c, k_c, e_c, seed=31)
        wts_c = [a.to(dev) for a in workloads.moe_experts(e_c, h_c, i_c, seed=32)]
        x_c = workloads.act_normal_bf16(t_c, h_c, seed=33).to(dev)
        ids_d, w_d = ids_c.to(dev), w_c.to(dev)
        y_c = torch.empty((t_c, h_c), dtype=torch.bfloat16, device=dev)
        ws_c = torch.empty(bfp8.moe_forward_workspace_bytes(t_c, k_c, e_c, h_c, i_c), dtype=torch.uint8, device=dev)

        def chain_calls(n):
            for _ in range(n):
                bfp8.moe_forward(x_c, ids_d, w_d, *wts_c, out=y_c, workspace=ws_c)

        us = graph_time_us(chain_calls, 3)
        # the steps one by one, for the breakdown
        rop, por, lay, _ = bfp8.moe_dispatch(ids_d, e_c)
        q_c, s_c = bfp8.quant_act_scatter(x_c, rop, k_c, lay.numel())  # each token once, scales at its rows
        proj_c = bfp8.grouped_gemm_gathered(q_c, s_c, wts_c[0], wts_c[1], lay, por, k_c)
        q2_c, s2_c = bfp8.swiglu_quant(proj_c, lay)
        out_c = bfp8.grouped_gemm_contiguous(q2_c, s2_c, wts_c[2], wts_c[3], lay)
        steps = {
            "dispatch": graph_time_us(lambda n: [bfp8.moe_dispatch(ids_d, e_c) for _ in range(n)], 8),
            "quant_tokens": graph_time_us(lambda n: [bfp8.quant_act_scatter(x_c, rop, k_c, lay.numel())
                                                     for _ in range(n)], 8),
            "grouped_up": graph_time_us(lambda n: [bfp8.grouped_gemm_gathered(q_c, s_c, wts_c[0], wts_c[1], lay, por,
                                                                              k_c, out=proj_c) for _ in range(n)], 3),
            "swiglu_quant": graph_time_us(lambda n: [bfp8.swiglu_quant(proj_c, lay) for _ in range(n)], 8),
            "grouped_down": graph_time_us(lambda n: [bfp8.grouped_gemm_contiguous(q2_c, s2_c, wts_c[2], wts_c[3], lay,
                                                                                  out=out_c) for _ in range(n)], 3),
            "combine": graph_time_us(lambda n: [bfp8.moe_combine(out_c, rop, w_d) for _ in range(n)], 8),
        }
        pairs = int(((ids_c >= 0) & (ids_c < e_c)).sum())
        flops = 2.0 * pairs * (2 * i_c * h_c + h_c * i_c)
        wbytes = e_c * (2 * i_c * h_c + h_c * i_c) + 4 * e_c * ((2 * i_c // 128) * (h_c // 128) + (h_c // 128) * (i_c // 128))
        alg = wbytes + 2 * t_c * h_c * 2 + 8 * t_c * k_c
        configs["moe_chain"] = {"tokens": t_c, "top_k": k_c, "experts": e_c, "hidden": h_c, "intermediate": i_c,
                                "flops": "2 * pairs * (2I*H + H*I)", **roofline_entry(us, flops, alg),
                                "steps_us": {k_: round(v_, 2) for k_, v_ in steps.items()}}
        log(f"MoE chain T={t_c} top{k_c} of E={e_c} H={h_c} I={i_c}: {us:8.2f} us  "
            f"{configs['moe_chain']['tflops']:8.1f} TFLOP/s  {configs['moe_chain']['bound']} "
            f"frac {configs['moe_chain']['frac']:.3f}  steps " + ", ".join(f"{k_} {v_:.1f}" for k_, v_ in steps.items()))
        del wts_c, ws_c, proj_c, out_c, q_c, q2_c
        torch.cuda.empty_cache()

    ceilings = None
    if args.ceilings_only or (not args.no_ceilings and not args.only_m and not args.only_config):
        ceilings = measure_ceilings(torch, np, dev, stream, graph_time_us)
        log("ceilings: " + json.dumps(ceilings))
        if roofline is not None:
            roofline["peak_measured"] = ceilings["fp8_mfma_loop_tflops"]
            roofline["frac_measured"] = round(roofline["achieved"] / ceilings["fp8_mfma_loop_tflops"], 4)
        for m_, e_ in per_m.items():
            if e_["bound"] == "hbm":  # against one launch streaming the weight's 16 MiB from HBM
                e_["frac_measured"] = round(ceilings["hbm_read_16mib_cold_us"] / e_["gemm_us"], 4)
            else:
                e_["frac_measured"] = round(e_["tflops"] / ceilings["fp8_mfma_loop_tflops"], 4)
        if "gemm_1x64" in configs:
            # against the 32x32x64 products alone, and with the 16 promotion FMAs each takes
            for e_ in configs["gemm_1x64"]["per_m"].values():
                if e_["bound"] == "mfma":
                    e_["frac_measured"] = round(e_["tflops"] / ceilings["fp8_mfma32_loop_tflops"], 4)
                    e_["frac_promote_ceiling"] = round(e_["tflops"] / ceilings["fp8_mfma32_promote_tflops"], 4)

    cpu = None
    if not args.no_cpu_baseline and not args.only_m and not args.only_config and not args.ceilings_only:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline()
        log(f"cpu baseline: {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads")

    out = {
        "metric": "blocked-FP8 GEMM µs + TFLOP/s, N=K=4096, M=1..8192; % HBM/MFMA roofline",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic (seeded; fp32 activations U(-448,448), e4m3 weights, 128x128 fp32 scales U(0,1e-2))",
        "config": {"workload": "blockwise FP8 GEMM sweep N=K=4096, M in {1..8192}; per-1x128 activation "
                               "quantization + GEMM per M",
                   "n": N, "k": K, "m": list(sweep), "mode": args.mode, "weight_copies": copies},
        "roofline": roofline,
        "ceilings": ceilings,
        "cpu_baseline": cpu,
        "per_m": per_m,
        "configs": configs,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(out, ensure_ascii=False), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
