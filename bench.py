"""Benchmark of libfairy on one MI355X.

Workload (the metric's configuration): the LLaMA-2-7B attention projection,
a real 4096x4096 layer (N(0, 0.02^2), seed 200) converted on the GPU to the
widely-linear complex form U, W (2048x2048 each), PhaseQuant-quantised with
2 recursive residual stages and packed 16 codes per uint32 (P = 4 planes,
4 MiB).  A step is one decode GEMV of that layer on one batch of bf16
activations (batch 1 by default, N(0,1), seed 201).

Each timed step reads a different copy of the packed weights from a pool of
>= 512 MiB, so the codes really stream from HBM (no L2 / Infinity-Cache
reuse).  `value` is packed-weight GB/s over the timed steps.

Also reported: the roofline of the GEMV kernel (HBM-bound, achieved bytes
per launch over the average launch time from HIP events on the launch
stream), the CPU oracle on a bounded sample of the same workload, and the
other rows of the path (conversion, PhaseQuant, pack, larger batches, the
prefill GEMM) timed the same way.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--batch B]
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
POOL_BYTES = 512 << 20


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-rows", action="store_true", help="skip the per-row timings")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_complex_weight_amd import fairy as F
    from bit_complex_weight_amd import synth

    torch.cuda.set_device(0)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    stream = torch.cuda.current_stream()

    def ev_time(fn, iters):
        """Average ms per call of fn(i) over iters back-to-back calls (HIP events)."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(iters):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    # ---- build the layer on the GPU: conversion -> PhaseQuant -> pack -------
    rows, cols, S = 4096, 4096, 2
    n, m = rows // 2, cols // 2
    P = 2 * S
    log(f"building widely-linear {rows}x{cols} -> {n}x{m}, S={S}")
    R = synth.real_layer(rows, cols, seed=200)
    R_d = dev(R)
    planes = [torch.empty((n, m), dtype=torch.float32, device="cuda") for _ in range(4)]
    F.fairy_real_to_complex(R_d, n, m, *planes)
    count = n * m
    codes = torch.empty((P, n, m), dtype=torch.uint8, device="cuda")
    scales = torch.empty((P, 2), dtype=torch.float32, device="cuda")
    wsb = F.fairy_phasequant_workspace_bytes(count, S)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    F.fairy_phasequant(planes[0], planes[1], count, S, codes[0], scales[0], None, None, ws, wsb)
    F.fairy_phasequant(planes[2], planes[3], count, S, codes[S], scales[S], None, None, ws, wsb)
    nw = F.fairy_packed_words(n, m, P, F.FAIRY_LAYOUT_TILED64)
    packed = torch.empty(nw, dtype=torch.int32, device="cuda")
    F.fairy_pack(codes, P, n, m, F.FAIRY_LAYOUT_TILED64, packed)
    torch.cuda.synchronize()
    packed_bytes = nw * 4

    ncopy = max(2, math.ceil(POOL_BYTES / packed_bytes))
    pool = [packed.clone() for _ in range(ncopy)]
    descs = [F.make_clinear(n, m, S, 1, p, scales) for p in pool]

    B = args.batch
    rb, ib = synth.bf16_gaussian((B, m), seed=201)
    x_re, x_im = dev(rb.view(np.int16)), dev(ib.view(np.int16))
    y_re = torch.empty((B, n), dtype=torch.float32, device="cuda")
    y_im = torch.empty((B, n), dtype=torch.float32, device="cuda")

    def gemv(i):
        F.fairy_cgemv(descs[i % ncopy], x_re, x_im, F.FAIRY_BF16, B, m, y_re, y_im, n)

    # ---- timed region: the K steps are captured once as a HIP graph (K GEMV
    # launches, each on its own weight copy) and replayed, so the host-side
    # launch cost of the Python binding is not part of the measurement.
    for i in range(args.warmup):
        gemv(i)
    torch.cuda.synchronize()
    eager_y = (y_re.clone(), y_im.clone())
    eager_ms = ev_time(gemv, min(args.steps, 200))
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(args.steps):
                gemv(i)
    torch.cuda.synchronize()
    y_re.zero_(); y_im.zero_()
    graph.replay()                                   # untimed warm replay
    torch.cuda.synchronize()
    if not (torch.equal(y_re, eager_y[0]) and torch.equal(y_im, eager_y[1])):
        raise SystemExit("graph replay output differs from the eager GEMV output")
    t0 = time.perf_counter()
    ms = ev_time(lambda i: graph.replay(), 1) / args.steps
    wall = time.perf_counter() - t0
    gbs = packed_bytes / (ms * 1e-3) / 1e9
    alg_bytes = packed_bytes + B * m * 2 * 2 + B * n * 2 * 4
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    log(f"GEMV B={B}: graph {ms * 1e3:.2f} us/launch ({gbs:.0f} GB/s packed), eager {eager_ms * 1e3:.2f} us/call, "
        f"wall {wall:.4f}s for {args.steps}")

    result = {
        "metric": "GB/s & % HBM peak, 2-bit complex GEMV at LLaMA-2-7B shapes; prefill TOPS",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "widely-linear complex GEMV, LLaMA-2-7B attention projection (real 4096x4096 "
                        "sigma=0.02 -> complex 2048x2048 U,W), PhaseQuant 2 residual stages, "
                        f"packed TILED64, bf16 activations, batch {B}",
            "n": n, "m": m, "stages": S, "planes": P, "batch": B,
            "packed_bytes": packed_bytes, "weight_pool_bytes": packed_bytes * ncopy,
            "complex_weights_per_s": P * n * m / (ms * 1e-3),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "k_cgemv_units<bf16>",
            "eager_ms_per_call": eager_ms,
            "alg_bytes_per_launch": alg_bytes,
        },
    }

    # ---- other rows of the path --------------------------------------------------
    if not args.no_rows:
        rows_out = {}
        it = 20
        ms_c = ev_time(lambda i: F.fairy_real_to_complex(R_d, n, m, *planes), it)
        rows_out["real_to_complex"] = {"ms": ms_c, "GB/s": (4 * rows * cols * 2) / (ms_c * 1e-3) / 1e9}
        ms_q = ev_time(lambda i: F.fairy_phasequant(planes[0], planes[1], count, S, codes[0], scales[0], None,
                                                    None, ws, wsb), it)
        rows_out["phasequant_S2_per_matrix"] = {"ms": ms_q, "unique_GB/s": (count * 8) / (ms_q * 1e-3) / 1e9}
        ms_p = ev_time(lambda i: F.fairy_pack(codes, P, n, m, F.FAIRY_LAYOUT_TILED64, packed), it)
        rows_out["pack"] = {"ms": ms_p, "GB/s": (P * count * 1.25) / (ms_p * 1e-3) / 1e9}
        for bb in (4, 16, 64):
            rbb, ibb = synth.bf16_gaussian((bb, m), seed=202)
            xr2, xi2 = dev(rbb.view(np.int16)), dev(ibb.view(np.int16))
            yr2 = torch.empty((bb, n), dtype=torch.float32, device="cuda")
            yi2 = torch.empty((bb, n), dtype=torch.float32, device="cuda")
            f = lambda i: F.fairy_cgemv(descs[i % ncopy], xr2, xi2, F.FAIRY_BF16, bb, m, yr2, yi2, n)
            f(0)
            msb = ev_time(f, 50)
            rows_out[f"gemv_bf16_B{bb}"] = {"ms": msb, "packed_GB/s": packed_bytes / (msb * 1e-3) / 1e9,
                                           "alg_Tadds/s": 2 * P * n * m * bb / (msb * 1e-3) / 1e12}
        xi8r, xi8i = synth.int8_uniform((1, m), seed=203)
        xr8, xi8 = dev(xi8r), dev(xi8i)
        f = lambda i: F.fairy_cgemv(descs[i % ncopy], xr8, xi8, F.FAIRY_I8, 1, m, y_re[:1], y_im[:1], n)
        f(0)
        ms8 = ev_time(f, 200)
        rows_out["gemv_i8_B1"] = {"ms": ms8, "packed_GB/s": packed_bytes / (ms8 * 1e-3) / 1e9}
        Mg = 2048
        rg, ig = synth.bf16_gaussian((Mg, m), seed=204)
        xgr, xgi = dev(rg.view(np.int16)), dev(ig.view(np.int16))
        ygr = torch.empty((Mg, n), dtype=torch.float32, device="cuda")
        ygi = torch.empty((Mg, n), dtype=torch.float32, device="cuda")
        fg = lambda i: F.fairy_cgemm(descs[0], xgr, xgi, F.FAIRY_BF16, Mg, m, ygr, ygi, n, None,
                                     F.FAIRY_ALGO_VALU)
        fg(0)
        msg = ev_time(fg, 3)
        rows_out["gemm_bf16_valu_M2048"] = {"ms": msg, "alg_TOPS": 2 * P * n * m * Mg / (msg * 1e-3) / 1e12}
        result["rows"] = rows_out
        log(json.dumps(rows_out))

    # ---- CPU oracle baseline (bounded sample of the same workload) ---------------
    if not args.no_cpu:
        import oracle
        cores = oracle.set_threads(int(os.environ.get("OMP_NUM_THREADS", "0")) or min(16, os.cpu_count() or 1))
        ur, ui, wr, wi = oracle.real_to_complex(R, n, m, f32=True)
        cu, su, _, _ = oracle.phasequant(ur, ui, S, want_resid=False)
        cw, sw, _, _ = oracle.phasequant(wr, wi, S, want_resid=False)
        oc = np.concatenate([cu, cw]); osc = np.concatenate([su, sw])
        xr, xi = synth.bf16_to_f32(rb), synth.bf16_to_f32(ib)
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.cgemv_dense(oc, osc, S, True, xr, xi)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or reps >= 1000:
                break
        result["cpu_baseline"] = {
            "value": round(packed_bytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{reps} full GEMVs of the same 2048x2048 S=2 widely-linear layer, batch {B}, "
                      f"dense fp64 oracle, {el:.1f}s",
        }

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
