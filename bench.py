"""Benchmark of libfairy on one MI355X.

Workload (the metric's configuration): the LLaMA-2-7B attention projection,
a real 4096x4096 layer (N(0, 0.02^2), seed 200) converted on the GPU to the
widely-linear complex form U, W (2048x2048 each), PhaseQuant-quantised with
2 recursive residual stages and packed 16 codes per uint32 (P = 4 planes,
4 MiB).  A step is one decode GEMV of that layer on one batch of bf16
activations (batch 1 by default, N(0,1), seed 201).

Each timed step reads a different copy of the packed weights from a pool of
>= 512 MiB.  A timed run is exactly K steps captured as one HIP graph
between two event record nodes (the graph's first and last node) and
replayed once untimed; 512 MiB are then read by another kernel, so that
neither the L2 nor the 256 MB Infinity Cache holds any weight copy, and the
time between the two event nodes of the next replay is the run's time (HIP
events around a whole replay add a fixed ~10 us per graph launch, reported
beside it).  There are
max(5, pool copies / K) such runs, over consecutive windows of the pool, and
`ms_per_step` is their median; the Python binding's launch cost is not
measured.  `value` is packed-weight GB/s at that time per step.

Also reported: the roofline of the GEMV kernel (HBM-bound: algorithmic bytes
per launch over that time), the CPU oracle on a bounded sample of the same
workload (all host cores and one core), and the other rows of the path
(conversion, PhaseQuant, pack, the MLP shapes, larger batches, the prefill
GEMM on the matrix cores and on the VALUs).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--batch B] [--sweep]
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
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "i8": 5000.0}   # dense
# plain (non-packed) VALU lane-operations per second: 256 CUs x 4 SIMDs x 16
# lanes x 2.4 GHz; one fp32 add per lane per clock per SIMD lane slot
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
GEMV_KERNEL = "k_cgemv_lp<bf16,P=4,BCH=1> (one row per wave, lane-fixed planes)"
# HBM bytes per launch of GEMV_KERNEL on this workload, from the FETCH_SIZE and
# WRITE_SIZE counters scaled by a plain copy's (profiles/gemv_lp_bf16_2048x2048_S2_B1.md);
# None whenever the kernel has changed since those counters were taken
GEMV_TRAFFIC_BYTES = 4364288
# SQ_ACTIVE_INST_VALU x 4 cycles / 1024 SIMDs over the kernel's traced
# duration at the nominal 2.4 GHz, from the same profile; None whenever the
# kernel has changed since
GEMV_VALU_BUSY = 0.39
POOL_BYTES = 512 << 20


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Bench:
    def __init__(self):
        import torch
        from bit_complex_weight_amd import fairy as F
        from bit_complex_weight_amd import synth
        self.torch, self.F, self.synth = torch, F, synth
        torch.cuda.set_device(0)
        self.stream = torch.cuda.current_stream()

    def dev(self, a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return self.torch.from_numpy(a).cuda()

    def ev_time(self, fn, iters):
        """Average ms per call of fn(i) over iters back-to-back calls (HIP events
        on the launch stream)."""
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(self.stream)
        for i in range(iters):
            fn(i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    def graph_time(self, fn, steps):
        """Capture `steps` calls fn(i) as one HIP graph, replay once untimed,
        then time one replay; returns (ms per call, graph)."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(steps):
                    fn(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ms = self.ev_time(lambda i: g.replay(), 1) / steps
        return ms, g

    def hip(self):
        """HIP runtime entry points for graphs with timestamp nodes, taken from
        the runtime torch itself loaded (the process keeps one HIP runtime)."""
        if getattr(self, "_hip", None) is None:
            import ctypes
            h = ctypes.CDLL(os.path.join(os.path.dirname(self.torch.__file__), "lib", "libamdhip64.so"))
            h.hipGetErrorString.restype = ctypes.c_char_p
            self._hip = (h, ctypes)
        return self._hip

    def timed_graph(self, fn, steps, stream):
        """Capture fn(j), j < steps, on `stream` into a HIP graph with an event
        record node before its first node and one after its last, so the
        time between the two events is exactly the captured launches (HIP
        events around a whole graph launch also count a fixed ~10 us that
        every graph launch costs, whatever its kernels).  Returns
        (graph exec, event before, event after, cleanup)."""
        torch = self.torch
        h, c = self.hip()
        P = c.c_void_p

        def ck(rc, what):
            if rc != 0:
                raise SystemExit(f"{what} failed: {h.hipGetErrorString(rc).decode()}")

        sp = P(stream.cuda_stream)
        e0, e1 = P(), P()
        ck(h.hipEventCreate(c.byref(e0)), "hipEventCreate")
        ck(h.hipEventCreate(c.byref(e1)), "hipEventCreate")
        ck(h.hipStreamBeginCapture(sp, 0), "hipStreamBeginCapture")
        with torch.cuda.stream(stream):
            for j in range(steps):
                fn(j)
        g = P()
        ck(h.hipStreamEndCapture(sp, c.byref(g)), "hipStreamEndCapture")
        n = c.c_size_t(0)
        ck(h.hipGraphGetNodes(g, None, c.byref(n)), "hipGraphGetNodes")
        nodes = (P * n.value)()
        ck(h.hipGraphGetNodes(g, nodes, c.byref(n)), "hipGraphGetNodes")
        nr = c.c_size_t(0)
        ck(h.hipGraphGetRootNodes(g, None, c.byref(nr)), "hipGraphGetRootNodes")
        roots = (P * nr.value)()
        ck(h.hipGraphGetRootNodes(g, roots, c.byref(nr)), "hipGraphGetRootNodes")
        leaves = []
        for i in range(n.value):
            nd = c.c_size_t(0)
            ck(h.hipGraphNodeGetDependentNodes(P(nodes[i]), None, c.byref(nd)), "hipGraphNodeGetDependentNodes")
            if nd.value == 0:
                leaves.append(nodes[i])
        n0, n1 = P(), P()
        ck(h.hipGraphAddEventRecordNode(c.byref(n0), g, None, c.c_size_t(0), e0), "hipGraphAddEventRecordNode")
        for r in roots:
            ck(h.hipGraphAddDependencies(g, c.byref(n0), c.byref(P(r)), c.c_size_t(1)), "hipGraphAddDependencies")
        la = (P * len(leaves))(*leaves)
        ck(h.hipGraphAddEventRecordNode(c.byref(n1), g, la, c.c_size_t(len(leaves)), e1), "hipGraphAddEventRecordNode")
        ge = P()
        ck(h.hipGraphInstantiate(c.byref(ge), g, None, None, c.c_size_t(0)), "hipGraphInstantiate")

        def launch():
            ck(h.hipGraphLaunch(ge, sp), "hipGraphLaunch")

        def elapsed_ms():
            ms = c.c_float()
            ck(h.hipEventElapsedTime(c.byref(ms), e0, e1), "hipEventElapsedTime")
            return ms.value

        def cleanup():
            h.hipGraphExecDestroy(ge)
            h.hipGraphDestroy(g)
            h.hipEventDestroy(e0)
            h.hipEventDestroy(e1)

        return launch, elapsed_ms, cleanup

    def graph_ms(self, fn, steps):
        """ms per call of fn(i) over `steps` calls captured as one HIP graph,
        timed between the graph's event nodes on a replay after one untimed
        replay (launch overhead of the Python binding excluded)."""
        st = self.torch.cuda.Stream()
        launch, elapsed_ms, cleanup = self.timed_graph(fn, steps, st)
        launch()
        launch()
        st.synchronize()
        ms = elapsed_ms() / steps
        cleanup()
        return ms

    def cold_runs(self, make_fn, steps, ncopy, flush):
        """Timed runs of exactly `steps` launches each, every run on cold
        weights.  Run r captures the launches make_fn(r*steps + j) (j <
        steps; copy (r*steps + j) % ncopy) as a HIP graph between two event
        record nodes, replays it once untimed, reads `flush` (>= 512 MiB,
        read only) so that neither the L2 nor the Infinity Cache holds any
        weight copy, then replays it again: the time between its two event
        nodes is the run's time.  max(5, ncopy/steps) runs, so the timed runs
        touch every copy of the pool.  Returns (median ms per launch, [ms per
        launch of each run], distinct copies read in the timed runs, median
        ms per launch timed around the whole graph launch)."""
        torch = self.torch
        runs = max(5, math.ceil(ncopy / steps))
        sink = torch.empty((flush.shape[0],), dtype=torch.float32, device="cuda")
        st = torch.cuda.Stream()
        per, outer, touched = [], [], set()
        for r in range(runs):
            base = r * steps
            launch, elapsed_ms, cleanup = self.timed_graph(lambda j: make_fn(base + j), steps, st)
            launch()
            with torch.cuda.stream(st):
                torch.sum(flush, dim=1, out=sink)
            o0 = torch.cuda.Event(enable_timing=True)
            o1 = torch.cuda.Event(enable_timing=True)
            o0.record(st)
            launch()
            o1.record(st)
            st.synchronize()
            per.append(elapsed_ms() / steps)
            outer.append(o0.elapsed_time(o1) / steps)
            touched.update((base + j) % ncopy for j in range(steps))
            cleanup()
        torch.cuda.synchronize()
        return float(np.median(per)), per, len(touched), float(np.median(outer))

    def widely_linear_layer(self, rows, cols, S, seed):
        """Real [rows][cols] N(0, 0.02^2) -> U, W -> S stages -> TILED64, all on the GPU."""
        torch, F = self.torch, self.F
        n, m = rows // 2, cols // 2
        P = 2 * S
        R = self.dev(self.synth.real_layer(rows, cols, seed))
        planes = [torch.empty((n, m), dtype=torch.float32, device="cuda") for _ in range(4)]
        F.fairy_real_to_complex(R, n, m, *planes)
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
        return dict(R=R, planes=planes, codes=codes, scales=scales, ws=ws, wsb=wsb, packed=packed,
                    n=n, m=m, S=S, P=P, count=count, packed_bytes=nw * 4)

    def pool(self, L, has_conj=1):
        ncopy = max(2, math.ceil(POOL_BYTES / L["packed_bytes"]))
        copies = [L["packed"].clone() for _ in range(ncopy)]
        descs = [self.F.make_clinear(L["n"], L["m"], L["S"], has_conj, p, L["scales"]) for p in copies]
        return copies, descs

    def gemv_rate(self, L, descs, B, xdtype, steps=200, seed=202):
        torch, F = self.torch, self.F
        n, m = L["n"], L["m"]
        if xdtype == F.FAIRY_I8:
            xr, xi = self.synth.int8_uniform((B, m), seed)
        else:
            xr, xi = self.synth.bf16_gaussian((B, m), seed)
        xr, xi = self.dev(xr), self.dev(xi)
        yr = torch.empty((B, n), dtype=torch.float32, device="cuda")
        yi = torch.empty((B, n), dtype=torch.float32, device="cuda")
        f = lambda i: F.fairy_cgemv(descs[i % len(descs)], xr, xi, xdtype, B, m, yr, yi, n)
        f(0)
        ms, _ = self.graph_time(f, steps)
        return ms

    def layer_step_rate(self, layers, B, grouped, steps=50, seed=206):
        """One step = the seven projections of a layer on one batch of bf16
        activations (the attention input for q, k, v and o; the MLP input for
        gate, up and down: widths 2048 / 2048 / 5504), either as seven
        fairy_cgemv launches or as four (q+k+v and gate+up grouped with
        fairy_cgemv_group).  Every projection reads its own pool of weight
        copies; timed between the event nodes of a graph of `steps` steps.
        Returns ms per step."""
        torch, F = self.torch, self.F
        pools = {k: self.pool(L) for k, L in layers.items()}
        xs, ys = {}, {}
        for k, L in layers.items():
            m = L["m"]
            if m not in xs:
                xr, xi = self.synth.bf16_gaussian((B, m), seed + m)
                xs[m] = (self.dev(xr), self.dev(xi))
            ys[k] = (torch.empty((B, L["n"]), dtype=torch.float32, device="cuda"),
                     torch.empty((B, L["n"]), dtype=torch.float32, device="cuda"))

        def one(k, i):
            L = layers[k]
            descs = pools[k][1]
            xr, xi = xs[L["m"]]
            F.fairy_cgemv(descs[i % len(descs)], xr, xi, F.FAIRY_BF16, B, L["m"], ys[k][0], ys[k][1], L["n"])

        def group(ks, i):
            L0 = layers[ks[0]]
            xr, xi = xs[L0["m"]]
            F.fairy_cgemv_group([pools[k][1][i % len(pools[k][1])] for k in ks], xr, xi, F.FAIRY_BF16, B, L0["m"],
                                [ys[k][0] for k in ks], [ys[k][1] for k in ks], [layers[k]["n"] for k in ks])

        def step(i):
            if grouped:
                group(["q", "k", "v"], i)
                one("o", i)
                group(["gate", "up"], i)
                one("down", i)
            else:
                for k in ("q", "k", "v", "o", "gate", "up", "down"):
                    one(k, i)

        step(0)
        st = torch.cuda.Stream()
        launch, elapsed_ms, cleanup = self.timed_graph(step, steps, st)
        launch()
        launch()
        st.synchronize()
        ms = elapsed_ms() / steps
        cleanup()
        del pools
        torch.cuda.empty_cache()
        return ms

    def group_rate(self, Ls, B, steps=100, seed=207):
        """fairy_cgemv_group over layers Ls (each with its own pool of
        copies) against the same layers launched one by one; ms per step."""
        torch, F = self.torch, self.F
        pools = [self.pool(L) for L in Ls]
        m = Ls[0]["m"]
        xr, xi = self.synth.bf16_gaussian((B, m), seed)
        xr, xi = self.dev(xr), self.dev(xi)
        ys = [(torch.empty((B, L["n"]), dtype=torch.float32, device="cuda"),
               torch.empty((B, L["n"]), dtype=torch.float32, device="cuda")) for L in Ls]
        out = {}
        for grouped in (True, False):
            def step(i):
                if grouped:
                    F.fairy_cgemv_group([p[1][i % len(p[1])] for p in pools], xr, xi, F.FAIRY_BF16, B, m,
                                        [y[0] for y in ys], [y[1] for y in ys], [L["n"] for L in Ls])
                else:
                    for L, p, y in zip(Ls, pools, ys):
                        F.fairy_cgemv(p[1][i % len(p[1])], xr, xi, F.FAIRY_BF16, B, m, y[0], y[1], L["n"])
            step(0)
            st = torch.cuda.Stream()
            launch, elapsed_ms, cleanup = self.timed_graph(step, steps, st)
            launch()
            launch()
            st.synchronize()
            out["grouped" if grouped else "separate"] = elapsed_ms() / steps
            cleanup()
        del pools
        torch.cuda.empty_cache()
        return out

    def lut_rate(self, L, descs, steps=200, seed=202):
        """Table-lookup GEMV, batch 1, bf16 activations, over the weight pool."""
        torch, F = self.torch, self.F
        n, m = L["n"], L["m"]
        xr, xi = self.synth.bf16_gaussian((1, m), seed)
        xr, xi = self.dev(xr), self.dev(xi)
        yr = torch.empty((1, n), dtype=torch.float32, device="cuda")
        yi = torch.empty((1, n), dtype=torch.float32, device="cuda")
        wsb = F.fairy_cgemv_lut_workspace_bytes(descs[0])
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        f = lambda i: F.fairy_cgemv_lut(descs[i % len(descs)], xr, xi, F.FAIRY_BF16, yr, yi, ws, wsb)
        f(0)
        ms, _ = self.graph_time(f, steps)
        return ms

    def attention_rate(self, h, sq, sk, d, causal, iters=10, seed=205):
        torch, F = self.torch, self.F
        bufs = []
        for i, rows in enumerate([sq, sq, sk, sk, sk, sk]):
            bufs.append(self.dev(self.synth.bf16_bits(self.synth.gaussian((h, rows, d), 1.0, seed + i))))
        o_re = torch.empty((h, sq, d), dtype=torch.float32, device="cuda")
        o_im = torch.empty_like(o_re)
        scale = 1.0 / math.sqrt(2 * d)
        f = lambda i: F.fairy_cattention(*bufs, F.FAIRY_BF16, h, sq, sk, d, scale, causal, o_re, o_im)
        f(0)
        return attention_entry(self.ev_time(f, iters), h, sq, sk, d, causal)

    def gemm_rate(self, L, desc, M, xdtype, algo, iters=5, seed=204, graph=False, workspace=False):
        torch, F = self.torch, self.F
        n, m = L["n"], L["m"]
        if xdtype == F.FAIRY_I8:
            xr, xi = self.synth.int8_uniform((M, m), seed)
        else:
            xr, xi = self.synth.bf16_gaussian((M, m), seed)
        xr, xi = self.dev(xr), self.dev(xi)
        yr = torch.empty((M, n), dtype=torch.float32, device="cuda")
        yi = torch.empty((M, n), dtype=torch.float32, device="cuda")
        ws, wsb = None, 0
        if workspace:  # the optional K-split partial sums
            wsb = F.fairy_cgemm_workspace_bytes(desc, M, xdtype, algo)
            ws = torch.empty((max(wsb, 16),), dtype=torch.uint8, device="cuda")
        f = lambda i: F.fairy_cgemm(desc, xr, xi, xdtype, M, m, yr, yi, n, None, algo, ws, wsb)
        f(0)
        if graph:  # short kernels: time graph replays, not host launches
            return self.graph_time(f, iters)[0]
        return self.ev_time(f, iters)


def attention_entry(ms, h, sq, sk, d, causal):
    """Useful work: scores 4 sq sk d (the real-equivalent dot products over 2d)
    plus the weighted sums 4 sq sk d (re and im); causal keeps the visible
    (query, key) pairs.  Matrix-core work of the kernel: 12 sq sk d per
    processed key chunk (the weights go through two bf16 MFMAs)."""
    kc = 128 if d <= 64 else 64  # keys per staged chunk
    if causal:
        pairs = sum(min(sk, i + (sk - sq) + 1) for i in range(sq))
        # a block of 128 queries walks the key chunks up to its last query's diagonal
        mfma_pairs = sum(((min(sk, qb * 128 + 128 + (sk - sq)) + kc - 1) // kc) * kc * 128
                         for qb in range((sq + 127) // 128))
    else:
        pairs = sq * sk
        mfma_pairs = ((sq + 127) // 128) * 128 * ((sk + kc - 1) // kc) * kc
    alg = 8.0 * h * pairs * d
    mf = 12.0 * h * mfma_pairs * d
    t = ms * 1e-3
    return {"ms": ms, "alg_TFLOPs": alg / t / 1e12, "mfma_TFLOPs": mf / t / 1e12,
            "mfma_frac": mf / t / 1e12 / MFMA_PEAK_TFLOPS["bf16"]}


def lut_entry(ms, ms_direct, L):
    """Table-lookup GEMV beside the direct decode on the same layer and input."""
    return {"ms": ms, "packed_GB/s": L["packed_bytes"] / (ms * 1e-3) / 1e9,
            "direct_ms": ms_direct, "direct_over_lut": round(ms_direct / ms, 3)}


def gemm_entry(ms, P, n, m, M, peak=None):
    alg = 2.0 * P * n * m * M            # additions of the multiplication-free form
    mfma_ops = 8.0 * P * n * m * M       # 2 x MACs on the ternary planes (4 MACs per code per token)
    out = {"ms": ms, "alg_TOPS": alg / (ms * 1e-3) / 1e12}
    if peak:
        t = mfma_ops / (ms * 1e-3) / 1e12
        out.update({"mfma_TOPS": t, "mfma_peak_TOPS": peak, "mfma_frac": t / peak})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-rows", action="store_true", help="skip the other rows of the path")
    ap.add_argument("--sweep", action="store_true", help="also run the full-layer sweep (slow)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--prefill", action="store_true",
                    help="only time the M=2048 prefill GEMM on the 2048x2048 S=2 layer (bf16 and int8, "
                         "matrix cores), e.g. under a profiler")
    ap.add_argument("--attention", action="store_true",
                    help="only time the complex attention at 32 heads x 2048 tokens, d 64 (causal and full), "
                         "e.g. under a profiler")
    ap.add_argument("--lut", action="store_true",
                    help="only time the table-lookup GEMV beside the direct one, batch 1, on the 2048x2048 "
                         "S=2 layer, e.g. under a profiler")
    ap.add_argument("--layer", action="store_true",
                    help="only time the whole S=2 layer step (7 projections, batch 1 and 4) as 7 launches and as "
                         "4 with the grouped GEMV, e.g. under a profiler")
    ap.add_argument("--quant", action="store_true",
                    help="only time PhaseQuant (S=2) and pack on the 2048x2048 layer, e.g. under a profiler")
    ap.add_argument("--calib", action="store_true",
                    help="only measure the ceilings: a plain 256 MiB copy (the byte-counter calibration "
                         "kernel), 4 MiB and 32 MiB copy launches and tiny launches in HIP graphs")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (libfairy has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    bn = Bench()
    torch, F, synth = bn.torch, bn.F, bn.synth
    if args.calib:
        print(json.dumps(calibrate(bn)), flush=True)
        return
    if args.attention:
        out = {f"cattention_32x2048_d64_{'causal' if c else 'full'}": bn.attention_rate(32, 2048, 2048, 64, c,
                                                                                      iters=args.steps)
               for c in (1, 0)}
        print(json.dumps(out), flush=True)
        return
    if args.lut:
        L = bn.widely_linear_layer(4096, 4096, 2, seed=200)
        copies, descs = bn.pool(L)
        ms_l = bn.lut_rate(L, descs, steps=args.steps)
        ms_d = bn.gemv_rate(L, descs, 1, F.FAIRY_BF16, steps=args.steps)
        print(json.dumps({"gemv_lut_2048x2048_bf16_B1": lut_entry(ms_l, ms_d, L)}), flush=True)
        return
    if args.quant:
        L = bn.widely_linear_layer(4096, 4096, 2, seed=200)
        n, m, S, P = L["n"], L["m"], L["S"], L["P"]
        pl, cd, sc, ws, wsb = L["planes"], L["codes"], L["scales"], L["ws"], L["wsb"]
        ms_q = bn.graph_ms(lambda i: F.fairy_phasequant(pl[0], pl[1], L["count"], S, cd[0], sc[0], None, None, ws,
                                                        wsb), args.steps)
        ms_p = bn.graph_ms(lambda i: F.fairy_pack(cd, P, n, m, F.FAIRY_LAYOUT_TILED64, L["packed"]), args.steps)
        # the whole conversion of the real layer in one call, checked against the steps
        q_packed, q_scales = torch.empty_like(L["packed"]), torch.empty_like(L["scales"])
        wsq = F.fairy_quantize_workspace_bytes(n, m, S, 1)
        wq = torch.empty(wsq, dtype=torch.uint8, device="cuda")
        ms_r = bn.graph_ms(lambda i: F.fairy_quantize_real(L["R"], n, m, S, q_packed, q_scales, wq, wsq), args.steps)
        if not (torch.equal(q_packed, L["packed"]) and torch.equal(q_scales, L["scales"])):
            raise SystemExit("fairy_quantize_real differs from the step-by-step conversion")
        print(json.dumps({"phasequant_S2_2048x2048": {"ms": ms_q, "unique_GB/s": (L["count"] * 8) / (ms_q * 1e-3) / 1e9},
                          "pack_P4_2048x2048": {"ms": ms_p, "GB/s": (P * L["count"] * 1.25) / (ms_p * 1e-3) / 1e9},
                          "quantize_real_4096x4096_S2": {"ms": ms_r,
                                                         "R_GB/s": (4 * n * m * 4) / (ms_r * 1e-3) / 1e9}}),
              flush=True)
        return
    if args.layer:
        proj = {"q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096), "o": (4096, 4096),
                "gate": (11008, 4096), "up": (11008, 4096), "down": (4096, 11008)}
        layers = {name: bn.widely_linear_layer(rr, cc, 2, 520 + i) for i, (name, (rr, cc)) in enumerate(proj.items())}
        tot = sum(L["packed_bytes"] for L in layers.values())
        out = {}
        for B in (1, 4):
            for grouped in (False, True):
                ms_l = bn.layer_step_rate(layers, B, grouped, steps=args.steps)
                out[f"layer_step_S2_B{B}_{'grouped' if grouped else 'separate'}"] = {
                    "ms": ms_l, "packed_GB/s": tot / (ms_l * 1e-3) / 1e9}
        print(json.dumps(out), flush=True)
        return
    if args.prefill:
        L = bn.widely_linear_layer(4096, 4096, 2, seed=200)
        d0 = F.make_clinear(L["n"], L["m"], L["S"], 1, L["packed"], L["scales"])
        out = {}
        for dt, dn in ((F.FAIRY_BF16, "bf16"), (F.FAIRY_I8, "i8")):
            msg = bn.gemm_rate(L, d0, 2048, dt, F.FAIRY_ALGO_MFMA, iters=args.steps)
            out[f"gemm_2048x2048_M2048_{dn}_mfma"] = gemm_entry(msg, L["P"], L["n"], L["m"], 2048,
                                                                MFMA_PEAK_TFLOPS[dn])
        print(json.dumps(out), flush=True)
        return

    # ---- the metric's workload ------------------------------------------------------
    log("building widely-linear 4096x4096 -> 2048x2048, S=2")
    L = bn.widely_linear_layer(4096, 4096, 2, seed=200)
    n, m, S, P, packed_bytes = L["n"], L["m"], L["S"], L["P"], L["packed_bytes"]
    copies, descs = bn.pool(L)
    ncopy = len(copies)

    B = args.batch
    rb, ib = synth.bf16_gaussian((B, m), seed=201)
    x_re, x_im = bn.dev(rb), bn.dev(ib)
    y_re = torch.empty((B, n), dtype=torch.float32, device="cuda")
    y_im = torch.empty((B, n), dtype=torch.float32, device="cuda")

    def gemv(i):
        F.fairy_cgemv(descs[i % ncopy], x_re, x_im, F.FAIRY_BF16, B, m, y_re, y_im, n)

    for i in range(args.warmup):
        gemv(ncopy - 1 - (i % ncopy))
    torch.cuda.synchronize()
    eager_y = (y_re.clone(), y_im.clone())
    eager_ms = bn.ev_time(gemv, min(args.steps, 200))
    y_re.zero_(); y_im.zero_()
    # read-only cache flush: 512 MiB as [32768][4096] fp32 (row sums, the
    # fastest streaming read among torch's reductions here)
    flush = torch.ones((32768, 4096), dtype=torch.float32, device="cuda")
    t0 = time.perf_counter()
    ms, run_ms, touched, ms_outer = bn.cold_runs(gemv, args.steps, ncopy, flush)
    wall = time.perf_counter() - t0
    if not (torch.equal(y_re, eager_y[0]) and torch.equal(y_im, eager_y[1])):
        raise SystemExit("graph replay output differs from the eager GEMV output")
    gbs = packed_bytes / (ms * 1e-3) / 1e9
    # the device's streaming ceiling: a 256 MiB device copy (bytes read + written)
    csrc = torch.empty((64 << 20,), dtype=torch.int32, device="cuda")
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    copy_ms = bn.ev_time(lambda i: cdst.copy_(csrc), 10)
    copy_gbs = 2 * csrc.numel() * 4 / (copy_ms * 1e-3) / 1e9
    # and its streaming-read rate: the flush read itself (512 MiB read, 128 KiB written)
    rsum = torch.empty((flush.shape[0],), dtype=torch.float32, device="cuda")
    torch.sum(flush, dim=1, out=rsum)
    read_ms = bn.ev_time(lambda i: torch.sum(flush, dim=1, out=rsum), 10)
    read_gbs = flush.numel() * 4 / (read_ms * 1e-3) / 1e9
    del csrc, cdst, rsum, flush
    alg_bytes = packed_bytes + B * m * 2 * 2 + B * n * 2 * 4
    hbm_achieved = alg_bytes / (ms * 1e-3) / 1e9
    # the multiplication-free form: two fp32 adds per code per batch column
    alg_adds = 2 * P * n * m * B
    alu_achieved = alg_adds / (ms * 1e-3) / 1e12
    log(f"GEMV B={B}: cold graph runs {ms * 1e3:.2f} us/launch median of {len(run_ms)} "
        f"({', '.join(f'{r * 1e3:.2f}' for r in run_ms)}), {gbs:.0f} GB/s packed; eager {eager_ms * 1e3:.2f} "
        f"us/call; {touched} distinct copies in the timed runs; wall {wall:.3f}s")

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
            "weight_bytes_timed_per_run": packed_bytes * min(args.steps, ncopy),
            "complex_weights_per_s": P * n * m / (ms * 1e-3),
            "hbm_frac_packed": round(gbs / HBM_PEAK_GBS, 4),
        },
        # The kernel streams the packed codes once (counter-measured traffic
        # within a few % of the algorithmic bytes), so its roof is HBM; the
        # vector ALU busy fraction from the counters stands beside it.
        "roofline": {
            "bound": "hbm",
            "achieved": round(hbm_achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(hbm_achieved / HBM_PEAK_GBS, 4),
            "traffic": GEMV_TRAFFIC_BYTES if B == 1 else None,
            "kernel": GEMV_KERNEL,
            "alg_bytes_per_launch": alg_bytes,
            "kernel_us_per_launch": round(ms * 1e3, 4),
            "timing": f"median of {len(run_ms)} cold runs of {args.steps} graph-replayed launches each, "
                      f"between two event record nodes of the graph (the first and last node); 512 MiB "
                      f"read before each timed replay",
            "us_per_launch_incl_graph_launch": round(ms_outer * 1e3, 4),
            "run_us_per_launch": [round(r * 1e3, 4) for r in run_ms],
            "distinct_weight_copies_timed": touched,
            "measured_copy_GBps": round(copy_gbs, 1),
            "frac_of_measured_copy": round(hbm_achieved / copy_gbs, 4),
            "measured_read_GBps": round(read_gbs, 1),
            "frac_of_measured_read": round(hbm_achieved / read_gbs, 4),
            "valu": {"alg_adds_per_launch": alg_adds, "alg_Tadds_per_s": round(alu_achieved, 3),
                     "peak_Tlane_ops_per_s": round(VALU_PEAK_TOPS, 2),
                     "busy_frac_counters": GEMV_VALU_BUSY if B == 1 else None},
            "eager_ms_per_call": eager_ms,
        },
    }

    # ---- other rows of the path ---------------------------------------------------------
    if not args.no_rows:
        rows_out = {}
        R, planes, codes, scales, ws, wsb = L["R"], L["planes"], L["codes"], L["scales"], L["ws"], L["wsb"]
        count = L["count"]
        ms_c = bn.graph_ms(lambda i: F.fairy_real_to_complex(R, n, m, *planes), 20)
        rows_out["real_to_complex_4096x4096"] = {"ms": ms_c, "GB/s": (4 * 4 * n * m * 2) / (ms_c * 1e-3) / 1e9}
        ms_q = bn.graph_ms(lambda i: F.fairy_phasequant(planes[0], planes[1], count, S, codes[0], scales[0], None,
                                                        None, ws, wsb), 20)
        rows_out["phasequant_S2_2048x2048"] = {"ms": ms_q, "unique_GB/s": (count * 8) / (ms_q * 1e-3) / 1e9}
        ms_p = bn.graph_ms(lambda i: F.fairy_pack(codes, P, n, m, F.FAIRY_LAYOUT_TILED64, L["packed"]), 20)
        rows_out["pack_P4_2048x2048"] = {"ms": ms_p, "GB/s": (P * count * 1.25) / (ms_p * 1e-3) / 1e9}
        # the whole conversion (split, PhaseQuant of U and W, pack) in one call
        q_packed, q_scales = torch.empty_like(L["packed"]), torch.empty_like(L["scales"])
        wsq = F.fairy_quantize_workspace_bytes(n, m, S, 1)
        wq = torch.empty(wsq, dtype=torch.uint8, device="cuda")
        ms_r = bn.graph_ms(lambda i: F.fairy_quantize_real(R, n, m, S, q_packed, q_scales, wq, wsq), 10)
        if not (torch.equal(q_packed, L["packed"]) and torch.equal(q_scales, L["scales"])):
            raise SystemExit("fairy_quantize_real differs from the step-by-step conversion")
        rows_out["quantize_real_4096x4096_S2"] = {"ms": ms_r, "R_GB/s": (4 * n * m * 4) / (ms_r * 1e-3) / 1e9}
        del wq
        for bb in (4, 16, 64):
            msb = bn.gemv_rate(L, descs, bb, F.FAIRY_BF16, steps=100)
            rows_out[f"gemv_2048x2048_bf16_B{bb}"] = {
                "ms": msb, "packed_GB/s": packed_bytes / (msb * 1e-3) / 1e9,
                "alg_Tadds/s": 2 * P * n * m * bb / (msb * 1e-3) / 1e12}
        ms8 = bn.gemv_rate(L, descs, 1, F.FAIRY_I8, steps=200)
        rows_out["gemv_2048x2048_i8_B1"] = {"ms": ms8, "packed_GB/s": packed_bytes / (ms8 * 1e-3) / 1e9}
        ms1 = ms if B == 1 else bn.gemv_rate(L, descs, 1, F.FAIRY_BF16, steps=200)
        rows_out["gemv_lut_2048x2048_bf16_B1"] = lut_entry(bn.lut_rate(L, descs), ms1, L)
        del copies, descs
        # q, k, v in one launch (three pools of the same quantised layer)
        gq = bn.group_rate([L, L, L], 1)
        rows_out["gemv_group_qkv_3x2048x2048_bf16_B1"] = {
            "ms": gq["grouped"], "separate_ms": gq["separate"],
            "packed_GB/s": 3 * packed_bytes / (gq["grouped"] * 1e-3) / 1e9,
            "separate_packed_GB/s": 3 * packed_bytes / (gq["separate"] * 1e-3) / 1e9}
        torch.cuda.empty_cache()
        # MLP shapes (gate/up: 11008x4096, down: 4096x11008)
        for name, (rr, cc, sd) in {"gate_up_5504x2048": (11008, 4096, 300),
                                   "down_2048x5504": (4096, 11008, 302)}.items():
            L2 = bn.widely_linear_layer(rr, cc, 2, sd)
            c2, d2 = bn.pool(L2)
            if name.startswith("gate"):
                gg = bn.group_rate([L2, L2], 1)
                rows_out["gemv_group_gate_up_2x5504x2048_bf16_B1"] = {
                    "ms": gg["grouped"], "separate_ms": gg["separate"],
                    "packed_GB/s": 2 * L2["packed_bytes"] / (gg["grouped"] * 1e-3) / 1e9,
                    "separate_packed_GB/s": 2 * L2["packed_bytes"] / (gg["separate"] * 1e-3) / 1e9}
            for bb in (1, 8):
                msm = bn.gemv_rate(L2, d2, bb, F.FAIRY_BF16, steps=200)
                rows_out[f"gemv_{name}_bf16_B{bb}"] = {
                    "ms": msm, "packed_GB/s": L2["packed_bytes"] / (msm * 1e-3) / 1e9}
                if bb == 1:
                    rows_out[f"gemv_lut_{name}_bf16_B1"] = lut_entry(bn.lut_rate(L2, d2), msm, L2)
            del c2, d2
            if name.startswith("gate"):
                # prefill GEMM, M = 2048 tokens, on the 5504-row layer
                d1 = F.make_clinear(L2["n"], L2["m"], 2, 1, L2["packed"], L2["scales"])
                msg = bn.gemm_rate(L2, d1, 2048, F.FAIRY_BF16, F.FAIRY_ALGO_MFMA)
                rows_out["gemm_5504x2048_M2048_bf16_mfma"] = gemm_entry(msg, 4, L2["n"], L2["m"], 2048,
                                                                        MFMA_PEAK_TFLOPS["bf16"])
                msg = bn.gemm_rate(L2, d1, 2048, F.FAIRY_I8, F.FAIRY_ALGO_MFMA)
                rows_out["gemm_5504x2048_M2048_i8_mfma"] = gemm_entry(msg, 4, L2["n"], L2["m"], 2048,
                                                                      MFMA_PEAK_TFLOPS["i8"])
                # the same prefill on the vector ALUs (direct decode, no matrix cores)
                for dt, dn in ((F.FAIRY_BF16, "bf16"), (F.FAIRY_I8, "i8")):
                    msg = bn.gemm_rate(L2, d1, 2048, dt, F.FAIRY_ALGO_VALU, iters=2)
                    rows_out[f"gemm_5504x2048_M2048_{dn}_valu"] = gemm_entry(msg, 4, L2["n"], L2["m"], 2048)
            del L2
            torch.cuda.empty_cache()
        d0 = F.make_clinear(n, m, S, 1, L["packed"], L["scales"])
        # the matrix-core GEMM at decode batch sizes, beside the VALU GEMV
        # rows: one launch over 32 row blocks, and split along K (with the
        # optional workspace) to fill the chip
        for mm in (16, 64):
            msg = bn.gemm_rate(L, d0, mm, F.FAIRY_BF16, F.FAIRY_ALGO_MFMA, iters=100, graph=True)
            rows_out[f"gemm_2048x2048_M{mm}_bf16_mfma"] = gemm_entry(msg, P, n, m, mm, MFMA_PEAK_TFLOPS["bf16"])
            msg = bn.gemm_rate(L, d0, mm, F.FAIRY_BF16, F.FAIRY_ALGO_MFMA, iters=100, graph=True, workspace=True)
            rows_out[f"gemm_2048x2048_M{mm}_bf16_mfma_splitk"] = gemm_entry(msg, P, n, m, mm,
                                                                           MFMA_PEAK_TFLOPS["bf16"])
        for dt, dn in ((F.FAIRY_BF16, "bf16"), (F.FAIRY_I8, "i8")):
            msg = bn.gemm_rate(L, d0, 2048, dt, F.FAIRY_ALGO_MFMA)
            rows_out[f"gemm_2048x2048_M2048_{dn}_mfma"] = gemm_entry(msg, P, n, m, 2048, MFMA_PEAK_TFLOPS[dn])
            msg = bn.gemm_rate(L, d0, 2048, dt, F.FAIRY_ALGO_VALU, iters=2)
            rows_out[f"gemm_2048x2048_M2048_{dn}_valu"] = gemm_entry(msg, P, n, m, 2048)
        # complex attention at the LLaMA-2-7B prefill shape: 32 heads, 2048
        # tokens, real head dim 128 = complex d 64
        for causal in (1, 0):
            rows_out[f"cattention_32x2048_d64_{'causal' if causal else 'full'}"] = bn.attention_rate(
                32, 2048, 2048, 64, causal)
        result["rows"] = rows_out
        log(json.dumps(rows_out))

    if args.sweep:
        result["sweep"] = full_layer_sweep(bn)

    # ---- CPU oracle baseline (bounded sample of the same workload) ---------------------
    if not args.no_cpu:
        import oracle
        Rh = synth.real_layer(4096, 4096, 200)
        ur, ui, wr, wi = oracle.real_to_complex(Rh, n, m, f32=True)
        t_q = time.perf_counter()
        cu, su, _, _ = oracle.phasequant(ur, ui, S, want_resid=False)
        t_q = time.perf_counter() - t_q
        cw, sw, _, _ = oracle.phasequant(wr, wi, S, want_resid=False)
        oc = np.concatenate([cu, cw]); osc = np.concatenate([su, sw])
        t_p = time.perf_counter()
        oracle.pack(oc, F.FAIRY_LAYOUT_TILED64)
        t_p = time.perf_counter() - t_p
        xr, xi = synth.bf16_to_f32(rb), synth.bf16_to_f32(ib)

        def oracle_rate(threads, seconds):
            used = oracle.set_threads(threads)
            reps, t0 = 0, time.perf_counter()
            while True:
                oracle.cgemv_dense(oc, osc, S, True, xr, xi)
                reps += 1
                el = time.perf_counter() - t0
                if el >= seconds or reps >= 100000:
                    return used, reps, el

        # all the host cores this process may use (a GPU's share of a shared
        # host can be fewer than the CPU count; OMP_NUM_THREADS states it),
        # then one core
        all_threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
        cores, reps, el = oracle_rate(all_threads, args.cpu_seconds)
        _, reps1, el1 = oracle_rate(1, args.cpu_seconds / 2)
        # a 64-token slice of the M = 2048 prefill on the same layer (all threads)
        oracle.set_threads(all_threads)
        gx_r, gx_i = synth.bf16_gaussian((64, m), seed=204)
        t_g = time.perf_counter()
        oracle.cgemv_dense(oc, osc, S, True, synth.bf16_to_f32(gx_r), synth.bf16_to_f32(gx_i))
        t_g = time.perf_counter() - t_g
        cpu_model = "unknown"
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        cpu_model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
        result["cpu_baseline"] = {
            "value": round(packed_bytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{reps} full GEMVs of the same 2048x2048 S=2 widely-linear layer, batch {B}, "
                      f"dense fp64 oracle over output rows on {cores} threads, {el:.1f}s",
            "single_thread": {"value": round(packed_bytes * reps1 / el1 / 1e9, 4), "unit": "GB/s",
                              "sample": f"{reps1} GEMVs on 1 thread, {el1:.1f}s"},
            "cpu_model": cpu_model, "nproc": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            # the other steps of the path, each run once by the oracle on this host
            "other_steps": {
                "phasequant_S2_2048x2048_ms_1thread": round(t_q * 1e3, 2),
                "pack_P4_2048x2048_tiled64_ms_1thread": round(t_p * 1e3, 2),
                "prefill_2048x2048_S2_ms_per_token": round(t_g * 1e3 / 64, 3),
                "prefill_sample": f"64 tokens of the M=2048 prefill, bf16 N(0,1), {all_threads} threads",
            },
        }

    print(json.dumps(result), flush=True)


def calibrate(bn):
    """Ceilings of the part, with plain copies: one of known size (256 MiB in,
    256 MiB out; its FETCH_SIZE / WRITE_SIZE calibrate the byte counters),
    copies moving 4 MiB and 32 MiB per launch over a 1 GiB pool, and tiny
    launches, each of the latter captured as a HIP graph."""
    torch = bn.torch
    out = {}
    src = torch.randint(0, 1 << 30, (64 << 20,), dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    ms = bn.ev_time(lambda i: dst.copy_(src), 10)
    out["copy_256MiB"] = {"ms": ms, "bytes_read": src.numel() * 4, "bytes_written": dst.numel() * 4,
                          "GB/s_read+write": 2 * src.numel() * 4 / (ms * 1e-3) / 1e9}
    pool = torch.ones((1 << 28,), dtype=torch.int32, device="cuda")     # 1 GiB
    for mib in (4, 32):
        # one launch moves `mib` MiB: a copy of mib/2 MiB between two distinct
        # slices of the pool (half read, half written)
        n = (mib << 20) // 8
        k = pool.numel() // (2 * n)
        f = lambda i: pool[(2 * (i % k) + 1) * n:(2 * (i % k) + 2) * n].copy_(pool[2 * (i % k) * n:(2 * (i % k) + 1) * n])
        f(0)
        ms, _ = bn.graph_time(f, 128)
        out[f"copy_{mib}MiB_traffic_per_launch"] = {"us": ms * 1e3, "GB/s": (mib << 20) / (ms * 1e-3) / 1e9}
    e = torch.empty((1,), dtype=torch.int32, device="cuda")
    ms, _ = bn.graph_time(lambda i: e.zero_(), 256)
    out["tiny_launch_us"] = ms * 1e3
    return out


def full_layer_sweep(bn):
    """All seven projections of a LLaMA-2-7B-shaped layer in widely-linear form
    with 1/2/3 residual stages and batch 1/4/16/64, plus a pure complex
    (no conjugate branch) 2048x2048 and 8192x2048 layer set with PhaseQuant
    timed on each.  Reports per-projection GEMV time and the layer total."""
    F, torch, synth = bn.F, bn.torch, bn.synth
    proj = {"q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096), "o": (4096, 4096),
            "gate": (11008, 4096), "up": (11008, 4096), "down": (4096, 11008)}
    out = {}
    for S in (1, 2, 3):
        layers = {name: bn.widely_linear_layer(rr, cc, S, 500 + 10 * S + i)
                  for i, (name, (rr, cc)) in enumerate(proj.items())}
        # PhaseQuant of every projection's U and W (rewrites the same codes
        # and scales the layer was packed from)
        pq = {}
        for name, L in layers.items():
            def quant(i, L=L):
                for k in (0, 2):
                    F.fairy_phasequant(L["planes"][k], L["planes"][k + 1], L["count"], S, L["codes"][k // 2 * S],
                                       L["scales"][k // 2 * S], None, None, L["ws"], L["wsb"])
            pq[name] = bn.ev_time(quant, 3)
        out[f"phasequant_layer_S{S}"] = {"ms_total": sum(pq.values()), "per_proj_ms": pq}
        log(f"sweep S={S}: PhaseQuant of U and W over the 7 projections {sum(pq.values()):.3f} ms")
        for B in (1, 4, 16, 64):
            tot_ms, tot_bytes, per = 0.0, 0, {}
            for name, L in layers.items():
                copies, descs = bn.pool(L)
                ms = bn.gemv_rate(L, descs, B, F.FAIRY_BF16, steps=100)
                per[name] = ms
                tot_ms += ms
                tot_bytes += L["packed_bytes"]
                del copies, descs
                torch.cuda.empty_cache()
            out[f"layer_S{S}_B{B}"] = {"ms_total": tot_ms, "packed_bytes": tot_bytes,
                                        "packed_GB/s": tot_bytes / (tot_ms * 1e-3) / 1e9, "per_proj_ms": per}
            log(f"sweep S={S} B={B}: {tot_ms * 1e3:.1f} us, {tot_bytes / (tot_ms * 1e-3) / 1e9:.0f} GB/s")
            # the whole layer as one step: seven launches, or four with q+k+v
            # and gate+up grouped
            for grouped in (False, True):
                ms_l = bn.layer_step_rate(layers, B, grouped)
                key = f"layer_step_S{S}_B{B}_{'grouped' if grouped else 'separate'}"
                out[key] = {"ms": ms_l, "launches": 4 if grouped else 7,
                            "packed_GB/s": tot_bytes / (ms_l * 1e-3) / 1e9}
                log(f"sweep S={S} B={B} layer step ({'4 grouped' if grouped else '7'} launches): "
                    f"{ms_l * 1e3:.1f} us, {tot_bytes / (ms_l * 1e-3) / 1e9:.0f} GB/s")
        del layers
        torch.cuda.empty_cache()
    # pure complex layers (no conjugate branch): per-component sigma 0.02
    for (n, m) in ((2048, 2048), (8192, 2048)):
        for S in (1, 2):
            re, im = synth.complex_gaussian((n, m), 0.02, 900 + n + S)
            count = n * m
            codes = torch.empty((S, n, m), dtype=torch.uint8, device="cuda")
            scales = torch.empty((S, 2), dtype=torch.float32, device="cuda")
            wsb = F.fairy_phasequant_workspace_bytes(count, S)
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            wre, wim = bn.dev(re), bn.dev(im)
            ms_q = bn.ev_time(lambda i: F.fairy_phasequant(wre, wim, count, S, codes, scales, None, None, ws, wsb), 5)
            nw = F.fairy_packed_words(n, m, S, F.FAIRY_LAYOUT_TILED64)
            packed = torch.empty(nw, dtype=torch.int32, device="cuda")
            F.fairy_pack(codes, S, n, m, F.FAIRY_LAYOUT_TILED64, packed)
            L = dict(n=n, m=m, S=S, packed=packed, scales=scales, packed_bytes=nw * 4)
            copies, descs = bn.pool(L, has_conj=0)
            for B in (1, 16):
                ms = bn.gemv_rate(L, descs, B, F.FAIRY_BF16, steps=100)
                out[f"complex_{n}x{m}_S{S}_B{B}"] = {"ms": ms, "packed_GB/s": nw * 4 / (ms * 1e-3) / 1e9,
                                                      "phasequant_ms": ms_q}
            del copies, descs
            torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
