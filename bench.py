#!/usr/bin/env python3
"""Benchmark of the BitLinear hot path on one MI355X.

Headline (the JSON line's `value`): decode GEMV weight throughput, GB/s of
packed 2-bit weights streamed per second, on the decode workload (M = 1
token, W 4096 x 4096 bf16 quantised once, x bf16 N(0,1) with 1% outliers at
+/-20). One step = one token through one layer: per-token INT8 quantisation
of x, then the integer product with the fused dequant epilogue. Steps rotate
over 128 distinct packed weight copies (512 MiB, twice the 256 MB
Infinity Cache), and the caches are flushed (a 512 MiB read) right before
every timed replay, so every timed launch reads its weights from HBM whatever
the step count.

The same run measures the other rows of the path and reports them under
"rows": the base-3 layout of the decode GEMV, weight packing, activation
quantisation at prefill size, the prefill GEMM (M = 2048, K = 4096,
N = 11008, INT8 TOPS), one transformer block's six BitLinear layers for one
decode token (four fused launches), at decode batch 16 and at prefill 512
(tokens/s), the training step at
M = K = N = 4096 (re-quantise, INT8 forward, bf16 straight-through backward
products) and, for context, the same decode and prefill layers with dense
bf16 weights through torch linear (hipBLASLt).

Timing: every measured sequence is captured once into a HIP graph and
replayed between two HIP events on the replay stream, so host-side launch
cost is not measured. `roofline` describes the dominant kernel (the 2-bit
fused decode step): algorithmic bytes per launch over its mean launch
duration in the timed graph, against the 8 TB/s datasheet peak and against
a measured ceiling, a plain streaming read of one 4 MiB buffer per launch
over the same rotation (rows.ceilings also holds a 512 MiB read, the graph
cadence of empty launches and an INT8 matrix-core loop). `cpu_baseline`
times the CPU oracle on a bounded sample of the same decode workload, plus
each stage of the pass on one thread and on all host threads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5033.0        # dense INT8 MFMA: 256 CU x 4 SIMD x 2048 ops/clk x 2.4 GHz
BF16_PEAK_TFLOPS = 2516.0      # dense bf16 MFMA: 256 CU x 4 SIMD x 1024 flops/clk x 2.4 GHz
METRIC = "BitLinear weight GB/s (decode GEMV) + INT8 TOPS (prefill), % of roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=128, help="distinct packed weight copies")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only", default="", help="comma list of rows to run (profiling runs)")
    ap.add_argument("--mode", default="full", choices=["full", "profile"],
                    help="profile: only the fused decode kernel (64 launches over rotating "
                         "weight copies; with --only prefill, 8 launches of the 2-bit prefill "
                         "GEMM instead) and a 512 MiB device copy, for counter runs")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding is described, not run.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from ternary_weight_linear_bitlinear_amd import build as _build
    if not os.path.exists(_build.LIB_PATH):
        _build.build_library()
    from ternary_weight_linear_bitlinear_amd import bitlinear as bl
    from ternary_weight_linear_bitlinear_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    only = set(filter(None, args.only.split(",")))

    def want(name):
        return not only or name in only

    def to_dev(a, bf16):
        if bf16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # probes: a plain streaming read (also the cache flush), empty launches
    # and an INT8 matrix-core loop
    import ctypes
    if not os.path.exists(_build.PROBES_PATH):
        _build.build_probes()
    probes = ctypes.CDLL(_build.PROBES_PATH)
    probes.probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_void_p]
    probes.probe_empty.argtypes = [ctypes.c_void_p]
    probes.probe_mfma_i8.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    probe_out = torch.empty(1 << 16, dtype=torch.int32, device=dev)

    def cur_stream():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def probe_read(buf, blocks, unroll):
        st = probes.probe_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                               blocks, unroll, ctypes.c_void_p(probe_out.data_ptr()), cur_stream())
        assert st == 0, f"probe_read: HIP error {st}"

    # 512 MiB read before every timed replay: evicts the 256 MB Infinity Cache
    # and the L2s, so timed launches find nothing of earlier replays in them
    flush_buf = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)

    def flush():
        probe_read(flush_buf, 2048, 4)

    def graph_ms(fn, n, warm=3, warm_ms=25.0):
        """Capture fn(0..n-1) into one HIP graph; replay it untimed at least `warm`
        times and for at least `warm_ms` of GPU time (clocks reach steady state:
        heavy GEMMs run ~10% slower in the first tens of milliseconds), flush the
        caches, then replay once between two HIP events on the replay stream.
        Returns ms per call."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(0)  # first call outside capture (sets kernel attributes)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        spent, reps = 0.0, 0
        while reps < warm or spent < warm_ms:
            torch.cuda.synchronize()
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            spent += a.elapsed_time(b)
            reps += 1
        flush()
        torch.cuda.synchronize()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / n

    rows = {}

    if args.mode == "profile":
        if "prefill" in only:
            q = synth.workload("prefill")
            xq, sc = bl.bitlinear_quant_acts(to_dev(q.x_store, True))
            packed, gamma = bl.bitlinear_pack_weights(to_dev(q.w_store, True), "2bit")
            y = torch.empty((q.M, q.N), dtype=torch.bfloat16, device=dev)
            for i in range(8):
                bl.bitlinear_forward(xq, sc, packed, gamma, q.N, q.K, "2bit", torch.bfloat16, y=y)
        else:
            p = synth.workload("decode")
            W = to_dev(p.w_store, True)
            x = to_dev(p.x_store, True)
            packed, gamma = bl.bitlinear_pack_weights(W, "2bit")
            copies = [packed.clone() for _ in range(args.copies)]
            y = torch.empty((1, p.N), dtype=torch.float32, device=dev)
            for i in range(64):
                bl.bitlinear_linear(x, copies[i % args.copies], gamma, p.N, "2bit", y=y)
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)  # calibration: reads and writes exactly 512 MiB
        torch.cuda.synchronize()
        log("profile mode done")
        return

    # ---------------------------------------------------------------- decode
    log("decode workload: generating inputs")
    p = synth.workload("decode")
    W = to_dev(p.w_store, True)
    R = args.copies
    xs = [to_dev(synth.make_problem(M=1, N=1, K=p.K, seed=1000 + r, dtype="bf16",
                                    outlier_frac=0.01).x_store, True) for r in range(R)]
    decode = {}
    # ternary codes in the 2-bit and base-3 layouts; the 1-bit variant's
    # binary codes of the same W in the 1-bit layout
    for layout in ("2bit", "base3", "1bit"):
        scheme = "binary" if layout == "1bit" else "ternary"
        packed, gamma = bl.bitlinear_pack_weights(W, layout, scheme)
        copies = [packed.clone() for _ in range(R)]
        y = torch.empty((1, p.N), dtype=torch.float32, device=dev)
        xq = torch.empty((1, p.K), dtype=torch.int8, device=dev)
        sc = torch.empty(4, dtype=torch.float32, device=dev)[:1]
        xq_r, sc_r = [], []
        for r in range(R):
            a, b = bl.bitlinear_quant_acts(xs[r])
            xq_r.append(a)
            sc_r.append(b)
        rb = packed.shape[1]
        wbytes = p.N * rb

        def step(i, copies=copies, gamma=gamma, layout=layout, y=y):
            # one token through one layer: fused quantise + multiply (one launch)
            r = i % R
            bl.bitlinear_linear(xs[r], copies[r], gamma, p.N, layout, y=y)

        def step_two(i, copies=copies, gamma=gamma, layout=layout, y=y, xq=xq, sc=sc):
            r = i % R
            bl.bitlinear_quant_acts(xs[r], xq=xq, scale=sc)
            bl.bitlinear_forward(xq, sc, copies[r], gamma, p.N, p.K, layout, y=y)

        def gemv(i, copies=copies, gamma=gamma, layout=layout, y=y):
            r = i % R
            bl.bitlinear_forward(xq_r[r], sc_r[r], copies[r], gamma, p.N, p.K, layout, y=y)

        def gemv_lut(i, copies=copies, gamma=gamma, y=y):
            r = i % R
            bl.bitlinear_forward_lut(xq_r[r], sc_r[r], copies[r], gamma, p.N, p.K, y=y)

        for i in range(args.warmup):
            step(i)
        # the timed region is one graph replay of exactly `steps` steps
        ms_step = graph_ms(step, args.steps)
        ms_two = graph_ms(step_two, args.steps)
        k_mean = graph_ms(gemv, 2 * R)
        lut_ms = graph_ms(gemv_lut, 2 * R) if layout == "base3" else None
        # fused kernel: packed weights + bf16 x + gamma + fp32 y
        alg = wbytes + 2 * p.K + 4 + 4 * p.N
        decode[layout] = dict(scheme=scheme, ms_per_step=ms_step, weight_bytes=wbytes,
                              weight_gbs=wbytes / (ms_step * 1e-3) / 1e9,
                              fused_alg_bytes=alg,
                              fused_gbs=alg / (ms_step * 1e-3) / 1e9,
                              two_launch_ms_per_step=ms_two,
                              forward_only_ms=k_mean,
                              forward_only_gbs=(wbytes + p.K + 8 + 4 * p.N) / (k_mean * 1e-3) / 1e9)
        if lut_ms is not None:
            # the same product by activation-side lookup tables (comparison)
            decode[layout]["lookup_table_forward_ms"] = lut_ms
            decode[layout]["lookup_table_forward_gbs"] = wbytes / (lut_ms * 1e-3) / 1e9
        log(f"decode {layout} ({scheme}): fused step {ms_step*1e3:.2f} us "
            f"({decode[layout]['fused_gbs']:.0f} GB/s), "
            f"two-launch step {ms_two*1e3:.2f} us, forward only {k_mean*1e3:.2f} us"
            + (f", lookup-table forward {lut_ms*1e3:.2f} us" if lut_ms is not None else ""))
        del copies
        torch.cuda.empty_cache()
    rows["decode_gemv"] = decode

    # ------------------------------------------------------------- ceilings
    # What the machine at hand reaches on the simplest kernels of each kind:
    # a streaming read of one 4 MiB buffer per launch (the decode layer's
    # weight bytes) over 128 rotating buffers, caches flushed; the same read
    # over 512 MiB in one launch; the graph cadence of empty launches; and
    # independent v_mfma_i32_32x32x32_i8 chains on register operands (dense
    # INT8 rate at the clock held under load). The read takes the best of a
    # few launch shapes.
    ceil = {}
    bufs = [torch.randint(0, 256, (4 << 20,), dtype=torch.uint8, device=dev) for _ in range(R)]
    best = None
    for blocks, unroll in ((256, 4), (512, 2), (1024, 1), (128, 8), (256, 2), (512, 4)):
        ms = graph_ms(lambda i, b=blocks, u=unroll: probe_read(bufs[i % R], b, u), R)
        if best is None or ms < best[0]:
            best = (ms, blocks, unroll)
    ceil["stream_read_4MiB"] = dict(ms=best[0], gbs=(4 << 20) / (best[0] * 1e-3) / 1e9,
                                    blocks=best[1], loads_in_flight=best[2],
                                    what="one 4 MiB buffer per launch, 128 rotating, cold caches")
    del bufs
    # the same over one 32 MiB buffer per launch (the 32768 x 4096 weight
    # stream below), 16 rotating buffers
    bufs = [torch.randint(0, 256, (32 << 20,), dtype=torch.uint8, device=dev) for _ in range(16)]
    best = None
    for blocks, unroll in ((1024, 2), (2048, 1), (512, 4), (1024, 4), (2048, 2)):
        ms = graph_ms(lambda i, b=blocks, u=unroll: probe_read(bufs[i % 16], b, u), 64)
        if best is None or ms < best[0]:
            best = (ms, blocks, unroll)
    ceil["stream_read_32MiB"] = dict(ms=best[0], gbs=(32 << 20) / (best[0] * 1e-3) / 1e9,
                                     blocks=best[1], loads_in_flight=best[2],
                                     what="one 32 MiB buffer per launch, 16 rotating, cold caches")
    del bufs
    big = torch.randint(0, 256, (512 << 20,), dtype=torch.uint8, device=dev)
    best = None
    for blocks, unroll in ((2048, 4), (4096, 2), (1024, 8), (8192, 1)):
        ms = graph_ms(lambda i, b=blocks, u=unroll: probe_read(big, b, u), 4)
        if best is None or ms < best[0]:
            best = (ms, blocks, unroll)
    ceil["stream_read_512MiB"] = dict(ms=best[0], gbs=(512 << 20) / (best[0] * 1e-3) / 1e9,
                                      blocks=best[1], loads_in_flight=best[2])
    del big
    ms = graph_ms(lambda i: probes.probe_empty(cur_stream()), 256)
    ceil["empty_launch_graph_us"] = ms * 1e3
    mf_blocks, mf_iters = 1024, 8000
    ms = graph_ms(lambda i: probes.probe_mfma_i8(mf_blocks, mf_iters,
                                                 ctypes.c_void_p(probe_out.data_ptr()),
                                                 cur_stream()), 1)
    mops = mf_blocks * 4 * mf_iters * 8 * 65536.0
    ceil["mfma_i8_loop"] = dict(ms=ms, tops=mops / (ms * 1e-3) / 1e12,
                                frac_of_peak=mops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS)
    rows["ceilings"] = ceil
    log(f"ceilings: 4 MiB read {ceil['stream_read_4MiB']['ms']*1e3:.2f} us "
        f"({ceil['stream_read_4MiB']['gbs']:.0f} GB/s), 32 MiB read "
        f"{ceil['stream_read_32MiB']['ms']*1e3:.2f} us ({ceil['stream_read_32MiB']['gbs']:.0f} GB/s), 512 MiB read "
        f"{ceil['stream_read_512MiB']['gbs']:.0f} GB/s, empty launch "
        f"{ceil['empty_launch_graph_us']:.2f} us, INT8 MFMA loop {ceil['mfma_i8_loop']['tops']:.0f} TOPS")
    torch.cuda.empty_cache()

    # Weight streaming at a size where launch latency no longer dominates:
    # one token against a 32768 x 4096 ternary matrix (32 MiB packed, the
    # shape of a vocabulary projection), 16 rotating copies.
    if want("stream"):
        ps = synth.make_problem(M=1, N=32768, K=4096, seed=9, dtype="bf16", outlier_frac=0.01)
        Ws = to_dev(ps.w_store, True)
        xs1 = to_dev(ps.x_store, True)
        ys = torch.empty((1, ps.N), dtype=torch.float32, device=dev)
        for layout, scheme, key in (("2bit", "ternary", "decode_stream_32768x4096"),
                                    ("1bit", "binary", "decode_stream_32768x4096_1bit")):
            pk, g = bl.bitlinear_pack_weights(Ws, layout, scheme)
            cps = [pk.clone() for _ in range(16)]
            f = lambda i, cps=cps, g=g, layout=layout: bl.bitlinear_linear(
                xs1, cps[i % 16], g, ps.N, layout, y=ys)
            ms = graph_ms(f, 64)
            alg = pk.numel() + 2 * ps.K + 4 + 4 * ps.N
            rows[key] = dict(ms=ms, alg_bytes=alg, gbs=alg / (ms * 1e-3) / 1e9,
                             frac_hbm=alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             frac_of_32MiB_read=(alg / (ms * 1e-3) / 1e9)
                             / ceil["stream_read_32MiB"]["gbs"])
            log(f"stream 32768x4096 {layout}: {ms*1e3:.2f} us = {alg/(ms*1e-3)/1e9:.0f} GB/s")
            del cps
        del Ws
        torch.cuda.empty_cache()

    # ------------------------------------------------------------------ pack
    if want("pack"):
        ws = torch.empty(bl.bitlinear_pack_workspace_bytes(p.N, p.K), dtype=torch.uint8, device=dev)
        pk = {}
        for layout in ("2bit", "base3", "1bit"):
            scheme = "binary" if layout == "1bit" else "ternary"
            packed = torch.empty((p.N, bl.bitlinear_packed_row_bytes(p.K, layout)),
                                 dtype=torch.uint8, device=dev)
            g = torch.empty(4, dtype=torch.float32, device=dev)[:1]
            f = lambda i, layout=layout, scheme=scheme, packed=packed, g=g: \
                bl.bitlinear_pack_weights(W, layout, scheme, packed=packed, gamma=g, workspace=ws)
            ms = graph_ms(f, 20)
            byt = 2 * p.N * p.K * 2 + packed.numel()  # W read by both passes + codes written
            pk[layout] = dict(ms=ms, gbs=byt / (ms * 1e-3) / 1e9)
            log(f"pack {layout}: {ms*1e3:.1f} us")
        rows["pack_decode_weights"] = pk

    # ------------------------------------------------------------- prefill
    if want("prefill"):
        log("prefill workload: generating inputs")
        q = synth.workload("prefill")
        Wp = to_dev(q.w_store, True)
        xp = to_dev(q.x_store, True)
        xq, sc = bl.bitlinear_quant_acts(xp)
        qa_ms = graph_ms(lambda i: bl.bitlinear_quant_acts(xp, xq=xq, scale=sc), 20)
        pre = {"quant_acts_ms": qa_ms,
               "quant_acts_gbs": (q.M * q.K * 3 + 4 * q.M) / (qa_ms * 1e-3) / 1e9}
        ops = 2.0 * q.M * q.N * q.K
        for layout in ("2bit", "base3", "1bit"):
            packed, gamma = bl.bitlinear_pack_weights(Wp, layout,
                                                      "binary" if layout == "1bit" else "ternary")
            y = torch.empty((q.M, q.N), dtype=torch.bfloat16, device=dev)
            f = lambda i, packed=packed, gamma=gamma, layout=layout, y=y: bl.bitlinear_forward(
                xq, sc, packed, gamma, q.N, q.K, layout, torch.bfloat16, y=y)
            ms = graph_ms(f, 10)
            pre[layout] = dict(gemm_ms=ms, tops=ops / (ms * 1e-3) / 1e12,
                               frac=ops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS,
                               frac_of_measured_mfma=ops / (ms * 1e-3) / 1e12 /
                               rows["ceilings"]["mfma_i8_loop"]["tops"])
            log(f"prefill {layout}: {ms*1e3:.1f} us = {pre[layout]['tops']:.0f} TOPS")
        rows["prefill_gemm"] = pre
        del Wp, xp, xq, sc
        torch.cuda.empty_cache()

    # ---------------------------------------------------------- block stack
    if want("block"):
        log("block stack: generating inputs")
        layers = []
        for i, (name, N, K) in enumerate(synth.BLOCK_LAYERS):
            pb = synth.block_layer(i, 1)
            packed, gamma = bl.bitlinear_pack_weights(to_dev(pb.w_store, True), "2bit")
            layers.append((name, N, K, packed, gamma))
        # Q, K and V read the same input: stacked into one packed matrix with
        # three gammas, they run as one launch
        rb4 = layers[0][3].shape[1]
        qkv = torch.empty((3 * 4096, rb4), dtype=torch.uint8, device=dev)
        qkv_g = torch.zeros(4, dtype=torch.float32, device=dev)
        for s_ in range(3):
            qkv[s_ * 4096:(s_ + 1) * 4096].copy_(layers[s_][3])
            qkv_g[s_:s_ + 1].copy_(layers[s_][4])
        blk = {}
        # one decode token through the block: four fused launches (quantise +
        # multiply each), Q|K|V stacked; 16 rotating copies (629 MB of codes)
        cps1 = [[(n, N, K, pk.clone() if c else pk, g) for (n, N, K, pk, g) in layers]
                for c in range(16)]
        qkvs1 = [qkv.clone() if c else qkv for c in range(16)]
        x1 = {K: to_dev(synth.make_problem(M=1, N=1, K=K, seed=77 + K, dtype="bf16").x_store, True)
              for K in (4096, 11008)}
        ys1 = [torch.empty((1, N), dtype=torch.bfloat16, device=dev) for (_, N, _, _, _) in layers]
        y1_qkv = torch.empty((1, 3 * 4096), dtype=torch.bfloat16, device=dev)

        def block1(i):
            c = i % len(cps1)
            bl.bitlinear_linear_segmented(x1[4096], qkvs1[c], qkv_g, (4096, 4096, 4096), "2bit",
                                          torch.bfloat16, y=y1_qkv)
            for j in (3, 4, 5):
                _, N, K, pk, g = cps1[c][j]
                bl.bitlinear_linear(x1[K], pk, g, N, "2bit", torch.bfloat16, y=ys1[j])

        ms = graph_ms(block1, 32)
        blk["M1"] = dict(ms_per_block=ms, tokens_per_s=1 / (ms * 1e-3),
                         weight_gbs=sum(l[3].numel() for l in layers) / (ms * 1e6),
                         launches=4)
        log(f"block M=1: {ms*1e3:.1f} us/block, four fused launches ({1/(ms*1e-3):.3g} tok/s, "
            f"{blk['M1']['weight_gbs']:.0f} GB/s of codes)")
        del cps1, qkvs1
        torch.cuda.empty_cache()
        for M in (16, 512):
            ncopy = 16 if M == 16 else 1
            cps = [[(n, N, K, pk.clone() if c else pk, g) for (n, N, K, pk, g) in layers]
                   for c in range(ncopy)]
            qkvs = [qkv.clone() if c else qkv for c in range(ncopy)]
            xin = {K: to_dev(synth.make_problem(M=M, N=1, K=K, seed=77 + K, dtype="bf16").x_store, True)
                   for K in (4096, 11008)}
            ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for (_, N, _, _, _) in layers]
            y_qkv = torch.empty((M, 3 * 4096), dtype=torch.bfloat16, device=dev)
            qbuf = {K: (torch.empty((M, K), dtype=torch.int8, device=dev),
                        torch.empty(M, dtype=torch.float32, device=dev)) for K in (4096, 11008)}

            def block_separate(i, cps=cps, xin=xin, ys=ys, qbuf=qbuf):
                # six launches; Q, K, V share one quantised input
                ls = cps[i % len(cps)]
                for j, (_, N, K, pk, g) in enumerate(ls):
                    if j in (0, 3, 4, 5):
                        bl.bitlinear_quant_acts(xin[K], xq=qbuf[K][0], scale=qbuf[K][1])
                    bl.bitlinear_forward(qbuf[K][0], qbuf[K][1], pk, g, N, K, "2bit",
                                         torch.bfloat16, y=ys[j])

            def block(i, cps=cps, qkvs=qkvs, xin=xin, ys=ys, qbuf=qbuf, y_qkv=y_qkv):
                # Q|K|V stacked (one launch), then O, up and down
                c = i % len(cps)
                xq4, sc4 = qbuf[4096]
                bl.bitlinear_quant_acts(xin[4096], xq=xq4, scale=sc4)
                bl.bitlinear_forward_segmented(xq4, sc4, qkvs[c], qkv_g, (4096, 4096, 4096), 4096,
                                               "2bit", torch.bfloat16, y=y_qkv)
                for j in (3, 4, 5):
                    _, N, K, pk, g = cps[c][j]
                    bl.bitlinear_quant_acts(xin[K], xq=qbuf[K][0], scale=qbuf[K][1])
                    bl.bitlinear_forward(qbuf[K][0], qbuf[K][1], pk, g, N, K, "2bit",
                                         torch.bfloat16, y=ys[j])

            n_rep = 32 if M == 16 else 8
            ms = graph_ms(block, n_rep)
            ms_sep = graph_ms(block_separate, n_rep)
            blk[f"M{M}"] = dict(ms_per_block=ms, tokens_per_s=M / (ms * 1e-3),
                                ms_per_block_six_launches=ms_sep)
            log(f"block M={M}: {ms*1e3:.1f} us/block with Q|K|V stacked ({M/(ms*1e-3):.3g} tok/s), "
                f"{ms_sep*1e3:.1f} us as six launches")
            del cps, qkvs
            torch.cuda.empty_cache()
        rows["block_stack"] = blk

    # -------------------------------------------------------- training step
    # Latent bf16 weights are re-quantised every step (absmean + 2-bit pack),
    # then activation quantisation, the INT8 forward GEMM and the two
    # straight-through-estimator backward products on the bf16 matrix cores.
    if want("train"):
        log("training step: generating inputs")
        t = synth.workload("train")
        Wt = to_dev(t.w_store, True)
        xt = to_dev(t.x_store, True)
        gyt = to_dev(t.grad_y_store, True)
        pk_t = torch.empty((t.N, bl.bitlinear_packed_row_bytes(t.K, "2bit")), dtype=torch.uint8,
                           device=dev)
        g_t = torch.empty(4, dtype=torch.float32, device=dev)[:1]
        ws_t = torch.empty(bl.bitlinear_pack_workspace_bytes(t.N, t.K), dtype=torch.uint8,
                           device=dev)
        xq_t = torch.empty((t.M, t.K), dtype=torch.int8, device=dev)
        sc_t = torch.empty(t.M, dtype=torch.float32, device=dev)
        y_t = torch.empty((t.M, t.N), dtype=torch.bfloat16, device=dev)
        gx_t = torch.empty((t.M, t.K), dtype=torch.float32, device=dev)
        gw_t = torch.empty((t.N, t.K), dtype=torch.float32, device=dev)
        parts = {
            "requant_pack": lambda i: bl.bitlinear_pack_weights(Wt, "2bit", packed=pk_t, gamma=g_t,
                                                                workspace=ws_t),
            "quant_acts": lambda i: bl.bitlinear_quant_acts(xt, xq=xq_t, scale=sc_t),
            "forward_int8": lambda i: bl.bitlinear_forward(xq_t, sc_t, pk_t, g_t, t.N, t.K, "2bit",
                                                           torch.bfloat16, y=y_t),
            "backward_input_bf16": lambda i: bl.bitlinear_backward_input(gyt, pk_t, g_t, t.K,
                                                                         grad_x=gx_t),
            "backward_weight_bf16": lambda i: bl.bitlinear_backward_weight(gyt, xt, grad_w=gw_t),
        }
        flop = 2.0 * t.M * t.N * t.K
        tr = {}
        for name, f in parts.items():
            tr[name + "_ms"] = graph_ms(f, 10)

        def train_step(i):
            for f in parts.values():
                f(i)

        tr["step_ms"] = graph_ms(train_step, 10)
        tr["forward_int8_tops"] = flop / (tr["forward_int8_ms"] * 1e-3) / 1e12
        tr["forward_int8_frac"] = tr["forward_int8_tops"] / INT8_PEAK_TOPS
        for name in ("backward_input_bf16", "backward_weight_bf16"):
            tf = flop / (tr[name + "_ms"] * 1e-3) / 1e12
            tr[name + "_tflops"] = tf
            tr[name + "_frac"] = tf / BF16_PEAK_TFLOPS
        tr["tokens_per_s"] = t.M / (tr["step_ms"] * 1e-3)
        # grad_x read from the other layouts' packed rows of the same weights,
        # and from fp32 grad_y (three bf16 pieces); grad_W from fp32 operands
        # (six piece products); beside the step, not in it
        var = {}
        for lay, sch in (("base3", "ternary"), ("1bit", "binary")):
            pk_l, g_l = bl.bitlinear_pack_weights(Wt, lay, sch)
            var[lay + "_ms"] = graph_ms(
                lambda i: bl.bitlinear_backward_input(gyt, pk_l, g_l, t.K, lay, grad_x=gx_t), 10)
            del pk_l, g_l
        gy32, x32 = gyt.float(), xt.float()
        var["fp32_grad_y_2bit_ms"] = graph_ms(
            lambda i: bl.bitlinear_backward_input(gy32, pk_t, g_t, t.K, grad_x=gx_t), 10)
        var["backward_weight_fp32_ms"] = graph_ms(
            lambda i: bl.bitlinear_backward_weight(gy32, x32, grad_w=gw_t), 10)
        del gy32, x32
        tr["backward_other_inputs"] = var
        rows["train_step_4096"] = tr
        log(f"training step: {tr['step_ms']*1e3:.0f} us/step (fwd {tr['forward_int8_ms']*1e3:.0f}, "
            f"bwd in {tr['backward_input_bf16_ms']*1e3:.0f}, bwd w {tr['backward_weight_bf16_ms']*1e3:.0f} us)")
        del Wt, xt, gyt, pk_t, xq_t, y_t, gx_t, gw_t
        torch.cuda.empty_cache()

    # ------------------------------------------------- bf16 comparison lines
    # What a GPU without ternary kernels runs: the same layers with dense bf16
    # weights through the vendor GEMM (torch linear -> hipBLASLt), and the vendor
    # dense INT8 GEMM on the prefill shape. Context for the ternary path's
    # numbers, not part of the path.
    if want("bf16_baseline"):
        log("bf16 dense baseline (torch linear)")
        base = {}
        # weights [N, K] as a linear layer stores them (2-D products only)
        F = torch.nn.functional
        Wd = torch.randn((p.N, p.K), device=dev).mul_(0.02).to(torch.bfloat16)
        nrot = 20  # 20 x 32 MiB: past the 256 MB Infinity Cache
        wds = [Wd.clone() for _ in range(nrot)]
        xd = xs[0]
        ms = graph_ms(lambda i: F.linear(xd, wds[i % nrot]), 2 * nrot)
        wb = p.N * p.K * 2
        base["decode_gemv_bf16"] = dict(ms=ms, weight_bytes=wb, gbs=wb / (ms * 1e-3) / 1e9,
                                        ternary_speedup=ms / decode["2bit"]["ms_per_step"])
        log(f"bf16 decode GEMV: {ms*1e3:.2f} us ({wb/(ms*1e-3)/1e9:.0f} GB/s), ternary fused "
            f"step is {base['decode_gemv_bf16']['ternary_speedup']:.2f}x faster")
        del wds
        q = synth.WORKLOADS["prefill"]
        xb = torch.randn((q["M"], q["K"]), device=dev).to(torch.bfloat16)
        Wb = torch.randn((q["N"], q["K"]), device=dev).mul_(0.02).to(torch.bfloat16)
        ms = graph_ms(lambda i: F.linear(xb, Wb), 10)
        ops = 2.0 * q["M"] * q["N"] * q["K"]
        base["prefill_gemm_bf16"] = dict(ms=ms, tflops=ops / (ms * 1e-3) / 1e12,
                                         frac=ops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS)
        if "prefill_gemm" in rows:
            base["prefill_gemm_bf16"]["ternary_speedup"] = ms / rows["prefill_gemm"]["2bit"]["gemm_ms"]
        log(f"bf16 prefill GEMM: {ms*1e3:.1f} us ({base['prefill_gemm_bf16']['tflops']:.0f} TFLOP/s)")
        # dense INT8 x INT8 -> INT32 on the same shape (torch._int_mm -> hipBLASLt)
        xi = torch.randint(-127, 128, (q["M"], q["K"]), dtype=torch.int8, device=dev)
        wi = torch.randint(-1, 2, (q["K"], q["N"]), dtype=torch.int8, device=dev)
        ms = graph_ms(lambda i: torch._int_mm(xi, wi), 10)
        base["prefill_gemm_int8_dense"] = dict(ms=ms, tops=ops / (ms * 1e-3) / 1e12,
                                               frac=ops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS)
        log(f"dense int8 prefill GEMM: {ms*1e3:.1f} us ({base['prefill_gemm_int8_dense']['tops']:.0f} TOPS)")
        rows["bf16_dense_baseline"] = base
        del xb, Wb, xi, wi
        torch.cuda.empty_cache()

    # --------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nthreads = oracle.num_threads()  # all host threads (OpenMP default)
        codes, _, gamma = oracle.ternary_codes(p.w)
        n = 0
        t0 = time.perf_counter()
        while True:
            xq_, s_, _ = oracle.quant_acts(p.x)
            acc_ = oracle.int_product(xq_, codes)
            oracle.epilogue(acc_, gamma, s_)
            n += 1
            if time.perf_counter() - t0 > args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        wb = decode["2bit"]["weight_bytes"]

        def median_ms(f, reps=3):
            ts = []
            for _ in range(reps):
                t1 = time.perf_counter()
                f()
                ts.append((time.perf_counter() - t1) * 1e3)
            return sorted(ts)[len(ts) // 2]

        def stages(prob):
            """Median of 3 runs of each stage of the pass on this problem."""
            g32 = oracle.absmean(prob.w)[0]
            cds = oracle.ternary_codes(prob.w)[0]
            xq1, s1, _ = oracle.quant_acts(prob.x)
            acc1 = oracle.int_product(xq1, cds)
            return {"absmean_ms": median_ms(lambda: oracle.absmean(prob.w)),
                    "ternarise_ms": median_ms(lambda: oracle.ternary_codes(prob.w, gamma=g32)),
                    "pack_2bit_ms": median_ms(lambda: oracle.pack(cds, "2bit")),
                    "quant_acts_ms": median_ms(lambda: oracle.quant_acts(prob.x)),
                    "int_product_ms": median_ms(lambda: oracle.int_product(xq1, cds)),
                    "epilogue_ms": median_ms(lambda: oracle.epilogue(acc1, g32, s1))}

        per_stage = {}
        tiny = synth.workload("tiny")
        for label, prob in (("tiny_M8_N256_K256_f32", tiny), ("decode_M1_N4096_K4096_bf16", p)):
            per_stage[label] = {}
            for th in (1, nthreads):
                oracle.set_num_threads(th)
                per_stage[label][f"threads_{th}"] = stages(prob)
        oracle.set_num_threads(nthreads)
        cpu = {"value": wb * n / dt / 1e9, "unit": "GB/s", "cores": nthreads,
               "kind": "oracle",
               "sample": f"{n} decode steps (quant_acts + int64 product + fp64 epilogue, M=1, "
                         f"K=N=4096) in {dt:.1f} s on {nthreads} threads; value = 2-bit weight "
                         "bytes per step / time. stages: each stage of the pass (median of 3) on "
                         "1 thread and on all threads, for the tiny and decode workloads",
               "host_cpus": os.cpu_count(),
               "stages": per_stage}
        log(f"cpu baseline: {cpu['value']:.3f} GB/s on {cpu['cores']} threads; decode stages "
            f"1 thread: {per_stage['decode_M1_N4096_K4096_bf16']['threads_1']}")

    # ------------------------------------------------------------ roofline
    d2 = decode["2bit"]
    roof = {"kernel": "linear_decode_kernel<2bit> (fused decode step, M=1, 4096x4096)",
            "bound": "hbm", "achieved": d2["fused_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": d2["fused_gbs"] / HBM_PEAK_GBS, "traffic": None,
            "alg_bytes_per_launch": d2["fused_alg_bytes"],
            "launch_ms_mean": d2["ms_per_step"],
            "measured_ceiling": {
                "what": "plain streaming read of one 4 MiB buffer per launch, 128 rotating "
                        "buffers, caches flushed (rows.ceilings.stream_read_4MiB)",
                "gbs": rows["ceilings"]["stream_read_4MiB"]["gbs"],
                "frac": d2["fused_gbs"] / rows["ceilings"]["stream_read_4MiB"]["gbs"]}}
    counters = os.path.join(ROOT, "profiles", "decode_fused_2bit_counters.json")
    if os.path.exists(counters):
        with open(counters) as f:
            c = json.load(f)
        src = os.path.join(ROOT, "ternary_weight_linear_bitlinear_amd", "csrc", "skinny.hip")
        if not os.path.exists(src):
            src = None
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] if src else None
        if sha and c.get("source_sha") == sha:
            roof["traffic"] = c.get("hbm_bytes_per_launch")

    ms = d2["ms_per_step"]
    line = {
        "metric": METRIC, "value": d2["weight_gbs"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "decode GEMV: M=1 token, W 4096x4096 bf16 ~N(0,0.02) quantised "
                               "once (absmean ternary, 2-bit packed), x bf16 ~N(0,1) + 1% +/-20 "
                               "outliers; step = per-token INT8 quantisation + integer product + "
                               "dequant (one fused launch); 128 rotating weight copies "
                               "(512 MiB), caches flushed before the timed replay",
                   "M": 1, "K": 4096, "N": 4096, "layout": "2bit", "out": "fp32"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
