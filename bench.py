#!/usr/bin/env python3
"""Throughput of the WNA16 quantized linear layer on one MI355X.

Headline (one JSON line on stdout): wq_gemm decode throughput at M = 1,
K = 5120, N = 17408, b = 5, 6 and 7, in TB/s of algorithmic bytes (packed codes
+ bf16 scales + activations + output).  One step = one wq_gemm call for each
of the three bit widths.  Weights are the tiled (repacked) layout, rotated over
--copies device copies per bit width so that the 256 MB Infinity Cache cannot
serve them; activations and workspaces are resident in HBM before timing.
The timed steps are captured in one HIP graph and replayed (12 us kernels would
otherwise measure Python launch overhead).

Also reported on the same line:
  roofline      the b = 6 decode kernel: algorithmic bytes per launch over its
                average duration (HIP events on the launch stream), against the
                8 TB/s HBM peak;
  cpu_baseline  the CPU oracle (fp64, OpenMP) on the same decode layers;
  decode_sweep  TB/s of wq_gemm at M = 4 and 16 on the same layer;
  prefill       TFLOP/s of wq_gemm at M = 4096 (up: K 5120 -> N 17408, down:
                K 17408 -> N 5120, b = 6) against the 2.5 PFLOP/s bf16 peak;
  w4a8          TOP/s of wq_gemm_a8 at M = 2048 / 8192 (K 5120, N 17408) against
                the 5.0 POPS int8 peak, with wq_gemm at b = 4 on the same shape;
  stack         the 64-layer mixed-bit (7 / 5 / 6) stack plus the 8-bit 248320 x
                5120 vocabulary head (9.98 GB of weights): M = 1 in TB/s, M = 512
                in TFLOP/s.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0
DECODE_N, DECODE_K = 17408, 5120
DECODE_BITS = (5, 6, 7)


def log(msg: str):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def algorithmic_bytes(M: int, N: int, K: int, b: int) -> int:
    return N * (K * b // 32) * 4 + N * (K // 128) * 2 + M * K * 2 + M * N * 2


class DecodeLayer:
    def __init__(self, b: int, copies: int, torch, wq, synth):
        w = synth.decode(M=1, b=b, N=DECODE_N, K=DECODE_K)
        self.b, self.w = b, w
        packed = wq.wq_pack(w.codes, b)
        packed_d = torch.from_numpy(packed.view(np.int32)).cuda()
        scales_d = torch.from_numpy(w.scales.view(np.int16)).cuda().view(torch.bfloat16)
        blob = wq.wq_repack(packed_d, scales_d, w.K, b)
        self.blobs = [blob] + [blob.clone() for _ in range(copies - 1)]
        del packed_d, scales_d
        self.A = torch.from_numpy(w.A.view(np.int16)).cuda().view(torch.bfloat16)
        self.Y = torch.empty((1, w.N), dtype=torch.bfloat16, device="cuda")
        nbytes = wq.wq_workspace_bytes(wq.WQ_OP_GEMM, 1, w.N, w.K, b)
        self.ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        self.bytes = algorithmic_bytes(1, w.N, w.K, b)

    def call(self, wq, i: int):
        wq.wq_gemm(self.A, self.blobs[i % len(self.blobs)], wq.WQ_LAYOUT_TILED, None, self.w.N,
                   self.b, Y=self.Y, ws=self.ws)


def graph_time(torch, fn, reps: int, warmup: int, warm_s: float = 0.0) -> float:
    """Capture fn() once, replay warmup + reps times; seconds per replay.
    warm_s > 0: after the warmup replays, keep replaying (untimed) for about
    warm_s seconds first.  A GEMM of ~1 ms measured right after the light
    decode benches ran up to 20% slower over its first ten replays than
    later in the same process (the shader clock rises under sustained
    matrix load)."""
    fn()  # first call outside capture (device checks, lazy init)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    if warm_s > 0:
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        one = max(time.perf_counter() - t0, 1e-6)
        for _ in range(int(warm_s / one) + 1):
            g.replay()
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3 / reps


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(oracle, synth, target_s: float):
    """The oracle on the same decode step (b = 5, 6, 7 at M = 1), repeated
    until target_s seconds of CPU time have passed; then, once each, a
    64-row slice of the prefill layer (M = 64 of the M = 4096 up shape, K
    5120 -> N 17408, b = 6) and of the W4A8 layer (M = 64, K 5120 -> N 17408,
    b = 4), whose per-row rates stand for the full layers (the oracle's cost is
    linear in M)."""
    layers = []
    for b in DECODE_BITS:
        w = synth.decode(M=1, b=b, N=DECODE_N, K=DECODE_K)
        layers.append((w, oracle.pack(w.codes, b)))
    steps, t0 = 0, time.perf_counter()
    while True:
        for w, p in layers:
            oracle.wna16(w.A, p, w.scales, w.b)
        steps += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    total = sum(algorithmic_bytes(1, w.N, w.K, w.b) for w, _ in layers)
    out = {"value": total * steps / el / 1e12, "unit": "TB/s", "cores": oracle.num_threads(),
           "cores_available": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
           "kind": "oracle",
           "sample": "%d full decode steps (M=1, K=5120, N=17408, b=5/6/7) in %.1f s, fp64"
                     % (steps, el)}
    w = synth.prefill(M=64, N=DECODE_N, K=DECODE_K, b=6)
    p = oracle.pack(w.codes, 6)
    t0 = time.perf_counter()
    oracle.wna16(w.A, p, w.scales, 6)
    el = time.perf_counter() - t0
    out["prefill_slice"] = {"TFLOP/s": 2.0 * 64 * w.N * w.K / el / 1e12, "s": el,
                            "sample": "64 rows of the M=4096 prefill layer (K=5120, N=17408, "
                                      "b=6), fp64; the rate stands for all 4096 rows"}
    w = synth.w4a8(M=64)
    p = oracle.pack(w.codes, 4)
    t0 = time.perf_counter()
    oracle.w4a8(w.A, p, w.scales)
    el = time.perf_counter() - t0
    out["w4a8_slice"] = {"TOP/s": 2.0 * 64 * w.N * w.K / el / 1e12, "s": el,
                         "sample": "64 rows of the W4A8 layer (K=%d, N=%d, b=4): int8 "
                                   "activation quantization and integer group sums; the rate "
                                   "stands for M=2048 and 8192" % (w.K, w.N)}
    return out


def bench_prefill(torch, wq, synth, reps: int):
    out = {}
    for name, (K, N) in (("up", (5120, 17408)), ("down", (17408, 5120))):
        w = synth.prefill(M=4096, N=N, K=K, b=6)
        packed = wq.wq_pack(w.codes, 6)
        blob = wq.wq_repack(torch.from_numpy(packed.view(np.int32)).cuda(),
                            torch.from_numpy(w.scales.view(np.int16)).cuda().view(torch.bfloat16),
                            K, 6)
        A = torch.from_numpy(w.A.view(np.int16)).cuda().view(torch.bfloat16)
        Y = torch.empty((w.M, N), dtype=torch.bfloat16, device="cuda")

        def fn():
            wq.wq_gemm(A, blob, wq.WQ_LAYOUT_TILED, None, N, 6, Y=Y)

        t = graph_time(torch, fn, reps, 2, warm_s=0.05)
        tf = 2.0 * w.M * N * K / t / 1e12
        out[name] = {"M": w.M, "N": N, "K": K, "b": 6, "ms": t * 1e3, "TFLOP/s": tf,
                     "frac_of_peak": tf / BF16_PEAK_TFLOPS}
        del blob, A, Y
    return out


def bench_embed(torch, wq, synth, reps: int):
    """Quantized embedding gather: 4096 token ids from the 248,320 x 5,120
    table at b = 6 and 8 (dense layout).  The table is filled on the device
    from a seeded generator (any words are a valid dense table; the values do
    not change the gather's timing); 8 output buffers rotate so the written
    rows (42 MB each) do not stay in the 256 MB Infinity Cache.  Algorithmic
    bytes: per token the row's codes K*b/8 and scales 2K/128 read, the id
    read, 2K written."""
    V, K, T, copies = synth.EMBED_VOCAB, synth.EMBED_HIDDEN, 4096, 8
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    ids = torch.from_numpy(synth.embed_ids(T, V)).cuda()
    out = {}
    for b in (6, 8):
        words = torch.randint(-(1 << 31), 1 << 31, (V, K * b // 32), dtype=torch.int32,
                              device="cuda", generator=gen)
        scales = (torch.randn((V, K // 128), device="cuda", generator=gen) * 0.01).to(torch.bfloat16)
        Ys = [torch.empty((T, K), dtype=torch.bfloat16, device="cuda") for _ in range(copies)]

        def fn():
            for Y in Ys:
                wq.wq_embed(ids, words, scales, K, b, Y=Y)

        t = graph_time(torch, fn, reps, 2) / copies
        byts = T * (K * b // 8 + 2 * K // 128 + 8 + 2 * K)
        out["b%d" % b] = {"T": T, "V": V, "K": K, "us": t * 1e6, "bytes": byts,
                          "GB/s": byts / t / 1e9, "frac_of_hbm_peak": byts / t / 1e9 / HBM_PEAK_GBS}
        del words, scales, Ys
    return out


def bench_zero_points(torch, wq, synth, reps: int, copies: int):
    """Zero points (b = 4, 8) and per-channel scales against the symmetric
    kernels on the same layer (K 5120 -> N 17408, tiled): decode M = 1 with
    rotating weight copies, prefill M = 4096."""
    K, N = 5120, 17408
    rng = np.random.default_rng(9)
    out = {}
    for b in (4, 8):
        codes = synth.draw_codes(rng, N, K, b)
        scales = synth.draw_scales_halfnormal_signed(rng, N, K // 128)
        z = torch.from_numpy(rng.integers(0, 1 << b, size=(N, K // 128), dtype=np.uint8)).cuda()
        words = torch.from_numpy(wq.wq_pack(codes, b).view(np.int32)).cuda()
        s_d = torch.from_numpy(scales.view(np.int16)).cuda().view(torch.bfloat16)
        blobs = [wq.wq_repack(words, s_d, K, b) for _ in range(copies)]
        s1 = s_d[:, :1].contiguous()
        blobs_pc = [wq.wq_repack(words, s1, K, b, group=K) for _ in range(copies)]
        byts = algorithmic_bytes(1, N, K, b)
        A1 = torch.from_numpy(synth.draw_act(rng, 1, K).view(np.int16)).cuda().view(torch.bfloat16)
        Y1 = torch.empty((1, N), dtype=torch.bfloat16, device="cuda")
        res = {}
        for name, bl, kw in (("symmetric", blobs, {}), ("zero_points", blobs, {"zeros": z}),
                             ("per_channel", blobs_pc, {"group": K})):
            it = [0]

            def f(bl=bl, kw=kw):
                wq.wq_gemm(A1, bl[it[0] % copies], wq.WQ_LAYOUT_TILED, None, N, b, Y=Y1, **kw)
                it[0] += 1

            t = graph_time(torch, lambda: [f() for _ in range(copies)], reps, 2) / copies
            res["decode_M1_" + name] = {"us": t * 1e6, "TB/s": byts / t / 1e12}
        A = torch.from_numpy(synth.draw_act(rng, 4096, K).view(np.int16)).cuda().view(torch.bfloat16)
        Y = torch.empty((4096, N), dtype=torch.bfloat16, device="cuda")
        for name, kw in (("symmetric", {}), ("zero_points", {"zeros": z})):
            t = graph_time(torch, lambda: wq.wq_gemm(A, blobs[0], wq.WQ_LAYOUT_TILED, None, N, b,
                                                     Y=Y, **kw), max(2, reps // 4), 1, warm_s=0.05)
            res["prefill_M4096_" + name] = {"ms": t * 1e3,
                                            "TFLOP/s": 2.0 * 4096 * N * K / t / 1e12}
        out["b%d" % b] = res
        del blobs, blobs_pc, A, Y
    return out


def bench_grouped(torch, wq, synth, reps: int):
    """Grouped (mixture-of-experts) layer, synthetic: 64 experts of
    K 5120 -> N 2048 at b = 6, top-4 routing.  Decode: one token (4 experts,
    one row each; algorithmic bytes = the 4 experts' weights), 16 calls with
    different routings per timed replay so the experts read (~500 MB) do
    not stay in the Infinity Cache; prefill: 1024 tokens (4096 rows, uniform
    random routing; 2 * rows * N * K flops)."""
    E, N, K, b, topk = 64, 2048, 5120, 6, 4
    rng = np.random.default_rng(10)
    eb = wq.wq_repacked_bytes(wq.WQ_LAYOUT_TILED, N, K, b)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(10)
    words = torch.randint(-(1 << 31), 1 << 31, (N, K * b // 32), dtype=torch.int32, device="cuda",
                          generator=gen)
    W = torch.empty(E * eb, dtype=torch.uint8, device="cuda")
    for e in range(E):  # distinct scales per expert, codes shared (values do not change timing)
        s = (torch.randn((N, K // 128), device="cuda", generator=gen) * 0.01).to(torch.bfloat16)
        wq.wq_repack(words, s, K, b, out=W[e * eb:(e + 1) * eb])
    out = {}
    for name, T, calls in (("decode_T1", 1, 16), ("prefill_T1024", 1024, 1)):
        offs = []
        for _ in range(calls):
            experts = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(T)])
            sizes = np.bincount(experts.ravel(), minlength=E)
            offs.append(np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64))
        rows = T * topk
        A = torch.from_numpy(synth.draw_act(rng, rows, K).view(np.int16)).cuda().view(torch.bfloat16)
        Y = torch.empty((rows, N), dtype=torch.bfloat16, device="cuda")

        def fn():
            for off in offs:
                wq.wq_gemm_grouped(A, W, eb, off, N, b, Y=Y)

        t = graph_time(torch, fn, reps, 2, warm_s=0.05) / calls
        active = float(np.mean([(np.diff(off) > 0).sum() for off in offs]))
        byts = active * algorithmic_bytes(0, N, K, b) + rows * K * 2 + rows * N * 2
        out[name] = {"experts": E, "active": active, "rows": rows, "us": t * 1e6,
                     "TB/s": byts / t / 1e12, "TFLOP/s": 2.0 * rows * N * K / t / 1e12}
    del W
    return out


def hip_ceilings(torch, quick: bool):
    """Practical ceilings measured with the committed measurement kernels of
    libwq_ceilings.so (csrc_ceilings/ceilings.hip):
      stream_read  a plain 128-bit streaming read over the b = 6 decode
                   layer's algorithmic byte count, rotating 8 buffers (past
                   the 256 MB Infinity Cache), the best of a sweep over
                   workgroup counts and loads in flight per lane;
      mfma_bf16    back-to-back v_mfma_f32_32x32x16_bf16, 2 waves per SIMD;
      mfma_i8      the same with v_mfma_i32_16x16x64_i8;
      mfma_fold    v_mfma_f32_32x32x16_bf16 / v_mfma_i32_32x32x32_i8 with NV
                   vector-ALU fold operations after each MFMA (2 waves per
                   SIMD, two chains): what a GEMM that folds per-group sums
                   into fp32 keeps of the matrix-core rate."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "weight_only_bit_wq_amd", "libwq_ceilings.so"))
    P, L, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.wqc_stream_read.argtypes = [P, L, I, I, P, P]
    lib.wqc_mfma_loop.argtypes = [I, I, I, I, P, P]
    lib.wqc_mfma_fold.argtypes = [I, I, I, I, P, P]
    for f in (lib.wqc_stream_read, lib.wqc_mfma_loop, lib.wqc_mfma_fold):
        f.restype = I

    def st():
        return P(torch.cuda.current_stream().cuda_stream)

    def check(rc, what):
        if rc != 0:
            raise RuntimeError("%s failed: hipError %d" % (what, rc))

    out = {}
    nbytes = algorithmic_bytes(1, DECODE_N, DECODE_K, 6) // 16 * 16
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(8)]
    for bb in bufs:
        bb.fill_(1)
    # Quick: the best configurations of the full sweep on MI355X.
    sweep = ((512, 8), (1024, 8), (1024, 2)) if quick else \
        tuple((w, u) for w in (256, 512, 1024, 2048, 4096, 8192) for u in (1, 2, 4, 8))
    sink = torch.empty(max(w for w, _ in sweep) * 256, dtype=torch.int32, device="cuda")
    table, best = [], None
    for wgs, unroll in sweep:
        def fn(wgs=wgs, unroll=unroll):
            for i in range(32):
                check(lib.wqc_stream_read(P(bufs[i % 8].data_ptr()), nbytes, wgs, unroll,
                                          P(sink.data_ptr()), st()), "wqc_stream_read")
        t = graph_time(torch, fn, 3, 1) / 32
        row = {"workgroups": wgs, "loads_in_flight": unroll, "us": t * 1e6,
               "TB/s": nbytes / t / 1e12}
        table.append(row)
        if best is None or row["TB/s"] > best["TB/s"]:
            best = row
    out["stream_read"] = dict(best, bytes=nbytes, frac_of_hbm_peak=best["TB/s"] * 1e3 / HBM_PEAK_GBS)
    if not quick:
        out["stream_read"]["sweep"] = table
    del bufs
    # MFMA-only loops: 2 or 4 waves per SIMD (512 or 1024 workgroups of 4
    # waves), 4 or 8 accumulator chains per wave; the best of each
    # instruction is the ceiling.
    instrs = ((0, "v_mfma_f32_32x32x16_bf16", 32 * 32 * 16, "bf16"),
              (1, "v_mfma_f32_16x16x32_bf16", 16 * 16 * 32, "bf16"),
              (2, "v_mfma_i32_16x16x64_i8", 16 * 16 * 64, "i8"),
              (3, "v_mfma_i32_32x32x32_i8", 32 * 32 * 32, "i8"))
    configs = ((1024, 8), (1024, 4)) if quick else ((512, 4), (512, 8), (1024, 4), (1024, 8))
    fs = torch.empty(1024 * 256, dtype=torch.float32, device="cuda")
    for op, name, mnk, kind in instrs:
        best = None
        for wgs, chains in configs:
            iters = 1000
            t = graph_time(torch, lambda: check(lib.wqc_mfma_loop(op, chains, wgs, iters,
                                                                  P(fs.data_ptr()), st()),
                                                "wqc_mfma_loop"), 5, 1)
            rate = wgs * 4 * iters * chains * 2 * mnk / t / 1e12
            peak = BF16_PEAK_TFLOPS if kind == "bf16" else INT8_PEAK_TOPS
            row = {"instr": name, "workgroups": wgs, "chains": chains, "us": t * 1e6,
                   ("TFLOP/s" if kind == "bf16" else "TOP/s"): rate, "frac_of_peak": rate / peak}
            if best is None or row["frac_of_peak"] > best["frac_of_peak"]:
                best = row
        out["mfma_" + name.split("_", 2)[2]] = best
    # MFMA with per-MFMA vector-ALU folds, 512 workgroups of 4 waves.
    fold = []
    for op, name, mnk, kind in ((0, "v_mfma_f32_32x32x16_bf16", 32 * 32 * 16, "bf16"),
                                (1, "v_mfma_i32_32x32x32_i8", 32 * 32 * 32, "i8")):
        for nv in ((0, 4, 8) if quick else (0, 2, 4, 6, 8, 10, 12)):
            wgs, iters = 512, 500
            t = graph_time(torch, lambda: check(lib.wqc_mfma_fold(op, nv, wgs, iters,
                                                                  P(fs.data_ptr()), st()),
                                                "wqc_mfma_fold"), 5, 1)
            rate = wgs * 4 * iters * 16 * 2 * mnk / t / 1e12
            peak = BF16_PEAK_TFLOPS if kind == "bf16" else INT8_PEAK_TOPS
            fold.append({"instr": name, "valu_per_mfma": nv, "us": t * 1e6,
                         "frac_of_peak": rate / peak})
    out["mfma_fold"] = fold
    return out


def ceilings_run(torch):
    """The committed ceiling kernels with their full streaming-read sweep,
    plus torch's own kernels for comparison, timed eagerly with events: an
    HBM read (torch.sum over a 4 GiB buffer) and copy (2 GiB to 2 GiB, read
    + write bytes), torch's bf16 GEMM (hipBLASLt) at the prefill shapes
    with the weight stored [N, K] as the library's is (Y = A @ W^T), and
    torch's int8 GEMM (torch._int_mm, int32 out) at the W4A8 shapes.  The
    GEMMs run for ~50 ms untimed first (the shader clock rises under
    sustained matrix load)."""
    def eager(fn, reps, warm_s=0.0):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warm_s:
            fn()
            torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            fn()
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / 1e3 / reps

    out = hip_ceilings(torch, quick=False)
    big = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
    t = eager(lambda: big.sum(), 20)
    out["torch_hbm_read"] = {"bytes": big.numel() * 4, "us": t * 1e6,
                             "TB/s": big.numel() * 4 / t / 1e12,
                             "frac_of_hbm_peak": big.numel() * 4 / t / 1e9 / HBM_PEAK_GBS}
    half = big.view(2, -1)
    t = eager(lambda: half[1].copy_(half[0]), 20)
    out["torch_hbm_copy"] = {"bytes": big.numel() * 4, "us": t * 1e6,
                             "TB/s": big.numel() * 4 / t / 1e12,
                             "frac_of_hbm_peak": big.numel() * 4 / t / 1e9 / HBM_PEAK_GBS}
    del big, half
    for name, (K, N) in (("torch_gemm_bf16_up", (5120, 17408)),
                         ("torch_gemm_bf16_down", (17408, 5120))):
        A = torch.randn((4096, K), device="cuda").to(torch.bfloat16)
        W = torch.randn((N, K), device="cuda").to(torch.bfloat16)
        t = eager(lambda: torch.matmul(A, W.t()), 20, warm_s=0.05)
        tf = 2.0 * 4096 * N * K / t / 1e12
        out[name] = {"M": 4096, "N": N, "K": K, "us": t * 1e6, "TFLOP/s": tf,
                     "frac_of_peak": tf / BF16_PEAK_TFLOPS}
        del A, W
    K, N = 5120, 17408
    for M in (2048, 8192):
        A = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda")
        W = torch.randint(-128, 128, (N, K), dtype=torch.int8, device="cuda")
        try:
            t = eager(lambda: torch._int_mm(A, W.t()), 20, warm_s=0.05)
        except RuntimeError as e:  # not every build has an int8 GEMM
            out["torch_int_mm_M%d" % M] = {"error": str(e).splitlines()[0][:200]}
        else:
            top = 2.0 * M * N * K / t / 1e12
            out["torch_int_mm_M%d" % M] = {"M": M, "N": N, "K": K, "us": t * 1e6, "TOP/s": top,
                                           "frac_of_int8_peak": top / INT8_PEAK_TOPS}
        del A, W
    return out


def bench_decode_sweep(torch, wq, synth, reps: int, copies: int):
    """wq_gemm at M = 4 and 16 on the decode layer (K 5120 -> N 17408), b = 5,
    6, 7, in TB/s of algorithmic bytes; rotating weight copies as in the
    headline step."""
    out = {}
    for b in DECODE_BITS:
        w = synth.decode(M=16, b=b, N=DECODE_N, K=DECODE_K)
        packed = wq.wq_pack(w.codes, b)
        packed_d = torch.from_numpy(packed.view(np.int32)).cuda()
        scales_d = torch.from_numpy(w.scales.view(np.int16)).cuda().view(torch.bfloat16)
        blob = wq.wq_repack(packed_d, scales_d, w.K, b)
        blobs = [blob] + [blob.clone() for _ in range(copies - 1)]
        del packed_d, scales_d
        for M in (4, 16):
            A = torch.from_numpy(np.ascontiguousarray(w.A[:M]).view(np.int16)).cuda().view(torch.bfloat16)
            Y = torch.empty((M, w.N), dtype=torch.bfloat16, device="cuda")
            nb = wq.wq_workspace_bytes(wq.WQ_OP_GEMM, M, w.N, w.K, b)
            ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device="cuda")
            n = 64

            def fn():
                for i in range(n):
                    wq.wq_gemm(A, blobs[i % copies], wq.WQ_LAYOUT_TILED, None, w.N, b, Y=Y, ws=ws)

            t = graph_time(torch, fn, reps, 1) / n
            byts = algorithmic_bytes(M, w.N, w.K, b)
            out["b%d_M%d" % (b, M)] = {"us": t * 1e6, "TB/s": byts / t / 1e12,
                                      "frac_of_hbm_peak": byts / t / 1e9 / HBM_PEAK_GBS}
        del blobs, blob
    return out


# One GPU's shard of the decode layer under 8-way tensor parallelism
# (column-parallel up projection: N / 8; row-parallel down projection: K / 8).
SHARD_SHAPES = (("up_N2176", 5120, 2176), ("down_K2176", 2176, 5120))


def bench_shards(torch, wq, synth, reps: int, copies: int):
    """The b = 6 layer at one shard's shape of an 8-way split: decode M = 1
    (rotating weight copies) in TB/s of algorithmic bytes and prefill
    M = 4096 in TFLOP/s.  Only the kernels: the all-reduce of the
    row-parallel partial sums is not part of the library."""
    out = {}
    b = 6
    rng = np.random.default_rng(11)
    for name, K, N in SHARD_SHAPES:
        codes = synth.draw_codes(rng, N, K, b)
        scales = synth.draw_scales_halfnormal_signed(rng, N, K // 128)
        words = torch.from_numpy(wq.wq_pack(codes, b).view(np.int32)).cuda()
        s_d = torch.from_numpy(scales.view(np.int16)).cuda().view(torch.bfloat16)
        blobs = [wq.wq_repack(words, s_d, K, b) for _ in range(copies)]
        A1 = torch.from_numpy(synth.draw_act(rng, 1, K).view(np.int16)).cuda().view(torch.bfloat16)
        Y1 = torch.empty((1, N), dtype=torch.bfloat16, device="cuda")
        ws1 = torch.zeros(max(wq.wq_workspace_bytes(wq.WQ_OP_GEMM, 1, N, K, b), 256),
                          dtype=torch.uint8, device="cuda")
        n = 64

        def fn():
            for i in range(n):
                wq.wq_gemm(A1, blobs[i % copies], wq.WQ_LAYOUT_TILED, None, N, b, Y=Y1, ws=ws1)

        t = graph_time(torch, fn, reps, 1) / n
        byts = algorithmic_bytes(1, N, K, b)
        res = {"K": K, "N": N, "b": b,
               "decode_M1": {"us": t * 1e6, "TB/s": byts / t / 1e12,
                             "frac_of_hbm_peak": byts / t / 1e9 / HBM_PEAK_GBS}}
        A = torch.from_numpy(synth.draw_act(rng, 4096, K).view(np.int16)).cuda().view(torch.bfloat16)
        Y = torch.empty((4096, N), dtype=torch.bfloat16, device="cuda")
        ws = torch.zeros(max(wq.wq_workspace_bytes(wq.WQ_OP_GEMM, 4096, N, K, b), 256),
                         dtype=torch.uint8, device="cuda")
        t = graph_time(torch, lambda: wq.wq_gemm(A, blobs[0], wq.WQ_LAYOUT_TILED, None, N, b, Y=Y,
                                                 ws=ws), max(2, reps // 2), 1, warm_s=0.05)
        tf = 2.0 * 4096 * N * K / t / 1e12
        res["prefill_M4096"] = {"us": t * 1e6, "TFLOP/s": tf, "frac_of_peak": tf / BF16_PEAK_TFLOPS}
        out[name] = res
        del blobs, A, Y, ws, ws1
    return out


def bench_w4a8(torch, wq, synth, reps: int):
    out = {}
    w0 = synth.w4a8(M=16)
    packed = wq.wq_pack(w0.codes, 4)
    blob = wq.wq_repack(torch.from_numpy(packed.view(np.int32)).cuda(),
                        torch.from_numpy(w0.scales.view(np.int16)).cuda().view(torch.bfloat16),
                        w0.K, 4)
    rng = np.random.default_rng(3)
    for M in (2048, 8192):
        A_bits = synth.draw_act(rng, M, w0.K, outlier_frac=0.01)
        A = torch.from_numpy(A_bits.view(np.int16)).cuda().view(torch.bfloat16)
        Y = torch.empty((M, w0.N), dtype=torch.bfloat16, device="cuda")
        ws = torch.zeros(wq.wq_workspace_bytes(wq.WQ_OP_GEMM_A8, M, w0.N, w0.K, 4),
                         dtype=torch.uint8, device="cuda")

        def f8():
            wq.wq_gemm_a8(A, blob, wq.WQ_LAYOUT_TILED, None, w0.N, 4, Y=Y, ws=ws)

        def f16():
            wq.wq_gemm(A, blob, wq.WQ_LAYOUT_TILED, None, w0.N, 4, Y=Y)

        t8 = graph_time(torch, f8, reps, 2, warm_s=0.05)
        t16 = graph_time(torch, f16, reps, 2, warm_s=0.05)
        ops = 2.0 * M * w0.N * w0.K
        out["M%d" % M] = {"ms": t8 * 1e3, "TOP/s": ops / t8 / 1e12,
                          "frac_of_int8_peak": ops / t8 / 1e12 / INT8_PEAK_TOPS,
                          "wna16_b4_ms": t16 * 1e3, "speedup_vs_wna16_b4": t16 / t8}
        del A, Y, ws
    # W8A8: 8-bit codes of the same shape, int8 activations, against WNA16 b = 8.
    M = 2048
    codes8 = synth.draw_codes(np.random.default_rng(8), w0.N, w0.K, 8)
    blob8 = wq.wq_repack(torch.from_numpy(wq.wq_pack(codes8, 8).view(np.int32)).cuda(),
                         torch.from_numpy(w0.scales.view(np.int16)).cuda().view(torch.bfloat16),
                         w0.K, 8)
    A = torch.from_numpy(synth.draw_act(rng, M, w0.K, outlier_frac=0.01).view(np.int16)).cuda() \
        .view(torch.bfloat16)
    Y = torch.empty((M, w0.N), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(wq.wq_workspace_bytes(wq.WQ_OP_GEMM_A8, M, w0.N, w0.K, 8),
                     dtype=torch.uint8, device="cuda")
    t8 = graph_time(torch, lambda: wq.wq_gemm_a8(A, blob8, wq.WQ_LAYOUT_TILED, None, w0.N, 8,
                                                 Y=Y, ws=ws), reps, 2, warm_s=0.05)
    t16 = graph_time(torch, lambda: wq.wq_gemm(A, blob8, wq.WQ_LAYOUT_TILED, None, w0.N, 8, Y=Y),
                     reps, 2, warm_s=0.05)
    ops = 2.0 * M * w0.N * w0.K
    out["W8A8_M%d" % M] = {"ms": t8 * 1e3, "TOP/s": ops / t8 / 1e12,
                           "frac_of_int8_peak": ops / t8 / 1e12 / INT8_PEAK_TOPS,
                           "wna16_b8_ms": t16 * 1e3, "speedup_vs_wna16_b8": t16 / t8}
    del A, Y, ws, blob8
    return out


CAL_BYTES = 64 << 20
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "decode_b6_m1_hbm_traffic.md")
DECODE_SOURCES = ("weight_only_bit_wq_amd/csrc/wq_decode_kernel.h",
                  "weight_only_bit_wq_amd/csrc/wq_device.h",
                  "weight_only_bit_wq_amd/csrc/wq_decode.hip")


def decode_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the b = 6 decode kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().split()[0]
    if vals.get("source_hash") != decode_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def pmc_run(torch, wq, synth, copies: int):
    """Kernels for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE: the b = 6 decode
    kernel, then two single-purpose kernels of known size (a 64 MiB fill writes
    64 MiB, a 64 MiB sum reads 64 MiB) to scale the counters."""
    l6 = DecodeLayer(6, copies, torch, wq, synth)
    for i in range(16):
        l6.call(wq, i)
    torch.cuda.synchronize()
    bufs = [torch.empty(CAL_BYTES // 4, dtype=torch.float32, device="cuda") for _ in range(copies)]
    out = torch.empty((), dtype=torch.float32, device="cuda")
    for i in range(16):
        bufs[i % copies].fill_(1.0)
    torch.cuda.synchronize()
    for i in range(16):
        torch.sum(bufs[i % copies], dim=0, out=out)
    torch.cuda.synchronize()
    log("pmc run done: decode b=6 M=1 x16 (%d algorithmic bytes each); fill x16 and sum x16 "
        "of %d bytes; decode source hash %s" % (l6.bytes, CAL_BYTES, decode_source_hash()))


def pmc_layer_run(torch, wq, synth, M: int):
    """Kernels for rocprofv3 --pmc activity counters: three calls of the
    K 5120 -> N 17408, b = 6 layer at batch M (the first one warms the
    caches)."""
    K, N = 5120, 17408
    w = synth.prefill(M=M, N=N, K=K, b=6) if M > 16 else synth.decode(M=M, b=6, N=N, K=K)
    packed = wq.wq_pack(w.codes, 6)
    blob = wq.wq_repack(torch.from_numpy(packed.view(np.int32)).cuda(),
                        torch.from_numpy(w.scales.view(np.int16)).cuda().view(torch.bfloat16), K, 6)
    A = torch.from_numpy(w.A.view(np.int16)).cuda().view(torch.bfloat16)
    Y = torch.empty((w.M, N), dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        wq.wq_gemm(A, blob, wq.WQ_LAYOUT_TILED, None, N, 6, Y=Y)
    torch.cuda.synchronize()
    log("pmc layer run done: M=%d K=5120 N=17408 b=6 x3" % M)


def pmc_a8_run(torch, wq, synth, M: int):
    """Kernels for rocprofv3 --pmc activity counters: three calls of the W4A8
    layer (K 5120 -> N 17408, b = 4) at batch M (the first one warms the
    caches)."""
    w = synth.w4a8(M=M)
    packed = wq.wq_pack(w.codes, 4)
    blob = wq.wq_repack(torch.from_numpy(packed.view(np.int32)).cuda(),
                        torch.from_numpy(w.scales.view(np.int16)).cuda().view(torch.bfloat16),
                        w.K, 4)
    A = torch.from_numpy(w.A.view(np.int16)).cuda().view(torch.bfloat16)
    Y = torch.empty((M, w.N), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(wq.wq_workspace_bytes(wq.WQ_OP_GEMM_A8, M, w.N, w.K, 4), dtype=torch.uint8,
                     device="cuda")
    for _ in range(3):
        wq.wq_gemm_a8(A, blob, wq.WQ_LAYOUT_TILED, None, w.N, 4, Y=Y, ws=ws)
    torch.cuda.synchronize()
    log("pmc a8 run done: M=%d K=%d N=%d b=4 x3" % (M, w.K, w.N))


def bench_stack(torch, wq, reps: int):
    """The 64-layer mixed-bit stack + 8-bit head: M = 1 (HBM-bound, TB/s of
    algorithmic bytes) and M = 512 (TFLOP/s).  One forward = 129 wq_gemm calls,
    captured in one graph."""
    from weight_only_bit_wq_amd import synth
    from weight_only_bit_wq_amd.stack import Stack
    st = Stack(torch, wq)
    out = {"layers": synth.STACK_LAYERS, "weight_bytes": st.bytes(0)}
    for M in (1, 512):
        x = torch.from_numpy(synth.stack_input(M).view(np.int16)).cuda().view(torch.bfloat16)
        bufs = st.buffers(M)
        t = graph_time(torch, lambda: st.forward(x, bufs), reps, 1, warm_s=0.05)
        if M == 1:
            bps = st.bytes(1) / t
            out["M1"] = {"ms": t * 1e3, "TB/s": bps / 1e12, "frac_of_hbm_peak": bps / 1e9 / HBM_PEAK_GBS}
        else:
            fl = st.flops(M) / t
            out["M512"] = {"ms": t * 1e3, "TFLOP/s": fl / 1e12,
                           "frac_of_peak": fl / 1e12 / BF16_PEAK_TFLOPS}
        del bufs, x
    del st
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=8, help="weight copies per bit width")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-secondary", action="store_true", help="skip prefill and W4A8 figures")
    ap.add_argument("--pmc-run", action="store_true",
                    help="no timing: 16 launches of the b=6 decode kernel, then a 64 MiB fill and "
                         "a 64 MiB sum (known-size references for rocprofv3 --pmc byte counters)")
    ap.add_argument("--ceilings", action="store_true",
                    help="no library timing: practical ceilings (streaming read of the decode "
                         "layer's bytes, torch bf16 GEMM at the prefill shapes), one JSON line")
    ap.add_argument("--pmc-layer", type=int, default=0, metavar="M",
                    help="no timing: three calls of the K=5120, N=17408, b=6 layer at batch M "
                         "(for rocprofv3 --pmc activity counters)")
    ap.add_argument("--pmc-a8", type=int, default=0, metavar="M",
                    help="no timing: three calls of the W4A8 layer (K=5120, N=17408, b=4) at "
                         "batch M (for rocprofv3 --pmc activity counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import weight_only_bit_wq_amd as wq
    from weight_only_bit_wq_amd import synth

    if not torch.cuda.is_available() or not wq.wq_device_supported(0):
        print("bench.py needs an MI355X (gfx950) GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.pmc_run:
        pmc_run(torch, wq, synth, args.copies)
        return
    if args.ceilings:
        print(json.dumps(ceilings_run(torch)), flush=True)
        return
    if args.pmc_layer > 0:
        pmc_layer_run(torch, wq, synth, args.pmc_layer)
        return
    if args.pmc_a8 > 0:
        pmc_a8_run(torch, wq, synth, args.pmc_a8)
        return

    log("setting up decode layers (b=5,6,7; %d copies each)" % args.copies)
    layers = [DecodeLayer(b, args.copies, torch, wq, synth) for b in DECODE_BITS]
    torch.cuda.synchronize()
    step_bytes = sum(l.bytes for l in layers)

    def steps_fn(n):
        def fn():
            for i in range(n):
                for l in layers:
                    l.call(wq, i)
        return fn

    # Warmup: W steps, untimed; then exactly K steps timed, synchronised on
    # both sides.  The K steps are one captured graph.
    fn = steps_fn(args.steps)
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    if args.warmup:
        wfn = steps_fn(args.warmup)
        gw = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw):
            wfn()
        gw.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    stop.record()
    torch.cuda.synchronize()
    total_s = start.elapsed_time(stop) / 1e3
    ms_per_step = total_s * 1e3 / args.steps
    value = step_bytes * args.steps / total_s / 1e12
    log("decode step: %.2f us, %.3f TB/s" % (ms_per_step * 1e3, value))

    # Roofline of the dominant kernel (b = 6 decode): launches of that kernel
    # alone, rotating copies, timed with events on its stream.
    l6 = layers[1]
    reps = max(64, args.steps)
    t6 = graph_time(torch, lambda: [l6.call(wq, i) for i in range(reps)], 3, 1) / reps
    achieved = l6.bytes / t6 / 1e9
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                "kernel": "decode_rows_kernel<B=6, RW=8, S=4, TMAX=2> (one-row decode, tiled layout)",
                "us_per_launch": t6 * 1e6,
                "bytes_per_launch": l6.bytes}
    log("b=6 decode kernel: %.2f us/launch, %.0f GB/s" % (t6 * 1e6, achieved))

    per_b = {}
    for l in layers:
        tb = graph_time(torch, lambda l=l: [l.call(wq, i) for i in range(reps)], 3, 1) / reps
        per_b["b%d" % l.b] = {"us": tb * 1e6, "TB/s": l.bytes / tb / 1e12,
                              "frac_of_hbm_peak": l.bytes / tb / 1e9 / HBM_PEAK_GBS}
    del layers, l6, g
    torch.cuda.empty_cache()

    result = {
        "metric": "wq_gemm TB/s (M=1, % HBM peak) and TFLOP/s (M=4096, % MFMA peak) at b=5/6/7",
        "value": value, "unit": "TB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded uniform codes, signed half-normal group scales, N(0,1) bf16 activations)",
        "config": {"workload": "decode M=1, K=5120, N=17408, b=5/6/7, group 128, tiled layout, "
                               "%d rotating weight copies per b" % args.copies,
                   "M": 1, "K": DECODE_K, "N": DECODE_N, "bits": list(DECODE_BITS),
                   "step": "3 wq_gemm calls (b=5,6,7)", "parallelism": "none (1 GPU)"},
        "decode_per_b": per_b,
        "roofline": roofline,
    }
    if not args.no_secondary:
        log("practical ceilings (quick)")
        ceil = hip_ceilings(torch, quick=True)
        result["ceilings"] = ceil
        sr = ceil["stream_read"]["TB/s"] * 1e3
        roofline["ceiling"] = {"kind": "stream_read", "GB/s": sr}
        roofline["frac_of_ceiling"] = roofline["achieved"] / sr
        for v in per_b.values():
            v["frac_of_ceiling"] = v["TB/s"] * 1e3 / sr
        torch.cuda.empty_cache()
        log("decode M=4/16")
        result["decode_sweep"] = bench_decode_sweep(torch, wq, synth, 3, args.copies)
        torch.cuda.empty_cache()
        for v in result["decode_sweep"].values():
            v["frac_of_ceiling"] = v["TB/s"] * 1e3 / sr
        log("prefill M=4096")
        result["prefill"] = bench_prefill(torch, wq, synth, reps=10)
        bf = ceil["mfma_f32_32x32x16_bf16"]["TFLOP/s"]
        for v in result["prefill"].values():
            v["frac_of_ceiling"] = v["TFLOP/s"] / bf
        torch.cuda.empty_cache()
        log("w4a8 M=2048/8192")
        result["w4a8"] = bench_w4a8(torch, wq, synth, reps=10)
        i8 = max(ceil["mfma_i32_16x16x64_i8"]["TOP/s"], ceil["mfma_i32_32x32x32_i8"]["TOP/s"])
        for v in result["w4a8"].values():
            v["frac_of_ceiling"] = v["TOP/s"] / i8
        torch.cuda.empty_cache()
        log("zero points / per-channel scales, b=4/8")
        result["zero_points"] = bench_zero_points(torch, wq, synth, 10, args.copies)
        torch.cuda.empty_cache()
        log("grouped layer: 64 experts 5120 -> 2048, b=6, top-4")
        result["grouped"] = bench_grouped(torch, wq, synth, 10)
        torch.cuda.empty_cache()
        log("embedding gather T=4096 from 248320 x 5120, b=6/8")
        result["embed"] = bench_embed(torch, wq, synth, reps=20)
        torch.cuda.empty_cache()
        log("8-way shard shapes, b=6: up N=2176, down K=2176")
        result["shards_p8"] = bench_shards(torch, wq, synth, 10, args.copies)
        torch.cuda.empty_cache()
        log("stack: 64 mixed-bit layers + 8-bit head, M=1 and 512")
        result["stack"] = bench_stack(torch, wq, reps=3)
    if not args.no_cpu:
        import oracle
        log("cpu oracle baseline (~%.0f s)" % args.cpu_seconds)
        result["cpu_baseline"] = cpu_baseline(oracle, synth, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
