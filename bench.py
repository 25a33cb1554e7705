"""Benchmark of the libqmm hot path on one MI355X.

Headline (one step = one decode GEMV through the C ABI):
  qmv, x f16 [1, 4096], W [4096, 4096] quantized affine 4-bit, group 64, fp16
  scales/biases. Every step reads a different copy of W from a pool of at
  least 1 GiB, so no step is served from the 256 MB MALL (a decode step
  walks a layer stack). value = algorithmic bytes / time in GB/s, where the
  algorithmic bytes are packed W + scales + biases + x + y.

The other rows of the hot path are measured in the same run and reported
under "rows": quantize, dequantize, qmv at bits 2/8 and M <= 16, the gathered
GEMV on a mixture-of-experts decode step (4 tokens, top-2 of 8 experts), the
gathered tile GEMM on a mixture-of-experts prefill step (8 blocks of 128
tokens), the non-transposed decode product (W [4096, 4096] quantized along N),
batched weights (8 batches at M = 1, 4 at M = 256), the floating-point modes'
decode GEMV (mxfp4, nvfp4, mxfp8) and their gathered form (mxfp4 experts), the
GEMV on the affine-packed layout, the chained qmm_t bench (10 loops of x =
qmm(qmm(x, W1), W2), M=1024), the quantized conv2d (x [1,64,64,320], 3x3,
groups 1 and 2) and the bf16 small-M sweep.

Timing: the K timed launches are captured in one HIP graph and replayed
between two HIP events on the launch stream, after a synchronize; a warmup
graph of W launches runs first. Inputs are seeded and synthetic and already
resident in HBM.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2516.6  # MI355X dense fp16/bf16 MFMA
POOL_BYTES = 1 << 30
METRIC = ("qmm GB/s (M≤16) & TFLOP/s (M≥1024) vs HBM/MFMA peak, "
          "4-bit g64 fp16")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(words, dt):
    from group_wise_affine_amd.devio import to_dev as _to_dev
    return _to_dev(words, dt)


def round_rows(d):
    """Round floats in a (nested) row dict for the JSON line."""
    if isinstance(d, dict):
        return {k: round_rows(v) for k, v in d.items()}
    return round(d, 4) if isinstance(d, float) else d


def alg_bytes(M, N, K, bits, gs, esize=2):
    return N * K * bits // 8 + N * (K // gs) * 2 * esize + M * K * esize + M * N * esize


class Timer:
    """Capture `launch(i)` for i in range(n) into one HIP graph and time its
    replays: `warmup` untimed replays, then `reps` replays, each between two
    HIP events recorded on the launch stream (the stream every launch is
    queued on), with a synchronize before and after the timed replays."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.Stream()

    def graph(self, launch, n):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            for i in range(n):
                launch(i)
        return g

    def replays(self, launch, n, reps, warmup=1):
        """ms of each of `reps` timed replays of an n-launch graph."""
        torch = self.torch
        with torch.cuda.stream(self.stream):
            for i in range(min(2, n)):  # eager first calls
                launch(i)
        torch.cuda.synchronize()
        g = self.graph(launch, n)
        with torch.cuda.stream(self.stream):
            for _ in range(max(warmup, 1)):
                g.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        with torch.cuda.stream(self.stream):
            ev[0].record(self.stream)
            for r in range(reps):
                g.replay()
                ev[r + 1].record(self.stream)
        torch.cuda.synchronize()
        del g
        return [ev[r].elapsed_time(ev[r + 1]) for r in range(reps)]

    def run(self, launch, n, warmup=1, reps=5):
        """Median ms per launch over `reps` replays of an n-launch graph, after
        at least `warmup` untimed launches (whole replays)."""
        ts = sorted(self.replays(launch, n, reps, -(-max(warmup, 1) // n)))
        return ts[len(ts) // 2] / n


def make_layer(torch, Q, synth, dt, N, K, gs, bits, seed, sigma=1.0):
    w = to_dev(synth.normal((N, K), seed=seed, sigma=sigma, dt=dt), dt)
    return Q.qmm_quantize(w, gs, bits)


def pooled(torch, layer, min_bytes=POOL_BYTES):
    """Distinct device copies of (wq, s, b) totalling >= min_bytes."""
    wq, s, b = layer
    per = wq.numel() * 4 + s.numel() * s.element_size() * 2
    P = max(2, -(-min_bytes // per))
    wqs = wq.unsqueeze(0).expand(P, *wq.shape).contiguous()
    ss = s.unsqueeze(0).expand(P, *s.shape).contiguous()
    bs = b.unsqueeze(0).expand(P, *b.shape).contiguous()
    return wqs, ss, bs, P


def bench_qmv(torch, Q, synth, timer, dt, M, N, K, bits, gs, steps, warmup, fn=None,
              seed=0, sigma=1.0):
    fn = fn or Q.qmv
    layer = make_layer(torch, Q, synth, dt, N, K, gs, bits, seed + 1, sigma)
    wqs, ss, bs, P = pooled(torch, layer)
    x = to_dev(synth.normal((M, K), seed=seed, dt=dt), dt)
    y = torch.empty((M, N), dtype=x.dtype, device=x.device)

    def launch(i):
        j = i % P
        fn(x, wqs[j], ss[j], bs[j], gs, bits, out=y)

    ms = timer.run(launch, steps, warmup)
    nbytes = alg_bytes(M, N, K, bits, gs)
    del wqs, ss, bs
    torch.cuda.empty_cache()
    return {"us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": nbytes,
            "pool_copies": P}


def bench_headline(torch, Q, synth, timer, steps, warmup):
    """The headline: one step = one decode token through a stack of P layers,
    the decode GEMV qmv(x f16 [1, 4096], W_l [4096, 4096] 4-bit g64) once per
    layer l, each layer a distinct copy of W in HBM (P copies, >= 1 GiB in
    all, 4x the 256 MB MALL, so no layer is served from a cache). The P
    launches of a step are one HIP graph; `warmup` untimed steps, then
    `steps` timed steps, each between HIP events on the launch stream.
    Per-launch time = median step time / P."""
    dt, M, N, K, bits, gs = "f16", 1, 4096, 4096, 4, 64
    layer = make_layer(torch, Q, synth, dt, N, K, gs, bits, 1)
    wqs, ss, bs, P = pooled(torch, layer)
    x = to_dev(synth.normal((M, K), seed=0, dt=dt), dt)
    y = torch.empty((M, N), dtype=x.dtype, device=x.device)

    def launch(i):
        Q.qmv(x, wqs[i], ss[i], bs[i], gs, bits, out=y)

    ts = timer.replays(launch, P, max(steps, 1), max(warmup, 1))
    srt = sorted(ts)
    med = srt[len(srt) // 2]
    per = med / P
    nbytes = alg_bytes(M, N, K, bits, gs)
    del wqs, ss, bs
    torch.cuda.empty_cache()
    return {"us": per * 1e3, "GB/s": nbytes / (per * 1e-3) / 1e9, "bytes": nbytes,
            "layers_per_step": P, "ms_per_step": med,
            "step_ms_min": srt[0], "step_ms_max": srt[-1],
            "timed_ms_total": sum(ts)}


CEILING_LIB = os.path.join(ROOT, "group_wise_affine_amd", "libqmm_ceiling.so")


def bench_ceiling(torch, timer, steps, warmup, nbytes=9453568, gemv_grid=(256, 640)):
    """Single-launch floor at the headline's size: (a) one launch that only
    streams `nbytes` (the headline GEMV's algorithmic bytes) from HBM with
    16-byte nontemporal loads, each launch reading a distinct slice of a
    >= 1 GiB pool (best of a few grid shapes); (b) an empty kernel of the
    headline GEMV's grid (256 workgroups of 640 threads) and of one
    workgroup. Timed like the other rows (median over graph replays)."""
    import ctypes
    L = ctypes.CDLL(CEILING_LIB)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.qmm_ceiling_read.argtypes = [vp, i64, vp, i32, i32, vp]
    L.qmm_ceiling_empty.argtypes = [i32, i32, vp]
    stride = -(-nbytes // 4096) * 4096
    P = max(2, -(-POOL_BYTES // stride))
    pool = torch.empty(P * stride, dtype=torch.uint8, device="cuda")
    pool.fill_(7)
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    base = pool.data_ptr()

    def stream():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    res = {}
    best = None
    for blocks, threads in ((256, 512), (512, 512), (1024, 256), (2048, 256), (256, 1024)):
        def launch(i, blocks=blocks, threads=threads):
            rc = L.qmm_ceiling_read(ctypes.c_void_p(base + (i % P) * stride), nbytes,
                                    ctypes.c_void_p(sink.data_ptr()), blocks, threads, stream())
            assert rc == 0
        ms = timer.run(launch, P, warmup)
        r = {"us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9, "blocks": blocks,
             "threads": threads}
        if best is None or r["us"] < best["us"]:
            best = r
    best["bytes"] = nbytes
    best["pool_slices"] = P
    best["hbm_frac"] = best["GB/s"] / HBM_PEAK_GBS
    res[f"read_{nbytes}B_one_launch"] = best
    for blocks, threads in (gemv_grid, (1, 64)):
        def launch(i, blocks=blocks, threads=threads):
            assert L.qmm_ceiling_empty(blocks, threads, stream()) == 0
        ms = timer.run(launch, 200, warmup)
        res[f"empty_kernel_{blocks}x{threads}"] = {"us": ms * 1e3}
    del pool
    torch.cuda.empty_cache()
    return res


def bench_gather(torch, Q, synth, timer, steps, warmup, E=8, T=4, topk=2, N=4096, K=4096,
                 bits=4, gs=64):
    """Mixture-of-experts decode through the gathered GEMV: T tokens x [1, K]
    f16, each routed to topk of E experts W_e [N, K] (4-bit g64), one call for
    the T*topk products. The routing is a seeded permutation of the experts
    (T*topk == E), so every expert is read once per step. Every step reads a
    different copy of the expert stack from a >= 1 GiB pool."""
    import numpy as np
    assert T * topk == E
    layers = [make_layer(torch, Q, synth, "f16", N, K, gs, bits, 100 + e) for e in range(E)]
    stack = tuple(torch.stack([l[i] for l in layers]) for i in range(3))
    del layers
    wqs, ss, bs, P = pooled(torch, stack)
    x = to_dev(np.stack([synth.normal((1, K), seed=7 + t) for t in range(T)]), "f16")
    lhs = torch.tensor([t for t in range(T) for _ in range(topk)], dtype=torch.int32,
                       device="cuda")
    rhs = torch.tensor(np.random.default_rng(5).permutation(E).tolist(), dtype=torch.int32,
                       device="cuda")
    y = torch.empty((E, 1, N), dtype=torch.float16, device="cuda")

    def launch(i):
        j = i % P
        Q.gather_qmv(x, wqs[j], ss[j], bs[j], lhs, rhs, gs, bits, out=y)

    ms = timer.run(launch, steps, warmup)
    nbytes = E * (N * K * bits // 8 + N * (K // gs) * 4) + T * K * 2 + E * N * 2
    del wqs, ss, bs
    torch.cuda.empty_cache()
    return {"us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": nbytes,
            "pool_copies": P,
            "workload": f"{T} tokens x top-{topk} of {E} experts [{N},{K}] {bits}-bit g{gs} f16"}


def bench_gather_prefill(torch, Q, synth, timer, steps, warmup, E=8, M=128, N=4096, K=4096,
                         bits=4, gs=64):
    """Mixture-of-experts prefill through the gathered tile GEMM: E blocks of
    M tokens x [M, K] f16 (tokens grouped by expert), block z multiplied by
    expert rhs[z] (a seeded permutation of the E experts W_e [N, K], 4-bit
    g64), one qmm_gather_qmm call. Every step reads a different copy of the
    expert stack from a >= 1 GiB pool."""
    import numpy as np
    layers = [make_layer(torch, Q, synth, "f16", N, K, gs, bits, 100 + e) for e in range(E)]
    stack = tuple(torch.stack([l[i] for l in layers]) for i in range(3))
    del layers
    wqs, ss, bs, P = pooled(torch, stack)
    x = to_dev(synth.normal((E, M, K), seed=11), "f16")
    rhs = torch.tensor(np.random.default_rng(6).permutation(E).tolist(), dtype=torch.int32,
                       device="cuda")
    y = torch.empty((E, M, N), dtype=torch.float16, device="cuda")
    ms = timer.run(lambda i: Q.gather_qmm(x, wqs[i % P], ss[i % P], bs[i % P], None, rhs, gs,
                                          bits, out=y), steps, warmup)
    nbytes = E * alg_bytes(M, N, K, bits, gs)
    del wqs, ss, bs
    torch.cuda.empty_cache()
    return {"us": ms * 1e3, "TFLOP/s": 2 * E * M * N * K / (ms * 1e-3) / 1e12,
            "mfma_frac": 2 * E * M * N * K / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
            "GB/s": nbytes / (ms * 1e-3) / 1e9, "pool_copies": P,
            "workload": f"{E} blocks of {M} tokens, each x one of {E} experts [{N},{K}] "
                        f"{bits}-bit g{gs} f16"}


def bench_fp(torch, Q, synth, timer, steps, warmup, bits, gs, M=1, N=4096, K=4096):
    """Decode GEMV in a floating-point mode (mxfp4 / nvfp4 / mxfp8) on an
    f16 [4096, 4096] weight; every step reads a different copy of W from a
    >= 1 GiB pool."""
    w = to_dev(synth.normal((N, K), seed=1), "f16")
    wq, sc = Q.fp_quantize(w, gs, bits)
    del w
    per = wq.numel() * 4 + sc.numel()
    P = max(2, -(-POOL_BYTES // per))
    wqs = wq.unsqueeze(0).expand(P, *wq.shape).contiguous()
    scs = sc.unsqueeze(0).expand(P, *sc.shape).contiguous()
    x = to_dev(synth.normal((M, K), seed=0), "f16")
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    ms = timer.run(lambda i: Q.fp_qmv(x, wqs[i % P], scs[i % P], gs, bits, out=y), steps, warmup)
    nbytes = N * K * bits // 8 + N * (K // gs) + M * K * 2 + M * N * 2
    del wqs, scs
    torch.cuda.empty_cache()
    return {"us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": nbytes,
            "pool_copies": P}


def bench_fp_qmm(torch, Q, synth, timer, steps, warmup, bits, gs, M=1024, N=4096, K=4096):
    """fp-mode product at large M on the MFMA tile kernel (qmm_fp_t): x f16
    [1024, 4096], W [4096, 4096] quantized on the GPU; every step reads a
    different copy of W from a >= 1 GiB pool."""
    w = to_dev(synth.normal((N, K), seed=1), "f16")
    wq, sc = Q.fp_quantize(w, gs, bits)
    del w
    per = wq.numel() * 4 + sc.numel()
    P = max(2, -(-POOL_BYTES // per))
    wqs = wq.unsqueeze(0).expand(P, *wq.shape).contiguous()
    scs = sc.unsqueeze(0).expand(P, *sc.shape).contiguous()
    x = to_dev(synth.normal((M, K), seed=0), "f16")
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    ms = timer.run(lambda i: Q.fp_qmm_t(x, wqs[i % P], scs[i % P], gs, bits, out=y), steps, warmup)
    fl = 2 * M * N * K
    del wqs, scs
    torch.cuda.empty_cache()
    return {"us": ms * 1e3, "TFLOP/s": fl / (ms * 1e-3) / 1e12,
            "mfma_frac": fl / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, "pool_copies": P,
            "workload": f"x f16 [{M},{K}] x W [{N},{K}], fp mode bits {bits} g{gs}"}


def bench_qmm_t_prefill(torch, Q, synth, timer, steps, warmup, dt="f16", M=1024, N=4096, K=4096,
                        bits=4, gs=64):
    """Affine qmm_t at large M on the MFMA tile kernel: x [M, K] times W [N, K]
    quantized affine; every step reads a different copy of W from a >= 1 GiB
    pool."""
    layer = make_layer(torch, Q, synth, dt, N, K, gs, bits, 1, 1.0 if dt == "f16" else 0.02)
    wqs, ss, bs, P = pooled(torch, layer)
    x = to_dev(synth.normal((M, K), seed=0, dt=dt), dt)
    y = torch.empty((M, N), dtype=x.dtype, device="cuda")
    ms = timer.run(lambda i: Q.qmm_t(x, wqs[i % P], ss[i % P], bs[i % P], gs, bits, out=y),
                   steps, warmup)
    fl = 2 * M * N * K
    del wqs, ss, bs
    torch.cuda.empty_cache()
    return {"us": ms * 1e3, "TFLOP/s": fl / (ms * 1e-3) / 1e12,
            "mfma_frac": fl / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, "pool_copies": P,
            "workload": f"x {dt} [{M},{K}] x W [{N},{K}], affine {bits}-bit g{gs}"}


def bench_fp_gather(torch, Q, synth, timer, steps, warmup, E=8, T=4, topk=2, N=4096, K=4096):
    """Mixture-of-experts decode with mxfp4 experts: T tokens x [1, K] f16,
    each routed to topk of E experts W_e [N, K] (a seeded permutation, every
    expert read once per step), one qmm_fp_gather_qmv call. Every step reads a
    different copy of the expert stack from a >= 1 GiB pool."""
    import numpy as np
    parts = [Q.fp_quantize(to_dev(synth.normal((N, K), seed=100 + e), "f16"), 32, 4)
             for e in range(E)]
    wq = torch.stack([p[0] for p in parts])
    sc = torch.stack([p[1] for p in parts])
    del parts
    per = wq.numel() * 4 + sc.numel()
    P = max(2, -(-POOL_BYTES // per))
    wqs = wq.unsqueeze(0).expand(P, *wq.shape).contiguous()
    scs = sc.unsqueeze(0).expand(P, *sc.shape).contiguous()
    x = to_dev(np.stack([synth.normal((1, K), seed=7 + t) for t in range(T)]), "f16")
    lhs = torch.tensor([t for t in range(T) for _ in range(topk)], dtype=torch.int32,
                       device="cuda")
    rhs = torch.tensor(np.random.default_rng(5).permutation(E).tolist(), dtype=torch.int32,
                       device="cuda")
    y = torch.empty((E, 1, N), dtype=torch.float16, device="cuda")
    ms = timer.run(lambda i: Q.fp_gather_qmv(x, wqs[i % P], scs[i % P], lhs, rhs, 32, 4, out=y),
                   steps, warmup)
    nbytes = E * (N * K // 2 + N * (K // 32)) + T * K * 2 + E * N * 2
    del wqs, scs
    torch.cuda.empty_cache()
    return {"us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": nbytes,
            "pool_copies": P,
            "workload": f"{T} tokens x top-{topk} of {E} mxfp4 experts [{N},{K}] f16"}


def bench_affine_packed(torch, Q, synth, timer, steps, warmup, M=1, N=4096, K=4096, bits=4,
                        gs=64):
    """Decode GEMV on the affine-packed layout (4-bit g64 f16, [4096, 4096]); every
    step reads a different copy of the packed weight from a >= 1 GiB pool."""
    wq, s, b = make_layer(torch, Q, synth, "f16", N, K, gs, bits, 1)
    wp, sbp = Q.affine_pack(wq, s, b, gs, bits)
    del wq, s, b
    per = wp.numel() * 4 + sbp.numel() * 2
    P = max(2, -(-POOL_BYTES // per))
    wps = wp.unsqueeze(0).expand(P, *wp.shape).contiguous()
    sbps = sbp.unsqueeze(0).expand(P, *sbp.shape).contiguous()
    x = to_dev(synth.normal((M, K), seed=0), "f16")
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    ms = timer.run(lambda i: Q.qmv_affine_packed(x, wps[i % P], sbps[i % P], N, gs, bits, out=y),
                   steps, warmup)
    nbytes = alg_bytes(M, N, K, bits, gs)
    del wps, sbps
    torch.cuda.empty_cache()
    return {"us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": nbytes,
            "pool_copies": P}


def bench_batched(torch, Q, synth, timer, steps, warmup, B, M, N=4096, K=4096, bits=4, gs=64):
    """Batched product with one weight per batch: y[b] = x[b] . dequant(W_b)^T,
    x [B, M, K] f16, W_b [N, K] 4-bit g64 (qmm_t_batched). Every step reads a
    different copy of the weight stack from a >= 1 GiB pool."""
    layers = [make_layer(torch, Q, synth, "f16", N, K, gs, bits, 200 + e) for e in range(B)]
    stack = tuple(torch.stack([l[i] for l in layers]) for i in range(3))
    del layers
    wqs, ss, bs, P = pooled(torch, stack)
    x = to_dev(synth.normal((B, M, K), seed=9), "f16")
    y = torch.empty((B, M, N), dtype=torch.float16, device="cuda")
    ms = timer.run(lambda i: Q.qmm_t_batched(x, wqs[i % P], ss[i % P], bs[i % P], gs, bits,
                                             out=y), steps, warmup)
    nbytes = B * alg_bytes(M, N, K, bits, gs)
    del wqs, ss, bs
    torch.cuda.empty_cache()
    return {"us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": nbytes,
            "TFLOP/s": 2 * B * M * N * K / (ms * 1e-3) / 1e12, "pool_copies": P,
            "workload": f"{B} batches of x f16 [{M},{K}] x W_b [{N},{K}] {bits}-bit g{gs}"}


def bench_qmm_n(torch, Q, synth, timer, steps, warmup, M=1, K=4096, N=4096, bits=4, gs=64):
    """Non-transposed product y = x . dequant(W), x f16 [M, K], W [K, N]
    quantized along N (4-bit g64, f16): the GEMV at M = 1, the MFMA tile
    kernel at M = 1024; every step reads a different copy of W from a >= 1 GiB
    pool."""
    w = to_dev(synth.normal((K, N), seed=1), "f16")
    layer = Q.qmm_quantize(w, gs, bits)
    del w
    wqs, ss, bs, P = pooled(torch, layer)
    x = to_dev(synth.normal((M, K), seed=0), "f16")
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    ms = timer.run(lambda i: Q.qmm_n(x, wqs[i % P], ss[i % P], bs[i % P], gs, bits, out=y),
                   steps, warmup)
    nbytes = alg_bytes(M, N, K, bits, gs)
    del wqs, ss, bs
    torch.cuda.empty_cache()
    flops = 2 * M * N * K
    return {"us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": nbytes,
            "TFLOP/s": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
            "pool_copies": P, "workload": f"x f16 [{M},{K}], W [{K},{N}] {bits}-bit g{gs} along N"}


def bench_quantize(torch, Q, synth, timer, steps, warmup):
    N = K = 4096
    w = to_dev(synth.normal((N, K), seed=1), "f16")
    wq, s, b = Q.qmm_quantize(w, 64, 4)
    out = (wq, s, b)
    ms = timer.run(lambda i: Q.qmm_quantize(w, 64, 4, out=out), steps, warmup)
    nbytes = N * K * 2 + N * K // 2 + N * (K // 64) * 4
    res = {"quantize": {"us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9,
                        "workload": "W f16 [4096,4096] -> 4-bit g64"}}
    wo = torch.empty_like(w)
    ms = timer.run(lambda i: Q.qmm_dequantize(wq, s, b, 64, 4, out=wo), steps, warmup)
    res["dequantize"] = {"us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9,
                         "workload": "4-bit g64 [4096,4096] -> f16"}
    return res


def bench_chained(torch, Q, synth, timer, bits, steps, warmup, packed=False):
    """10 loops of x = qmm(qmm(x, W1), W2): x [1024,1024], W1 [4096,1024],
    W2 [1024,4096], g64 f16. One step = the 20 launches of the 10 loops.
    ``packed``: the weights in the affine-packed layout (qmm_t_affine_packed)."""
    gs = 64
    x = to_dev(synth.normal((1024, 1024), seed=0), "f16")
    l1 = make_layer(torch, Q, synth, "f16", 4096, 1024, gs, bits, 1)
    l2 = make_layer(torch, Q, synth, "f16", 1024, 4096, gs, bits, 2)
    h = torch.empty((1024, 4096), dtype=torch.float16, device="cuda")
    xs = [x.clone(), torch.empty_like(x)]
    if packed:
        l1 = Q.affine_pack(*l1, gs, bits)
        l2 = Q.affine_pack(*l2, gs, bits)

        def launch(i):
            for loop in range(10):
                Q.qmm_t_affine_packed(xs[loop % 2], *l1, 4096, gs, bits, out=h)
                Q.qmm_t_affine_packed(h, *l2, 1024, gs, bits, out=xs[(loop + 1) % 2])
    else:
        def launch(i):
            for loop in range(10):
                Q.qmm_t(xs[loop % 2], *l1, gs, bits, out=h)
                Q.qmm_t(h, *l2, gs, bits, out=xs[(loop + 1) % 2])

    ms = timer.run(launch, steps, warmup)
    flops = 10 * 2 * (2 * 1024 * 4096 * 1024)
    return {"us_per_10_loops": ms * 1e3, "TFLOP/s": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS}


def bench_conv(torch, Q, synth, timer, groups, steps, warmup):
    gs, bits = 64, 4
    x = to_dev(synth.normal((1, 64, 64, 320), seed=0), "f16")
    wc = to_dev(synth.normal((320, 3, 3, 320 // groups), seed=1, sigma=0.05), "f16")
    wq, s, b = Q.quantize_conv_weight(wc, gs, bits)
    y = torch.empty((1, 64, 64, 320), dtype=torch.float16, device="cuda")
    ms = timer.run(lambda i: Q.qconv2d_nhwc(x, wq, s, b, 320, 3, 3, (1, 1), (1, 1),
                                            groups, gs, bits, out=y), steps, warmup)
    flops = 2 * 64 * 64 * 320 * (9 * 320 // groups)
    return {"us": ms * 1e3, "TFLOP/s": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS}


ROUTE_SHAPES = [("f16", 4096, 4096, 4), ("f16", 4096, 4096, 2), ("f16", 4096, 4096, 8),
                ("f16", 8192, 2048, 4), ("f16", 2048, 8192, 4), ("f16", 512, 2048, 4),
                ("bf16", 4096, 4096, 4), ("bf16", 4096, 4096, 8), ("bf16", 2048, 8192, 4), ("bf16", 8192, 2048, 4),
                ("bf16", 2048, 2048, 4), ("bf16", 512, 2048, 4), ("bf16", 2048, 8192, 3),
                ("bf16", 8192, 2048, 6)]
ROUTE_MS = (1, 2, 3, 4, 5, 6, 8, 12, 16, 24, 32)
ROUTE_LAUNCHES = 24     # eager launches per (layer, kernel, M), each on its own weight copy


def route_table(torch, Q, synth):
    """Each affine product kernel (streaming GEMV, MFMA GEMV, tile GEMM)
    forced in turn on the layers above at M = 1..32 rows of x (g64; bf16
    weights at sigma 0.02), ROUTE_LAUNCHES eager launches per point on
    distinct copies of the weight from a >= 1 GiB pool, nothing else launched
    in between (so a kernel trace splits into the points in the order of the
    printed manifest). Prints the manifest, the automatic choice and the
    eager per-launch time (HIP events) of each point as one JSON line."""
    names = {Q.KERNEL_GEMV: "gemv", Q.KERNEL_MFMA_GEMV: "mfma_gemv", Q.KERNEL_TILE: "tile"}
    gs, rows = 64, []
    for dt, N, K, bits in ROUTE_SHAPES:
        tdt = torch.float16 if dt == "f16" else torch.bfloat16
        layer = make_layer(torch, Q, synth, dt, N, K, gs, bits, 1, 1.0 if dt == "f16" else 0.02)
        wqs, ss, bs, P = pooled(torch, layer)
        x = to_dev(synth.normal((max(ROUTE_MS), K), seed=0), dt)
        y = torch.empty((max(ROUTE_MS), N), dtype=tdt, device="cuda")
        torch.cuda.synchronize()
        for kern in (Q.KERNEL_GEMV, Q.KERNEL_MFMA_GEMV, Q.KERNEL_TILE):
            Q.force_kernel(kern)
            for M in ROUTE_MS:
                if Q.route(M, N, K, bits, tdt, gs) != kern:
                    continue
                xm, ym = x[:M], y[:M]
                ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ev0.record()
                for i in range(ROUTE_LAUNCHES):
                    Q.qmm_t(xm, wqs[i % P], ss[i % P], bs[i % P], gs, bits, out=ym)
                ev1.record()
                torch.cuda.synchronize()
                Q.force_kernel(Q.KERNEL_NONE)
                auto = names[Q.route(M, N, K, bits, tdt, gs)]
                Q.force_kernel(kern)
                rows.append({"dt": dt, "N": N, "K": K, "bits": bits, "M": M,
                             "kernel": names[kern], "auto": auto, "launches": ROUTE_LAUNCHES,
                             "eager_us": round(ev0.elapsed_time(ev1) * 1e3 / ROUTE_LAUNCHES, 3)})
        Q.force_kernel(Q.KERNEL_NONE)
        del wqs, ss, bs, layer
        torch.cuda.empty_cache()
    print(json.dumps({"route_table": rows}))


def cpu_threads():
    """Threads the oracle runs with on all cores: OMP_NUM_THREADS when set,
    else the CPUs this process may run on."""
    try:
        env = os.environ.get("OMP_NUM_THREADS")
        return max(1, int(env) if env else len(os.sched_getaffinity(0)))
    except (ValueError, OSError):
        return max(1, os.cpu_count() or 1)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(seconds=5.0):
    """The oracle as it stands, on the host cores, on bounded samples of the
    workloads: the headline decode qmv on one thread and on all threads
    (threads split the output columns; each output's summation order is
    unchanged), one loop of the chained qmm_t bench (two products) and the
    groups = 1 conv, on all threads."""
    import oracle as orc
    from group_wise_affine_amd import synth
    nt = cpu_threads()
    M, N, K, gs, bits = 1, 4096, 4096, 64, 4
    x = synth.normal((M, K), seed=0)
    w = synth.normal((N, K), seed=1)
    wq, s, b = orc.quantize(w, orc.F16, gs, bits)
    nbytes = alg_bytes(M, N, K, bits, gs)

    def timed(fn, budget):
        fn()  # warm
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return n, el

    modes = {}
    for name, threads in (("decode_qmv_1_thread", 1), ("decode_qmv_all_threads", nt)):
        n, el = timed(lambda: orc.qmm_t(x, wq, s, b, orc.F16, gs, bits, nthreads=threads),
                      seconds)
        modes[name] = {"GB/s": round(nbytes / (el / n) / 1e9, 4), "threads": threads,
                       "calls": n, "s": round(el, 2)}
    xc = synth.normal((1024, 1024), seed=0)
    wq1, s1, b1 = orc.quantize(synth.normal((4096, 1024), seed=1), orc.F16, gs, bits)
    wq2, s2, b2 = orc.quantize(synth.normal((1024, 4096), seed=2), orc.F16, gs, bits)
    t0 = time.perf_counter()
    _, h = orc.qmm_t(xc, wq1, s1, b1, orc.F16, gs, bits, nthreads=nt)
    orc.qmm_t(h, wq2, s2, b2, orc.F16, gs, bits, nthreads=nt)
    el = time.perf_counter() - t0
    fl = 2 * (2 * 1024 * 4096 * 1024)
    modes["chained_qmm_t_one_loop_all_threads"] = {
        "TFLOP/s": round(fl / el / 1e12, 6), "s": round(el, 2), "threads": nt,
        "us_per_10_loops_extrapolated": round(el * 10 * 1e6, 1)}
    xv = synth.normal((1, 64, 64, 320), seed=0)
    wc = synth.normal((320, 3, 3, 320), seed=1, sigma=0.05)
    cq, cs, cb = orc.quantize(orc.conv_weight_matrix(wc, 1, gs), orc.F16, gs, bits)
    t0 = time.perf_counter()
    orc.qconv2d_nhwc(xv, cq, cs, cb, orc.F16, 320, 3, 3, (1, 1), (1, 1), 1, gs, bits,
                     nthreads=nt)
    el = time.perf_counter() - t0
    fl = 2 * 64 * 64 * 320 * 2880
    modes["qconv2d_groups1_all_threads"] = {"TFLOP/s": round(fl / el / 1e12, 6),
                                            "s": round(el, 2), "threads": nt}
    head = modes["decode_qmv_all_threads"]
    return {"value": head["GB/s"], "unit": "GB/s", "cores": nt, "kind": "oracle",
            "sample": f"{head['calls']} oracle calls of the headline decode qmv (M=1, "
                      f"4096x4096, 4-bit g64 f16) in {head['s']} s on {nt} threads (threads "
                      f"split the output columns); modes also time one thread, one loop of "
                      f"the chained bench and the groups=1 conv",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(), "modes": modes}


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("common.hpp", "qmv.hip"):
        with open(os.path.join(ROOT, "group_wise_affine_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "qmv_decode_4096x4096_4bit_g64_f16_traffic.md")


def measured_traffic():
    """HBM bytes per launch of the headline kernel from the committed rocprofv3
    PMC summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known
    size), if it was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    vals = {}
    with open(TRAFFIC_SUMMARY) as fh:
        for line in fh:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def traffic_probe(torch, Q, synth, launches=20):
    """For rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs: plain device copies
    of 256 MiB between distinct buffers (2 GiB in all, so no copy reads data
    a cache still holds: the counter calibration, 256 MiB read and 256 MiB
    written per dispatch), then `launches` headline GEMV calls, each on its
    own copy of W."""
    bufs = [torch.full((64 << 20,), float(i), dtype=torch.float32, device="cuda")
            for i in range(8)]
    torch.cuda.synchronize()
    for i in range(4):
        bufs[4 + i].copy_(bufs[i])
    torch.cuda.synchronize()
    del bufs
    layer = make_layer(torch, Q, synth, "f16", 4096, 4096, 64, 4, 1)
    wqs, ss, bs, P = pooled(torch, layer)
    x = to_dev(synth.normal((1, 4096), seed=0), "f16")
    y = torch.empty((1, 4096), dtype=x.dtype, device=x.device)
    for i in range(launches):
        j = i % P
        Q.qmv(x, wqs[j], ss[j], bs[j], 64, 4, out=y)
    torch.cuda.synchronize()
    log(f"traffic probe: copy 4 x 256 MiB, qmv x {launches}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50,
                    help="timed headline steps (one step = one token through the layer pool)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline decode GEMV (for profiling)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run the PMC calibration copy and headline launches, print nothing else")
    ap.add_argument("--mfma-only", action="store_true",
                    help="time only the MFMA tile rows (chained 4-bit layers, conv), for profiling")
    ap.add_argument("--route-table", action="store_true",
                    help="force each product kernel in turn at M = 1..32 on the routing layers "
                         "(for a kernel trace and counters that the route is derived from)")
    ap.add_argument("--next-only", action="store_true",
                    help="time only the gathered, batched, non-transposed and fp-mode rows, "
                         "for profiling")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the path is measured on a single "
              "MI355X; the path shards over rows of W without communication, which "
              "this benchmark does not run.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from group_wise_affine_amd import qmm as Q
    from group_wise_affine_amd import synth
    torch.cuda.set_device(0)
    Q.lib()
    if args.traffic_probe:
        traffic_probe(torch, Q, synth)
        return
    if args.route_table:
        route_table(torch, Q, synth)
        return
    timer = Timer(torch)
    K_, W_ = args.steps, args.warmup
    if args.mfma_only:
        r = {"chained_bits4": bench_chained(torch, Q, synth, timer, 4, 10, 2),
             "chained_bits4_affine_packed": bench_chained(torch, Q, synth, timer, 4, 10, 2, True),
             "conv_groups1": bench_conv(torch, Q, synth, timer, 1, 50, 5),
             "conv_groups2": bench_conv(torch, Q, synth, timer, 2, 50, 5),
             "prefill_f16_1024x4096x4096": bench_qmm_t_prefill(torch, Q, synth, timer, 20, 5),
             "prefill_bf16_1024x4096x4096": bench_qmm_t_prefill(torch, Q, synth, timer, 20, 5,
                                                                "bf16"),
             "prefill_f16_4096x4096x4096": bench_qmm_t_prefill(torch, Q, synth, timer, 20, 5,
                                                               M=4096)}
        print(json.dumps({k: {kk: round(vv, 4) for kk, vv in v.items() if isinstance(vv, float)}
                          for k, v in r.items()}))
        return
    if args.next_only:
        r = {"gather_qmv_moe_decode": bench_gather(torch, Q, synth, timer, 200, 20),
             "gather_qmm_moe_prefill": bench_gather_prefill(torch, Q, synth, timer, 20, 5),
             "qmm_t_batched_B4_M256": bench_batched(torch, Q, synth, timer, 20, 5, 4, 256),
             "qmm_n_decode": bench_qmm_n(torch, Q, synth, timer, 200, 20),
             "qmm_n_prefill_M1024": bench_qmm_n(torch, Q, synth, timer, 20, 5, M=1024)}
        for name, bits, gs in (("mxfp4", 4, 32), ("nvfp4", 4, 16), ("mxfp8", 8, 32)):
            r[f"fp_qmv_{name}"] = bench_fp(torch, Q, synth, timer, 200, 20, bits, gs)
        r["fp_gather_qmv_moe_decode_mxfp4"] = bench_fp_gather(torch, Q, synth, timer, 200, 20)
        r["qmv_affine_packed_4bit"] = bench_affine_packed(torch, Q, synth, timer, 200, 20)
        print(json.dumps({k: {kk: round(vv, 4) for kk, vv in v.items() if isinstance(vv, float)}
                          for k, v in r.items()}))
        return

    log("headline: qmv 4-bit g64 f16 M=1 4096x4096, one step = one token through the layer pool")
    torch.cuda.synchronize()
    head = bench_headline(torch, Q, synth, timer, K_, W_)
    log(f"  {head['us']:.3f} us per launch, {head['GB/s']:.1f} GB/s "
        f"({head['layers_per_step']} layers per step)")

    rows = {}
    if not args.headline_only:
        n_small = max(50, min(K_, 500))
        rows["single_launch_floor_decode_size"] = round_rows(
            bench_ceiling(torch, timer, K_, 20))
        log("ceiling rows done")
        rows.update(bench_quantize(torch, Q, synth, timer, 20, 5))
        log("quantize/dequantize done")
        dec = {}
        for bits in (2, 4, 8):
            for M in (1, 2, 4, 8, 16):
                if bits != 4 and M != 1:
                    continue
                r = bench_qmv(torch, Q, synth, timer, "f16", M, 4096, 4096, bits, 64,
                              n_small, 20)
                dec[f"bits{bits}_M{M}"] = {k: round(v, 4) if isinstance(v, float) else v
                                           for k, v in r.items()}
        rows["qmv_decode_4096x4096_f16_g64"] = dec
        log("decode rows done")
        rows["gather_qmv_moe_decode_f16_g64"] = {
            k: round(v, 4) if isinstance(v, float) else v
            for k, v in bench_gather(torch, Q, synth, timer, n_small, 20).items()}
        log("gather row done")
        rows["gather_qmm_moe_prefill_f16_g64"] = {
            k: round(v, 4) if isinstance(v, float) else v
            for k, v in bench_gather_prefill(torch, Q, synth, timer, 20, 5).items()}
        log("gather prefill row done")
        rows["qmm_n_decode_4096x4096_f16_g64"] = {
            k: round(v, 4) if isinstance(v, float) else v
            for k, v in bench_qmm_n(torch, Q, synth, timer, n_small, 20).items()}
        rows["qmm_n_prefill_1024x4096x4096_f16_g64"] = round_rows(
            bench_qmm_n(torch, Q, synth, timer, 20, 5, M=1024))
        log("qmm_n row done")
        rows["qmm_t_batched_4096x4096_f16_g64"] = {
            f"B{B}_M{M}": {k: round(v, 4) if isinstance(v, float) else v
                           for k, v in bench_batched(torch, Q, synth, timer, n_small if M == 1
                                                     else 20, 5, B, M).items()}
            for (B, M) in [(8, 1), (4, 256)]}
        log("batched rows done")
        rows["fp_qmv_decode_4096x4096_f16"] = {
            name: {k: round(v, 4) if isinstance(v, float) else v
                   for k, v in bench_fp(torch, Q, synth, timer, n_small, 20, bits, gs).items()}
            for name, bits, gs in (("mxfp4", 4, 32), ("nvfp4", 4, 16), ("mxfp8", 8, 32))}
        rows["fp_qmm_t_1024x4096x4096_f16"] = {
            name: round_rows(bench_fp_qmm(torch, Q, synth, timer, 20, 5, bits, gs))
            for name, bits, gs in (("mxfp4", 4, 32), ("nvfp4", 4, 16), ("mxfp8", 8, 32))}
        log("fp rows done")
        rows["fp_gather_qmv_moe_decode_mxfp4"] = {
            k: round(v, 4) if isinstance(v, float) else v
            for k, v in bench_fp_gather(torch, Q, synth, timer, n_small, 20).items()}
        log("fp gather row done")
        rows["qmv_affine_packed_decode_4096x4096_f16_g64"] = {
            f"bits{bits}": {k: round(v, 4) if isinstance(v, float) else v
                            for k, v in bench_affine_packed(torch, Q, synth, timer, n_small, 20,
                                                            bits=bits).items()}
            for bits in (4, 8)}
        log("affine-packed rows done")
        ch = {}
        for bits in (2, 4, 8):
            for packed in (False, True):
                ch[f"bits{bits}" + ("_affine_packed" if packed else "")] = {
                    k: round(v, 4) for k, v in
                    bench_chained(torch, Q, synth, timer, bits, 10, 2, packed).items()}
        rows["qmm_t_chained_M1024_f16_g64"] = ch
        log("chained done")
        rows["qmm_t_prefill_4bit_g64"] = {
            f"{dt}_{M}x{N}x{K}": round_rows(bench_qmm_t_prefill(torch, Q, synth, timer, 20, 5,
                                                                dt, M, N, K))
            for dt, M, N, K in (("f16", 1024, 4096, 4096), ("bf16", 1024, 4096, 4096),
                                ("f16", 4096, 4096, 4096))}
        log("prefill rows done")
        rows["qconv2d_64x64x320_3x3_f16_4bit_g64"] = {
            f"groups{g}": {k: round(v, 4) for k, v in
                           bench_conv(torch, Q, synth, timer, g, 50, 5).items()}
            for g in (1, 2)}
        log("conv done")
        sweep = {}
        for (N, K) in [(2048, 2048), (512, 2048), (8192, 2048), (2048, 8192)]:
            for bits in (4, 3, 6):
                key = f"N{N}_K{K}_bits{bits}"
                sweep[key] = {}
                for M in (1, 2, 4, 8, 16, 32, 64, 512):
                    r = bench_qmv(torch, Q, synth, timer, "bf16", M, N, K, bits, 64,
                                  200, 20, fn=Q.qmm_t, sigma=0.02)
                    sweep[key][f"M{M}"] = {"us": round(r["us"], 3),
                                           "GB/s": round(r["GB/s"], 1),
                                           "TFLOP/s": round(2 * M * N * K / (r["us"] * 1e-6) / 1e12, 3)}
        rows["small_m_sweep_bf16_g64"] = sweep
        log("sweep done")

    achieved = head["GB/s"]
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(),
                "kernel": "qmv_kernel (streaming GEMV), one launch per layer",
                "us_per_launch": round(head["us"], 4)}
    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline()
    out = {
        "metric": METRIC,
        "value": round(head["GB/s"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_,
        "warmup": W_,
        "ms_per_step": round(head["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode qmv: x f16 [1,4096] ~N(0,1), W [4096,4096] ~N(0,1) "
                               "quantized affine 4-bit g64 with f16 scales/biases; one step = "
                               f"one token through a stack of {head['layers_per_step']} such "
                               "layers, each a distinct copy of W (>=1 GiB in all), one GEMV "
                               "launch per layer",
                   "M": 1, "N": 4096, "K": 4096, "bits": 4, "group_size": 64,
                   "layers_per_step": head["layers_per_step"],
                   "algorithmic_bytes_per_launch": head["bytes"],
                   "algorithmic_bytes_per_step": head["bytes"] * head["layers_per_step"],
                   "step_ms_min_median_max": [round(head["step_ms_min"], 6),
                                              round(head["ms_per_step"], 6),
                                              round(head["step_ms_max"], 6)]},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
