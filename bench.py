"""Benchmark of the gfx950 tile-rANS decode path on one MI355X.

Headline workload (a "step"): one full-model decode of the DiT-like denoiser, the largest
single-GPU configuration: 30 blocks x 5 linear weights ([11520, 3840], [3840, 3840],
[10240, 3840] x 2, [3840, 10240]), 150 distinct matrices, 5.31 G weights of 0.02 t(5) BF16 coded
at 4.0 bits per weight, decoded to BF16 as five grouped launches of 30 matrices (one decode
kernel each). The weights are drawn on the GPU (seed 3000 + 5 b + m) and coded by the device
encoder before timing; inputs are resident in HBM, and a step moves 13.4 GB, far beyond the
256 MB Infinity Cache.

Prints one JSON line (rank 0, N = 1): decoded-weight GB/s (container bytes written per second
over K back-to-back steps), the roofline of one 30-matrix decode launch from HIP events on the
launch stream, the oracle's CPU decode of a bounded sample of the same streams, and extra
sections: the 4096 x 4096 seven-decode step, the two lossless BF16 codings, the encoders, the
fused decode + GEMM forward of an 8192 x 8192 weight in both tile layouts (M = 4096 ... 1, BF16
and FP8 compute) and the 64-matrix mixed-rate set.

    python bench.py [--steps K] [--warmup W] [--settle S] [--no-cpu] [--no-gemm] [--step-only]
    python bench.py --trace-summary DIR/..._kernel_trace.csv --kernel decode_group --skip N
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, 8 TB/s


PROFILE_DIT = os.path.join(ROOT, "profiles", "decode_group_dit_model_counters.txt")
PROFILE_C2 = os.path.join(ROOT, "profiles", "decode_group_4096sq_step.txt")


def decode_source_sha() -> str:
    """SHA-256 of the decode kernel's sources, decode.hip, decode_core.h and kernels.h (the key of the
    committed counter summaries)."""
    import hashlib
    src = os.path.join(ROOT, "decode_tile_interleaved_rans_amd", "csrc")
    return hashlib.sha256(b"".join(open(os.path.join(src, f), "rb").read()
                                   for f in ("decode.hip", "decode_core.h", "kernels.h"))).hexdigest()


def profiled_traffic(path: str):
    """HBM bytes per decode launch from a committed rocprofv3 counter summary, or None when the
    decode kernel's source changed since the counters were taken."""
    try:
        kv = dict(l.split(": ", 1) for l in open(path).read().splitlines() if l and not l.startswith("#"))
        return int(kv["traffic_bytes_per_launch"]) if kv.get("kernel_source_sha256") == decode_source_sha() else None
    except (OSError, KeyError, ValueError):
        return None


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(sample, budget_s: float = 10.0):
    """The oracle decoding a bounded sample of the headline workload's streams to BF16 on the host
    cores: whole DiT-like blocks (5 matrices each, in block order) with 16 threads until about
    budget_s seconds have passed, then block 0 on one thread."""
    import oracle
    cores = min(16, os.cpu_count() or 1)
    t0 = time.time()
    out_bytes, blocks = 0, 0
    for b, streams in enumerate(sample):
        for st in streams:
            out, _ = oracle.decompress(st, oracle.BF16, n_threads=cores)
            out_bytes += out.nbytes
            del out
        blocks += 1
        if time.time() - t0 >= budget_s:
            break
    dt = time.time() - t0
    t1 = time.time()
    one_bytes = 0
    for st in sample[0]:
        out, _ = oracle.decompress(st, oracle.BF16, n_threads=1)
        one_bytes += out.nbytes
        del out
    dt1 = time.time() - t1
    return {"value": round(out_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{blocks} of the 30 DiT-like blocks (5 matrices, 177 M weights each; the streams the GPU "
                      f"decodes) decoded to BF16 by the oracle with {cores} threads in {dt:.1f} s",
            "one_core": {"value": round(one_bytes / dt1 / 1e9, 4), "unit": "GB/s",
                         "sample": f"block 0 (5 matrices) decoded to BF16 on one thread in {dt1:.1f} s"}}


def c2_items():
    """(name, stream bytes, container, actual bpp) of the 4096 x 4096 seven-decode step."""
    import decode_tile_interleaved_rans_amd as ep
    from decode_tile_interleaved_rans_amd import workloads as W
    w = W.student_t_rowscaled(4096, 4096, 2)
    items = []
    for t in (3.0, 4.0, 4.5):
        s, bpp = ep.compress(w, t, dtype=ep.BF16)
        items.append((f"lossy{t}_bf16", s, "bf16", bpp))
        items.append((f"lossy{t}_f16", s, "f16", bpp))
    s, bpp = ep.lossless_compress(w, dtype=ep.BF16)
    items.append(("lossless_bf16", s, "bf16", bpp))
    return items, w.shape


def c2_step_section(torch, ep, steps: int = 20):
    """The 4096 x 4096 BF16 Student-t(5) matrix with log-normal row scales at 3.0 / 4.0 / 4.5 bpp,
    each decoded to BF16 and FP16, plus its lossless BF16 decode: seven decodes in one grouped
    launch. Rotating copies of the step's buffers (> 2.5 GB between reuses) keep the Infinity
    Cache from serving repeats; per-launch HIP events on the launch stream."""
    items, (R, C) = c2_items()
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}
    out_b = len(items) * R * C * 2
    in_b = sum(len(s) for _, s, _, _ in items)
    n_sets = max(2, math.ceil(2.5e9 / (out_b + in_b)))
    sets = [([ep.upload(s) for _, s, _, _ in items],
             [torch.empty((R, C), dtype=tdt[ct], device="cuda") for _, _, ct, _ in items]) for _ in range(n_sets)]
    for k in range(3):
        ep.decompress_many(*sets[k % n_sets])
    torch.cuda.synchronize()
    ev = []
    for k in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        ep.decompress_many(*sets[k % n_sets])
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    for hs, _ in sets:
        for h in hs:
            h.check()
    us = [a.elapsed_time(b) * 1e3 for a, b in ev]
    t = float(np.mean(us))
    sets.clear()
    torch.cuda.empty_cache()
    log(f"4096^2 seven-decode step: {t:.1f} us per launch")
    return {"workload": "4096x4096 bf16 Student-t(5)x0.015 rows scaled by lognormal(0.5); lossy at 3.0/4.0/4.5 bpp "
                        "decoded to BF16 and FP16 + lossless BF16 decode, one grouped launch",
            "avg_launch_us": round(t, 2), "launch_us_min": round(min(us), 2), "bytes_per_launch": in_b + out_b,
            "algorithmic_gbs": round((in_b + out_b) / t / 1e3, 1),
            "hbm_frac": round((in_b + out_b) / t / 1e3 / HBM_PEAK_GBS, 4),
            "output_gbs": round(out_b / t / 1e3, 1), "traffic": profiled_traffic(PROFILE_C2),
            "per_decode": {n: {"actual_bpp": round(bpp, 4), "stream_bytes": len(s)} for n, s, _, bpp in items}}


def fused_gemm_section(torch, ep, reps: int = 15):
    """Fused decode + BF16 MFMA GEMM against the plain BF16 GEMM on the uncompressed weight.

    Workload: W = 0.02 t5 bf16 [8192, 8192] coded at 4.5 bpp, X ~ N(0, 1) bf16 [M, 8192],
    Y = X W^T in BF16 with fp32 accumulation, M = 4096 (prefill), 256, 64, 16 and 1. The weight is
    coded twice: in layout 0 (fused decode + matrix-vector kernel for M <= 4, transposing fused
    kernel for M <= 16) and in the row layout (every tile's rANS states on one tile row each; the
    fused kernel multiplies straight from the decoder's registers for M <= 64). Each rep is timed
    with HIP events on the launch stream and a 1 GiB buffer is rewritten between reps, so neither
    the weight nor the activations are served from the Infinity Cache."""
    from decode_tile_interleaved_rans_amd import workloads as W
    w, xb = W.prefill_case()
    t0 = time.time()
    # coded as CompressedLinear.from_linear codes a layer: probability precision n = 11
    s, bpp = ep.compress(w, 4.5, dtype=ep.BF16, prob_bits=ep.LAYER_PROB_BITS)
    log(f"encoded 8192x8192 at target 4.5: actual {bpp:.4f} bpp in {time.time() - t0:.2f} s")
    layer = ep.CompressedLinear(s)
    layer8 = ep.CompressedLinear(s, compute="fp8")
    sr, bppr = ep.compress(w, 4.5, dtype=ep.BF16, prob_bits=ep.LAYER_PROB_BITS, layout=ep.ROW_LAYOUT)
    layer_r = ep.CompressedLinear(sr)
    layer_r8 = ep.CompressedLinear(sr, compute="fp8")
    Wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    Xf = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    N, K = Wt.shape
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()

    def timed(fns):
        """Median and min per-rep time (us) of each function; the functions take turns within
        every rep, so clock and thermal drift affect them alike."""
        for fn in fns:
            for _ in range(2):
                fn()
        ds = [[] for _ in fns]
        for _ in range(reps):
            for i, fn in enumerate(fns):
                flush.fill_(1.0)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(st)
                fn()
                b.record(st)
                ds[i].append((a, b))
        torch.cuda.synchronize()
        out = []
        for d in ds:
            us = sorted(a.elapsed_time(b) * 1e3 for a, b in d)
            out.append((us[len(us) // 2], us[0]))
        return out

    wdec = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    (t_dec, _), (t_dec_r, _) = timed([lambda: layer.handle.decompress_into(wdec),
                                      lambda: layer_r.handle.decompress_into(wdec)])
    layer.handle.check()
    layer_r.handle.check()
    out = {"workload": "W 0.02 t5 bf16 [8192, 8192] at 4.5 bpp, X N(0,1) bf16 [M, 8192], Y = X W^T bf16, "
                       "fp32 accumulate",
           "prob_bits": ep.LAYER_PROB_BITS, "actual_bpp": round(bpp, 4), "stream_bytes": len(s), "decode_full_us": round(t_dec, 2),
           "row_layout": {"actual_bpp": round(bppr, 4), "stream_bytes": len(sr), "decode_full_us": round(t_dec_r, 2)},
           "reps": reps, "timing": "median of per-rep HIP events, the five variants interleaved within each "
                                   "rep, 1 GiB cache flush before every timed call"}
    # plain FP8 baseline: ep.gemm_fp8 on the weight and activations pre-quantized per row
    # (hipBLASLt from 512 rows, above 64 when K <= 4096, from 256 when N <= 4096; the library's own
    # kernel else)
    wq, ws = ep.quantize_rows_fp8(Wt)
    for M in (4096, 256, 64, 32, 16, 4, 1):
        X = Xf[:M].contiguous()
        xq, xs = ep.quantize_rows_fp8(X)
        (t_f, t_f_min), (t_o, _), (t_t, _), (t_f8, _), (t_o8, _), (t_r, t_r_min), (t_r8, _) = timed(
            [lambda: layer(X), lambda: ep.gemm_bf16(X, Wt), lambda: torch.matmul(X, Wt.t()),
             lambda: layer8(X), lambda: ep.gemm_fp8(xq, xs, wq, ws), lambda: layer_r(X), lambda: layer_r8(X)])
        layer.handle.check()
        layer8.handle.check()
        layer_r.handle.check()
        layer_r8.handle.check()
        fl = 2.0 * M * N * K
        out[f"M{M}"] = {
            "fused_us": round(t_f, 2), "fused_min_us": round(t_f_min, 2), "own_gemm_us": round(t_o, 2),
            "torch_matmul_us": round(t_t, 2),
            "overhead_vs_own_gemm": round(t_f / t_o - 1, 4), "overhead_vs_torch": round(t_f / t_t - 1, 4),
            "fused_tflops": round(fl / t_f / 1e6, 1), "own_gemm_tflops": round(fl / t_o / 1e6, 1),
            "torch_tflops": round(fl / t_t / 1e6, 1),
            # FP8 compute: weight decoded to E4M3 + row scales, activations quantized per row
            "fp8_fused_us": round(t_f8, 2), "fp8_plain_gemm_us": round(t_o8, 2),
            "fp8_overhead_vs_plain_fp8_gemm": round(t_f8 / t_o8 - 1, 4),
            "fp8_fused_vs_torch_bf16": round(t_f8 / t_t - 1, 4),
            "fp8_fused_tflops": round(fl / t_f8 / 1e6, 1), "fp8_plain_gemm_tflops": round(fl / t_o8 / 1e6, 1),
            # HBM-bound view for small M: X + compressed W + Y
            "fused_hbm_frac": round((2 * M * K + len(s) + 2 * M * N) / t_f / 1e3 / HBM_PEAK_GBS, 4),
            # the same weight in the row layout
            "row_layout": {"fused_us": round(t_r, 2), "fused_min_us": round(t_r_min, 2),
                           "vs_decode_alone": round(t_r / t_dec_r, 4), "overhead_vs_own_gemm": round(t_r / t_o - 1, 4),
                           "overhead_vs_torch": round(t_r / t_t - 1, 4), "fp8_fused_us": round(t_r8, 2),
                           "fp8_overhead_vs_plain_fp8_gemm": round(t_r8 / t_o8 - 1, 4)},
        }
        log(f"fused GEMM M={M}: fused {t_f:.1f} us, own GEMM {t_o:.1f} us, torch {t_t:.1f} us; "
            f"FP8 fused {t_f8:.1f} us, plain FP8 GEMM {t_o8:.1f} us; row layout {t_r:.1f} us, FP8 {t_r8:.1f} us")
    del flush, wdec, Wt, Xf, layer, layer8, layer_r, layer_r8, wq, ws
    torch.cuda.empty_cache()
    return out


def dit_forward_section(torch, ep, tokens=(4096, 256, 16), reps: int = 3):
    """The DiT-like model's 150 linear layers as compressed layers (coded as
    CompressedLinear.from_linear codes layers: row tile layout, prob_bits 11, 4.0 bpp target; the
    same GPU-drawn weights as the headline step), their forwards in model order at M tokens
    against torch.matmul on the same weights decoded to BF16 (X ~ N(0, 1) bf16 per input width,
    seed 600). The linear-layer part of one denoising step: the pages time the whole step of their
    image model with compressed against uncompressed weights; attention and the other layers of
    that step are outside the method and not modeled here."""
    from decode_tile_interleaved_rans_amd import workloads as W
    t0 = time.time()
    layers, ws = [], []
    for b in range(W.DIT_BLOCKS):
        for m, (R, Cc) in enumerate(W.DIT_BLOCK_SHAPES):
            w = W.gpu_student_t(R, Cc, 3000 + 5 * b + m, 0.02)
            st, _ = ep.compress_device(w, 4.0, prob_bits=ep.LAYER_PROB_BITS, layout=ep.LAYER_LAYOUT)
            del w
            lay = ep.CompressedLinear(st)
            layers.append(lay)
            ws.append(lay.handle.decompress(torch.bfloat16))
    torch.cuda.synchronize()
    for lay in layers:
        lay.handle.check()
    log(f"DiT-like forward: 150 layers coded and decoded in {time.time() - t0:.1f} s")
    weights = sum(w.numel() for w in ws)
    stream_bytes = sum(len(lay.stream) for lay in layers)
    out = {"workload": "the DiT-like model's 150 linear layers (5.31 G weights, 4.0 bpp target, row tile layout, "
                       "prob_bits 11) in model order, Y = X W^T bf16, against torch.matmul on the decoded BF16 weights",
           "actual_bpp": round(8 * stream_bytes / weights, 4), "reps": reps}
    for M in tokens:
        g = torch.Generator(device="cuda")
        g.manual_seed(600)
        xs = {c: torch.randn((M, c), generator=g, device="cuda").to(torch.bfloat16)
              for c in sorted({Cc for _, Cc in W.DIT_BLOCK_SHAPES})}
        xin = [xs[w.shape[1]] for w in ws]
        for lay, x in zip(layers, xin):
            lay(x)
        for x, w in zip(xin, ws):
            torch.matmul(x, w.T)
        torch.cuda.synchronize()
        tf, tt = [], []
        for _ in range(reps):
            a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            a.record()
            for lay, x in zip(layers, xin):
                lay(x)
            b.record()
            for x, w in zip(xin, ws):
                torch.matmul(x, w.T)
            c.record()
            torch.cuda.synchronize()
            tf.append(a.elapsed_time(b))
            tt.append(b.elapsed_time(c))
        for lay in layers:
            lay.handle.check()
        f, t = float(np.median(tf)), float(np.median(tt))
        out[f"M{M}"] = {"compressed_ms": round(f, 3), "torch_matmul_ms": round(t, 3), "overhead_vs_torch": round(f / t - 1, 4),
                        "tflops_compressed": round(2.0 * M * weights / f / 1e9, 1)}
        log(f"DiT-like forward M={M}: compressed {f:.2f} ms, torch.matmul {t:.2f} ms")
        if True:
            # the gate and up projections of each block take the same input: one grouped call
            # (ep_linear_forward_many: one fused launch up to 64 rows, one grouped slice decode
            # above) instead of two forwards; the other layers as above
            def grouped():
                for blk in range(W.DIT_BLOCKS):
                    L5 = layers[5 * blk:5 * blk + 5]
                    x5 = xin[5 * blk:5 * blk + 5]
                    L5[0](x5[0])
                    L5[1](x5[1])
                    ep.linear_forward_many(L5[2:4], x5[2])
                    L5[4](x5[4])
            grouped()
            torch.cuda.synchronize()
            tg = []
            for _ in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                grouped()
                b.record()
                torch.cuda.synchronize()
                tg.append(a.elapsed_time(b))
            for lay in layers:
                lay.handle.check()
            fg = float(np.median(tg))
            out[f"M{M}"]["compressed_grouped_ffn_ms"] = round(fg, 3)
            out[f"M{M}"]["grouped_overhead_vs_torch"] = round(fg / t - 1, 4)
            log(f"DiT-like forward M={M}: gate and up grouped {fg:.2f} ms")
        del xs, xin
    del layers, ws
    torch.cuda.empty_cache()
    return out


def lossless_section(torch, ep, reps: int = 10):
    """The two lossless BF16 codings of the 4096 x 4096 matrix side by side, outside the step:
    byte-plane tile rANS (the step's lossless decode) and the exponent-coded variant (exponent
    byte by tile rANS, sign and mantissa uncoded). Each launch decodes 8 copies of one stream
    (grouped), rotating over 4 buffer sets so that no launch finds its data in the Infinity
    Cache; median of per-launch HIP events."""
    from decode_tile_interleaved_rans_amd import workloads as W
    w = W.student_t_rowscaled(4096, 4096, 2)
    src = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    out = {}
    for name, kw in (("byte_planes", {}), ("exponent_coded", {"exponent_coded": True})):
        s, bpp = ep.lossless_compress(w, dtype=ep.BF16, **kw)
        sets = [([ep.upload(s) for _ in range(8)],
                 [torch.empty((4096, 4096), dtype=torch.bfloat16, device="cuda") for _ in range(8)]) for _ in range(4)]
        for k in range(2):
            ep.decompress_many(*sets[k % 4])
        ev = []
        for k in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            ep.decompress_many(*sets[k % 4])
            b.record()
            ev.append((a, b))
        torch.cuda.synchronize()
        for hs, outs in sets:
            for h in hs:
                h.check()
        if not all(torch.equal(o, src) for o in sets[0][1]):
            raise RuntimeError(f"lossless {name} decode differs from the input")
        us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))
        nbytes = 8 * (len(s) + 2 * w.size)
        out[name] = {"actual_bpp": round(bpp, 4), "us_per_matrix": round(us / 8, 2),
                     "algorithmic_gbs": round(nbytes / us / 1e3, 1), "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
        log(f"lossless {name}: {bpp:.4f} bpp, {us / 8:.1f} us per 4096^2 matrix")
        del sets
    torch.cuda.empty_cache()
    return out


def encoder_section(torch, ep, reps: int = 3):
    """The lossy encoders on the 8192 x 8192 BF16 weight at 4.5 bpp: the device encoder (weight in
    device memory, stream returned to the host) against the threaded host encoder; both produce
    the same bytes (checked). Wall-clock medians of reps calls."""
    from decode_tile_interleaved_rans_amd import workloads as W
    w, _ = W.prefill_case()
    t = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    ep.compress_device(t, 4.5)
    torch.cuda.synchronize()
    dev, host = [], []
    for _ in range(reps):
        t0 = time.perf_counter()
        sd, _ = ep.compress_device(t, 4.5)
        t1 = time.perf_counter()
        sh, _ = ep.compress(w, 4.5, dtype=ep.BF16)
        t2 = time.perf_counter()
        if sd != sh:
            raise RuntimeError("device and host encoders disagree")
        dev.append(t1 - t0)
        host.append(t2 - t1)
    d, h = float(np.median(dev)), float(np.median(host))
    log(f"encoders 8192^2 at 4.5: device {1e3 * d:.1f} ms, host {1e3 * h:.1f} ms")
    return {"workload": "W 0.02 t5 bf16 [8192, 8192] at 4.5 bpp, stream to host memory", "device_ms": round(1e3 * d, 2),
            "host_ms": round(1e3 * h, 2), "host_threads": os.cpu_count(), "device_gweights_per_s": round(w.size / d / 1e9, 3),
            "host_gweights_per_s": round(w.size / h / 1e9, 3), "identical_streams": True}


def dit_step(torch, ep, steps: int, warmup: int, cpu_blocks: int = 10, settle: int = 10):
    """The headline step: the DiT-like model decoded to BF16 as five grouped launches of 30
    matrices (after `settle` untimed steps and the W warm-up steps). Returns the timing record and
    the host bytes of the first cpu_blocks blocks' streams (the CPU baseline's sample)."""
    from decode_tile_interleaved_rans_amd import workloads as W
    t0 = time.time()
    hs, outs, in_sizes, sample = [], [], [], []
    for b in range(W.DIT_BLOCKS):
        blk = []
        for m, (R, Cc) in enumerate(W.DIT_BLOCK_SHAPES):
            w = W.gpu_student_t(R, Cc, 3000 + 5 * b + m, 0.02)
            st, _ = ep.compress_device(w, 4.0)
            del w
            hs.append(ep.upload(st))
            in_sizes.append(len(st))
            outs.append(torch.empty((R, Cc), dtype=torch.bfloat16, device="cuda"))
            if b < cpu_blocks:
                blk.append(st)
        if blk:
            sample.append(blk)
    torch.cuda.synchronize()
    log(f"DiT-like model: 150 matrices drawn and coded on the GPU in {time.time() - t0:.1f} s")
    G = 30
    groups = [(hs[i:i + G], outs[i:i + G]) for i in range(0, len(hs), G)]
    group_bytes = [sum(in_sizes[i:i + G]) + sum(o.numel() * 2 for o in outs[i:i + G]) for i in range(0, len(hs), G)]

    def step():
        for gh, go in groups:
            ep.decompress_many(gh, go)

    # The launch time falls from ~1000 to ~835 us over the first ~7 steps of a run (measured in the
    # kernel trace: the same launches, back to back); settle that before the W warm-up steps
    for _ in range(settle):
        step()
    for _ in range(warmup):
        step()
    # no host work between the warm-up and the timed steps: 150 handle checks here (one device
    # read each, ~8 ms) left the GPU idle long enough for its clocks to drop, and the timed steps
    # then ramped from ~990 back to ~835 us per launch; the error flags are sticky, so the checks
    # after the timed launches cover the warm-up too
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        step()                                       # back to back, no events between launches
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = a.elapsed_time(b)
    # per-launch durations: HIP events around each 30-matrix launch on the launch stream (the
    # current stream), over K further steps
    ev = []
    for _ in range(steps):
        for k, (gh, go) in enumerate(groups):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            ep.decompress_many(gh, go)
            e1.record()
            ev.append((k, e0, e1))
    torch.cuda.synchronize()
    for h in hs:
        h.check()
    durs = [e0.elapsed_time(e1) / 1e3 for _, e0, e1 in ev]
    bytes_launch = float(np.mean([group_bytes[k] for k, _, _ in ev]))
    t_launch = float(np.mean(durs))
    out_b = sum(o.numel() * 2 for o in outs)
    in_b = sum(in_sizes)
    weights = sum(o.numel() for o in outs)
    for h in hs:
        h.release()
    del outs, groups, hs
    torch.cuda.empty_cache()
    sec = ms / 1e3
    achieved = bytes_launch / t_launch / 1e9
    log(f"DiT-like model step: {ms / steps:.3f} ms; one 30-matrix launch {t_launch * 1e6:.1f} us")
    rec = {
        "value": round(out_b * steps / sec / 1e9, 2), "ms_per_step": round(ms / steps, 4), "wall_s": round(wall, 4),
        "weights_per_s": round(weights * steps / sec / 1e9, 3),
        "hbm_frac_step": round((in_b + out_b) * steps / sec / 1e9 / HBM_PEAK_GBS, 4),
        "gb_in": round(in_b / 1e9, 3), "gb_out": round(out_b / 1e9, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": profiled_traffic(PROFILE_DIT),
                     "kernel": "decode_group (one grouped launch of 30 DiT-like matrices -> BF16)",
                     "avg_launch_us": round(t_launch * 1e6, 2), "launch_us_min": round(min(durs) * 1e6, 2),
                     "bytes_per_launch": int(bytes_launch), "launches_timed": len(durs)},
    }
    return rec, sample


def kernel_matches(name: str, kernel: str) -> bool:
    """Whether a profiler's kernel name (namespaces, template arguments, parameter list) is `kernel`."""
    import re
    return re.search(r"(^|::|\s)" + re.escape(kernel) + r"\s*[(<]", name) is not None


def trace_summary(path: str, kernel: str, skip: int) -> str:
    """Text summary of a rocprofv3 kernel-trace CSV: the launches of `kernel` after the first
    `skip` (warm-up) ones, their mean / min / max duration, and the decode sources' hash."""
    import csv
    rows = [r for r in csv.DictReader(open(path)) if kernel_matches(r["Kernel_Name"], kernel)]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows[skip:]]
    lines = [f"kernel: {kernel}", f"launches_in_trace: {len(rows)}", f"skipped_warmup_launches: {skip}",
             f"launches_summarized: {len(d)}", f"mean_us: {np.mean(d):.2f}", f"min_us: {np.min(d):.2f}",
             f"max_us: {np.max(d):.2f}", f"median_us: {np.median(d):.2f}",
             f"kernel_source_sha256: {decode_source_sha()}"]
    return "\n".join(lines)


def pmc_summary(path: str, kernel: str, skip: int) -> str:
    """Text summary of a rocprofv3 counter-collection CSV: per counter, the values (KiB) of the
    dispatches of `kernel` after the first `skip`, and the largest value among copy kernels (the
    calibration copy of --copy-calibration)."""
    import csv
    vals, copies = {}, {}
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r.get("Dispatch_Id", 0) or 0))
    seen = {}
    for r in rows:
        name = r["Kernel_Name"]
        cname = r["Counter_Name"]
        v = float(r["Counter_Value"])
        if kernel_matches(name, kernel):
            k = seen.setdefault(cname, 0)
            seen[cname] = k + 1
            if k >= skip:
                vals.setdefault(cname, []).append(v)
        elif "copy" in name.lower():
            copies[cname] = max(copies.get(cname, 0.0), v)
    lines = []
    for c, v in vals.items():
        lines.append(f"{c}_dispatches: {len(v)}")
        lines.append(f"{c}_kib_mean: {np.mean(v):.1f}")
        lines.append(f"{c}_kib_values: " + " / ".join(f"{x:.0f}" for x in v[:8]))
    for c, v in copies.items():
        lines.append(f"copy_{c}_kib: {v:.0f}")
    lines.append(f"kernel_source_sha256: {decode_source_sha()}")
    return "\n".join(lines)


def pmc_table(path: str) -> str:
    """Mean counter values per kernel of a rocprofv3 counter-collection CSV (one line per kernel and
    counter: dispatches, mean)."""
    import csv
    acc = {}
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        key = (name[:120], r["Counter_Name"])
        acc.setdefault(key, []).append(float(r["Counter_Value"]))
    lines = []
    for (name, c), v in sorted(acc.items()):
        lines.append(f"{name} | {c} | dispatches {len(v)} | mean {np.mean(v):.1f}")
    return "\n".join(lines)


def mixed_section(torch, ep, steps: int = 5, reps: int = 5):
    """The 64-matrix mixed-rate set: rows and cols from {2048, 4096, 8192}, targets uniform in
    [2.5, 6.0] (workloads.mixed_rate_set), 1.55 G weights of 0.02 t5 BF16. The weights are drawn
    on the GPU (torch's generator seeded with the matrix seed; t5 = z / sqrt(chi2_5 / 5) from six
    normals) and coded by the device encoder, to keep the host out of the run. Timed: the whole set
    decoded to BF16, to FP8 E4M3 (+ row scales) and to INT8 (+ row scales), each as grouped
    launches of 32; then the compressed BF16 forward of all 64 layers (the same weights coded as
    CompressedLinear.from_linear codes layers: row tile layout, prob_bits 11) against torch.matmul
    on the decoded BF16 weights at M = 16, 256 and 4096 (X ~ N(0, 1) bf16, seeded 500 + i)."""
    from decode_tile_interleaved_rans_amd import workloads as W
    specs = W.mixed_rate_set()
    streams, streams_r, hs, bpps = [], [], [], []
    t0 = time.time()
    for R, Cc, tgt, seed, _ in specs:
        w = W.gpu_student_t(R, Cc, seed, 0.02)
        st, bpp = ep.compress_device(w, tgt)
        # the same weight in the tile layout of compressed layers, for the 64-layer forward
        streams_r.append(ep.compress_device(w, tgt, prob_bits=ep.LAYER_PROB_BITS, layout=ep.LAYER_LAYOUT)[0])
        del w
        streams.append(st)
        bpps.append(bpp)
        hs.append(ep.upload(st))
    log(f"mixed set: 64 matrices drawn and coded on the GPU (both layouts) in {time.time() - t0:.1f} s")
    n_w = sum(R * Cc for R, Cc, *_ in specs)
    in_b = sum(len(x) for x in streams)
    out = {"workload": "64 matrices, rows/cols in {2048, 4096, 8192}, targets U[2.5, 6.0], 0.02 t5 bf16, "
                       f"{n_w / 1e9:.3f} G weights, {in_b / 1e9:.3f} GB of streams",
           "actual_bpp_mean": round(float(np.mean(bpps)), 4)}
    dec = {}
    for name, dt, eb, scaled in (("bf16", torch.bfloat16, 2, False), ("fp8", torch.float8_e4m3fn, 1, True),
                                 ("int8", torch.int8, 1, True)):
        outs = [torch.empty((R, Cc), dtype=dt, device="cuda") for R, Cc, *_ in specs]
        scs = [torch.empty(R, dtype=torch.float32, device="cuda") for R, *_ in specs] if scaled else None
        ep.decompress_many(hs, outs, scs)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            ep.decompress_many(hs, outs, scs)
        b.record()
        torch.cuda.synchronize()
        for h in hs:
            h.check()
        ms = a.elapsed_time(b) / steps
        alg = in_b + n_w * eb + (sum(R for R, *_ in specs) * 4 * 2 if scaled else 0)
        dec[name] = {"ms": round(ms, 4), "output_gbs": round(n_w * eb / ms / 1e6, 1),
                     "algorithmic_gbs": round(alg / ms / 1e6, 1), "hbm_frac": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4),
                     "tweights_per_s": round(n_w / ms / 1e9, 4)}
        if name != "bf16":
            del outs
        else:
            wd = outs
        del scs
        log(f"mixed set to {name}: {ms:.3f} ms")
    out["decode"] = dec
    layers = [ep.CompressedLinear(st) for st in streams_r]   # as CompressedLinear.from_linear codes layers
    fused = {}
    for M in (16, 256, 4096):
        xs = []
        for (R, Cc, _, _, xseed) in specs:
            g = torch.Generator(device="cuda")
            g.manual_seed(xseed)
            xs.append(torch.randn((M, Cc), generator=g, device="cuda").to(torch.bfloat16))
        for lay, x in zip(layers, xs):
            lay(x)
        for x, w in zip(xs, wd):
            torch.matmul(x, w.T)
        torch.cuda.synchronize()
        tf, tt = [], []
        for _ in range(reps):
            a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            a.record()
            for lay, x in zip(layers, xs):
                lay(x)
            b.record()
            for x, w in zip(xs, wd):
                torch.matmul(x, w.T)
            c.record()
            torch.cuda.synchronize()
            tf.append(a.elapsed_time(b))
            tt.append(b.elapsed_time(c))
        f, t = float(np.median(tf)), float(np.median(tt))
        fused[f"M{M}"] = {"fused_ms": round(f, 4), "torch_matmul_ms": round(t, 4), "overhead_vs_torch": round(f / t - 1, 4)}
        log(f"mixed set forward M={M}: fused {f:.3f} ms, torch {t:.3f} ms")
        del xs
    out["forward_64_layers"] = fused
    for h in hs:
        h.release()
    del layers, wd
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle", type=int, default=10,
                    help="untimed steps before the warm-up steps (the launch time settles over the first ~7)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-gemm", action="store_true", help="skip the fused decode + GEMM measurement")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 256 MiB device copy first (reference for HBM byte counters)")
    ap.add_argument("--gemm-only", action="store_true",
                    help="profiling aid: run only the fused decode + GEMM measurement and print its JSON")
    ap.add_argument("--gemm-reps", type=int, default=15, help="timed reps per variant in the GEMM measurement")
    ap.add_argument("--encoder-only", action="store_true",
                    help="profiling aid: run only the encoder comparison and print its JSON")
    ap.add_argument("--c2-only", action="store_true",
                    help="profiling aid: run only the 4096 x 4096 seven-decode step and print its JSON")
    ap.add_argument("--mixed-only", action="store_true",
                    help="profiling aid: run only the 64-matrix mixed-rate set and print its JSON")
    ap.add_argument("--no-mixed", action="store_true", help="skip the 64-matrix mixed-rate set")
    ap.add_argument("--dit-forward-only", action="store_true",
                    help="profiling aid: run only the DiT-like model's compressed linear forward and print its JSON")
    ap.add_argument("--step-only", action="store_true",
                    help="profiling aid: time only the headline step (no other sections, no CPU baseline)")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="summarize a rocprofv3 kernel-trace CSV (no GPU work) and exit")
    ap.add_argument("--pmc-table", metavar="CSV",
                    help="mean counter values per kernel of a rocprofv3 counter CSV (no GPU work) and exit")
    ap.add_argument("--pmc-summary", metavar="CSV",
                    help="summarize a rocprofv3 counter-collection CSV (no GPU work) and exit")
    ap.add_argument("--kernel", default="decode_group", help="kernel name for --trace-summary / --pmc-summary")
    ap.add_argument("--skip", type=int, default=0, help="warm-up launches to leave out in --trace-summary")
    args = ap.parse_args()
    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.kernel, args.skip))
        return
    if args.pmc_table:
        print(pmc_table(args.pmc_table))
        return
    if args.pmc_summary:
        print(pmc_summary(args.pmc_summary, args.kernel, args.skip))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the decode path has no cross-GPU step (tiles, rows and "
              "matrices shard without exchange), so run it with --gpus 1.", file=sys.stderr)
        sys.exit(1)

    import torch
    import decode_tile_interleaved_rans_amd as ep

    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.gemm_only:
        print(json.dumps(fused_gemm_section(torch, ep, reps=args.gemm_reps)), flush=True)
        return
    if args.encoder_only:
        print(json.dumps(encoder_section(torch, ep)), flush=True)
        return
    if args.c2_only:
        print(json.dumps(c2_step_section(torch, ep)), flush=True)
        return
    if args.mixed_only:
        print(json.dumps(mixed_section(torch, ep)), flush=True)
        return
    if args.dit_forward_only:
        print(json.dumps(dit_forward_section(torch, ep)), flush=True)
        return
    head, sample = dit_step(torch, ep, args.steps, args.warmup, cpu_blocks=0 if args.no_cpu or args.step_only else 10,
                            settle=args.settle)
    c2 = lossless = encoders = fused = mixed = ditf = cpu = None
    if not args.step_only:
        c2 = c2_step_section(torch, ep)
        lossless = lossless_section(torch, ep)
        encoders = encoder_section(torch, ep)
        if not args.no_gemm:
            fused = fused_gemm_section(torch, ep, reps=args.gemm_reps)
        if not args.no_mixed:
            mixed = mixed_section(torch, ep)
        if not args.no_gemm:
            ditf = dit_forward_section(torch, ep)
        if not args.no_cpu:
            log("timing the oracle on the host cores")
            cpu = cpu_baseline(sample)
    line = {
        "metric": "decoded weight GB/s + % HBM roofline; fused decode+GEMM overhead vs BF16",
        "value": head["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u32 rANS state -> fp32 -> bf16", "data": "synthetic",
        "config": {"workload": "DiT-like 30-block denoiser, full-model decode per step: 150 distinct matrices "
                               "(per block [11520,3840], [3840,3840], [10240,3840] x2, [3840,10240]), 5.31 G weights "
                               "of 0.02 t(5) bf16 at 4.0 bpp -> BF16, five grouped launches of 30",
                   "matrices": 150, "weights": 5308416000, "target_bpp": 4.0, "gb_in": head["gb_in"],
                   "gb_out": head["gb_out"], "tile": "16x256, 32 rANS lanes", "prob_bits": 12},
        "weights_per_s": head["weights_per_s"], "weights_per_s_unit": "Gweights/s",
        "hbm_frac_step": head["hbm_frac_step"], "wall_s": head["wall_s"],
        "roofline": head["roofline"],
        "c2_step_4096sq": c2,
        "lossless_bf16_codings": lossless,
        "encoders": encoders,
        "fused_gemm": fused,
        "mixed_rate_set": mixed,
        "dit_forward": ditf,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
