"""GPU test of concurrent host callers: several Python threads, each on a HIP stream of its own,
upload, decode and run the compressed linear forward at the same time through the C ABI. They
share the library's per-device state (the cached CU count and kernel attributes) and each
stream has its own forward workspace.

Every decode must match the oracle bit for bit: the lossy stream decoded to BF16 and to FP8 with
row scales, and the lossless one back to the original BF16 bits. Every forward must stay within
2e-2 relative L2 of the fp64 product of the oracle-decoded weight, as in the single-caller tests.
The M = 64 forward runs the skinny GEMM, which is deterministic, so every thread must get the
same bits. The M = 3 forward runs the fused matrix-vector kernel, whose float atomics may sum in
any order, so it is held to the error bar only."""
import threading

import numpy as np
import pytest
import torch

import oracle
import decode_tile_interleaved_rans_amd as ep
from decode_tile_interleaved_rans_amd import workloads as W

pytestmark = pytest.mark.gpu

N_THREADS = 6
ITERS = 4


def rel_l2(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))


def test_concurrent_callers_on_separate_streams():
    R, Ccols = 384, 1024
    w = W.student_t(R, Ccols, seed=31).astype(np.float32)
    lossy, _ = ep.compress(w, 4.0)
    bits = W.to_bf16_bits(w)
    lossless, _ = ep.lossless_compress(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))

    want_bf16 = oracle.decompress(lossy, oracle.BF16, n_threads=8)[0]
    want_f8, want_f8_scale = oracle.decompress(lossy, oracle.F8E4M3, n_threads=8)
    w_hat = W.bf16_bits_to_f32(want_bf16).astype(np.float64)
    xs = {m: W.activations(m, Ccols, seed=500 + m) for m in (64, 3)}                  # bf16 bits
    y_ref = {m: W.bf16_bits_to_f32(x).astype(np.float64) @ w_hat.T for m, x in xs.items()}

    results, errors = [None] * N_THREADS, []
    start = threading.Barrier(N_THREADS)

    def worker(t):
        try:
            torch.cuda.set_device(0)
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                h_lossy = ep.upload(lossy, s)
                h_lossless = ep.upload(lossless, s)
                layer = ep.CompressedLinear(lossy)
                xg = {m: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() for m, x in xs.items()}
                start.wait()
                out = []
                for _ in range(ITERS):
                    bf = h_lossy.decompress(torch.bfloat16, stream=s)
                    f8, f8s = h_lossy.decompress(torch.float8_e4m3fn, stream=s)
                    ll = h_lossless.decompress(stream=s)
                    y64 = layer.forward(xg[64], stream=s)
                    y3 = layer.forward(xg[3], stream=s)
                    out.append((bf, f8, f8s, ll, y64, y3))
                h_lossy.check(s)
                h_lossless.check(s)
            s.synchronize()
            results[t] = [tuple(v.cpu() for v in it) for it in out]
        except BaseException as e:                       # reported by the main thread
            errors.append((t, repr(e)))
            start.abort()

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(N_THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors

    y64_first = None
    for t, its in enumerate(results):
        for i, (bf, f8, f8s, ll, y64, y3) in enumerate(its):
            where = f"thread {t} iteration {i}"
            assert np.array_equal(bf.view(torch.int16).numpy().view(np.uint16), want_bf16), where
            assert np.array_equal(f8.view(torch.uint8).numpy(), want_f8), where
            assert np.array_equal(f8s.numpy().view(np.uint32), want_f8_scale.view(np.uint32)), where
            assert np.array_equal(ll.view(torch.int16).numpy().view(np.uint16), bits), where
            assert rel_l2(y64.float().numpy(), y_ref[64]) < 2e-2, where
            assert rel_l2(y3.float().numpy(), y_ref[3]) < 2e-2, where
            if y64_first is None:
                y64_first = y64
            assert torch.equal(y64, y64_first), where


def test_concurrent_prefill_and_fused_forwards():
    """Four threads on streams of their own run, at the same time, the forwards whose GEMM is
    hipBLASLt's (1024 activation rows: BF16 slices, FP8 slices and the plain FP8 GEMM; the plan
    cache and each call's descriptor pointers are shared under one lock) and the row-layout fused
    kernel (40 rows). Every result must have the bits of the same call made alone first, and the
    lone calls match the fp64 products of the oracle's weights on sampled rows."""
    N, K, n_thr, iters = 1000, 2048, 4, 3
    w = W.student_t(N, K, seed=33).astype(np.float32)
    s, _ = ep.compress(w, 4.0, prob_bits=ep.LAYER_PROB_BITS, layout=ep.ROW_LAYOUT)
    bias = torch.from_numpy(W.activations(1, N, 34)[0].view(np.int16)).view(torch.bfloat16).cuda()
    layer, layer8 = ep.CompressedLinear(s, bias), ep.CompressedLinear(s, bias, compute="fp8")
    xb = {m: W.activations(m, K, seed=600 + m) for m in (1024, 40)}
    xg = {m: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() for m, x in xb.items()}
    wq, ws = ep.quantize_rows_fp8(torch.from_numpy(W.to_bf16_bits(w).view(np.int16)).view(torch.bfloat16).cuda())
    xq, xs = ep.quantize_rows_fp8(xg[1024])

    def calls(st=None):
        return (layer.forward(xg[1024], stream=st), layer8.forward(xg[1024], stream=st),
                ep.gemm_fp8(xq, xs, wq, ws, stream=st), layer.forward(xg[40], stream=st),
                layer8.forward(xg[40], stream=st))

    want = [y.cpu() for y in calls()]
    torch.cuda.synchronize()
    layer.handle.check()
    w_hat = W.bf16_bits_to_f32(oracle.decompress(s, oracle.BF16, n_threads=8)[0]).astype(np.float64)
    b64 = bias.float().cpu().numpy().astype(np.float64)
    rows = np.arange(0, 1024, 97)
    ref = W.bf16_bits_to_f32(xb[1024][rows]).astype(np.float64) @ w_hat.T + b64[None, :]
    assert rel_l2(want[0][rows].float().numpy(), ref) < 2e-2
    ref40 = W.bf16_bits_to_f32(xb[40]).astype(np.float64) @ w_hat.T + b64[None, :]
    assert rel_l2(want[3].float().numpy(), ref40) < 2e-2

    results, errors = [None] * n_thr, []
    start = threading.Barrier(n_thr)

    def worker(t):
        try:
            torch.cuda.set_device(0)
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                start.wait()
                out = [calls(st) for _ in range(iters)]
            st.synchronize()
            results[t] = [[y.cpu() for y in it] for it in out]
        except BaseException as e:                       # reported by the main thread
            errors.append((t, repr(e)))
            start.abort()

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(n_thr)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    for t, its in enumerate(results):
        for i, ys in enumerate(its):
            for j, (got, exp) in enumerate(zip(ys, want)):
                assert torch.equal(got, exp), f"thread {t} iteration {i} call {j}"
