"""GPU tests of the BF16 MFMA GEMM and of the compressed linear forward (decoding fused into the
layer's forward, "EntroPack PyTorch Guide", section "Replace one linear layer before a whole
model"), through the C ABI.

Reference: fp32 GEMM on the CPU of the BF16 inputs (exact in fp32) and, for the linear forward,
of the oracle-decoded BF16 weight; the bar is relative L2 error <= 2e-2 (BF16 output rounding
alone is about 2e-3)."""
import numpy as np
import pytest
import torch

import oracle
import decode_tile_interleaved_rans_amd as ep
from decode_tile_interleaved_rans_amd import workloads as W

pytestmark = pytest.mark.gpu


def rel_l2(got, want):
    got = got.astype(np.float64)
    want = want.astype(np.float64)
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


# shapes cover every tile choice: the skinny kernel (M <= 16, 32, 64: one, two or four 16-row
# tiles), 64 x 64 tiles (few output tiles), 128 x 128 tiles (2 x 256 of them or more) and
# 256 x 256 tiles (the prefill test below and the 4100 x 4000 case), with ragged M, N and K tails
@pytest.mark.parametrize("M,N,K", [(16, 256, 512), (256, 384, 1024), (130, 200, 264), (1, 8, 8), (300, 1000, 776),
                                   (33, 1000, 520), (64, 4100, 1032), (20, 17, 4104), (5, 4096, 8192),
                                   (2000, 4000, 136), (4100, 4000, 136)])
def test_gemm_bf16_matches_fp32(M, N, K):
    rng = np.random.default_rng(M + N + K)
    x = W.to_bf16_bits(rng.normal(0, 1, (M, K)))
    w = W.to_bf16_bits(rng.normal(0, 0.05, (N, K)))
    X, Wt = bf16_tensor(x).cuda(), bf16_tensor(w).cuda()
    y = ep.gemm_bf16(X, Wt)
    torch.cuda.synchronize()
    ref = W.bf16_bits_to_f32(x) @ W.bf16_bits_to_f32(w).T
    assert rel_l2(y.float().cpu().numpy(), ref) < 5e-3


def test_gemm_bf16_prefill_shape_sampled_rows():
    M, N, K = 4096, 8192, 8192
    rng = np.random.default_rng(9)
    X = torch.randn(M, K, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    Wt = (0.02 * torch.randn(N, K, generator=torch.Generator().manual_seed(2))).to(torch.bfloat16)
    y = ep.gemm_bf16(X.cuda(), Wt.cuda())
    torch.cuda.synchronize()
    rows = rng.choice(M, 48, replace=False)
    ref = X[rows].float() @ Wt.float().T
    assert rel_l2(y[rows].float().cpu().numpy(), ref.numpy()) < 5e-3


def linear_case(M, N, K, target, seed, bias=False):
    rng = np.random.default_rng(seed)
    w = (0.02 * rng.standard_t(5, (N, K))).astype(np.float32)
    x = W.to_bf16_bits(rng.normal(0, 1, (M, K)))
    s, _ = ep.compress(w, target)
    layer = ep.CompressedLinear(s, bias=None)
    b = None
    if bias:
        b = bf16_tensor(W.to_bf16_bits(rng.normal(0, 0.1, N))).cuda()
        layer.bias = b
    y = layer(bf16_tensor(x).cuda())
    torch.cuda.synchronize()
    layer.handle.check()
    w_hat = W.bf16_bits_to_f32(oracle.decompress(s, oracle.BF16, n_threads=16)[0])
    return y.float().cpu().numpy(), W.bf16_bits_to_f32(x), w_hat, (b.float().cpu().numpy() if bias else None)


@pytest.mark.parametrize("M,N,K,target", [(16, 512, 1024, 4.0), (256, 768, 2048, 4.5), (33, 300, 264, 3.0),
                                          (4, 4096, 512, 6.0)])
def test_linear_forward_matches_decoded_fp32_gemm(M, N, K, target):
    y, x, w_hat, _ = linear_case(M, N, K, target, seed=M + N)
    assert rel_l2(y, x @ w_hat.T) < 2e-2


@pytest.mark.parametrize("M,N,K,target,bias", [(1, 4096, 4096, 4.5, False), (2, 300, 264, 3.0, True),
                                                (3, 1000, 776, 6.0, True), (4, 17, 4104, 4.0, False),
                                                (1, 11520, 3840, 4.0, True)])
def test_fused_matrix_vector_few_rows(M, N, K, target, bias):
    """M <= 4 runs the fused decode + matrix-vector kernel (weights never stored): against the
    oracle-decoded BF16 weight in fp32; the kernel multiplies the unrounded fp32 weights, which
    differ from the BF16 container by at most half a BF16 step."""
    y, x, w_hat, b = linear_case(M, N, K, target, seed=M * 7 + N, bias=bias)
    ref = x @ w_hat.T + (b[None, :] if bias else 0.0)
    assert rel_l2(y, ref) < 2e-2


def test_linear_forward_with_bias_and_multi_slice():
    # 5000 x 16384 weight: 128 MiB slices of 4096 rows -> two slices, the last one ragged
    M, N, K = 64, 5000, 16384
    y, x, w_hat, b = linear_case(M, N, K, 4.0, seed=3, bias=True)
    assert rel_l2(y, x @ w_hat.T + b[None, :]) < 2e-2


def test_linear_forward_prefill_sampled_rows():
    M, N, K = 4096, 8192, 8192
    w, xb = W.prefill_case()
    s, bpp = ep.compress(w, 4.5, dtype=ep.BF16)
    layer = ep.CompressedLinear(s)
    X = bf16_tensor(xb).cuda()
    y = layer(X)
    y2 = layer(X)                                   # the GEMM library's kernel: the same bits again
    torch.cuda.synchronize()
    layer.handle.check()
    assert torch.equal(y, y2)
    w_hat = W.bf16_bits_to_f32(oracle.decompress(s, oracle.BF16, n_threads=16)[0])
    rows = np.random.default_rng(4).choice(M, 32, replace=False)
    ref = W.bf16_bits_to_f32(xb[rows]) @ w_hat.T
    assert rel_l2(y[rows].float().cpu().numpy(), ref) < 2e-2
    # two more token counts on this weight: M = 1 (fused matrix-vector kernel) and M = 16 (the
    # transposing fused decode + MFMA kernel)
    for m in (1, 16):
        ym = layer(X[:m].contiguous())
        torch.cuda.synchronize()
        refm = W.bf16_bits_to_f32(xb[:m]) @ w_hat.T
        assert rel_l2(ym.float().cpu().numpy(), refm) < 2e-2, m


@pytest.mark.parametrize("M", [256, 512, 1024])
@pytest.mark.parametrize("layout", [0, ep.ROW_LAYOUT])
def test_prefill_forward_through_the_gemm_library(layout, M):
    """From 512 activation rows (from 256 for this N <= 4096) the decoded slices are multiplied by
    hipBLASLt: a ragged N with a
    bias (its bias epilogue) and two slices of a wide K, sampled rows within 2e-2 of the fp32
    product of the oracle's weights, the same bits on a second call, and agreement with the own
    GEMM on the same decoded weight within the fp32 summation order."""
    N, K = 1000, 69632                              # 128 MiB slices of 960 rows: 960 + 40
    w = W.student_t(N, K, seed=12)
    s, _ = ep.compress(w, 4.0, dtype=ep.BF16, layout=layout)
    bias_bits = W.activations(1, N, 13)[0]
    layer = ep.CompressedLinear(s, bf16_tensor(bias_bits).cuda())
    xb = W.activations(M, K, 14)
    X = bf16_tensor(xb).cuda()
    y = layer(X)
    y2 = layer(X)
    wd = layer.handle.decompress(torch.bfloat16)
    yo = ep.gemm_bf16(X, wd)
    torch.cuda.synchronize()
    layer.handle.check()
    assert torch.equal(y, y2)
    b = W.bf16_bits_to_f32(bias_bits).astype(np.float64)
    assert rel_l2(y.float().cpu().numpy(), yo.float().cpu().numpy() + b[None, :]) < 3e-3
    w_hat = W.bf16_bits_to_f32(oracle.decompress(s, oracle.BF16, n_threads=16)[0]).astype(np.float64)
    rows = np.random.default_rng(15).choice(M, 24, replace=False)
    ref = W.bf16_bits_to_f32(xb[rows]).astype(np.float64) @ w_hat.T + b[None, :]
    assert rel_l2(y[rows].float().cpu().numpy(), ref) < 2e-2


def test_c5_linear_forward_token_counts():
    """Fused forward on three matrices of the mixed-rate set (different shapes and rates) at 16
    and 256 tokens: all rows (M = 16) or 32 sampled rows (M = 256) against the oracle-decoded
    weight in fp32."""
    items = W.mixed_rate_set()
    picked, shapes = [], set()
    for R, Cc, t, wseed, aseed in items:
        if (R, Cc) not in shapes and len(picked) < 3:
            shapes.add((R, Cc))
            picked.append((R, Cc, t, wseed, aseed))
    for R, Cc, t, wseed, aseed in picked:
        s, _ = ep.compress(W.student_t(R, Cc, wseed, 0.02), t, dtype=ep.BF16)
        layer = ep.CompressedLinear(s)
        w_hat = W.bf16_bits_to_f32(oracle.decompress(s, oracle.BF16, n_threads=16)[0])
        for M in (16, 256):
            xb = W.activations(M, Cc, aseed)
            y = layer(bf16_tensor(xb).cuda())
            torch.cuda.synchronize()
            layer.handle.check()
            rows = np.arange(M) if M <= 16 else np.random.default_rng(M).choice(M, 32, replace=False)
            ref = W.bf16_bits_to_f32(xb[rows]) @ w_hat.T
            assert rel_l2(y[rows].float().cpu().numpy(), ref) < 2e-2, (R, Cc, t, M)


def test_from_linear_roundtrip():
    lin = torch.nn.Linear(1024, 512, bias=True)
    layer = ep.CompressedLinear.from_linear(lin, 5.0)
    x = torch.randn(8, 1024)
    y = layer(x.cuda().to(torch.bfloat16))
    torch.cuda.synchronize()
    ref = lin(x).detach()
    # lossy 5 bpp weights: the layer output stays close to the original layer
    assert rel_l2(y.float().cpu().numpy(), ref.numpy()) < 0.05
    assert layer.actual_bpp > 5.0


def test_compressed_linear_save_and_reload_in_a_fresh_process(tmp_path):
    """A compressed layer saved to disk and rebuilt by a new process gives the same forward
    output, bit for bit."""
    import os
    import subprocess
    import sys
    lin = torch.nn.Linear(768, 320, bias=True)
    layer = ep.CompressedLinear.from_linear(lin, 4.0)
    x = bf16_tensor(W.activations(24, 768, 77))
    y = layer(x.cuda())
    y8 = ep.CompressedLinear(layer.stream, layer.bias, "fp8")(x.cuda())
    torch.cuda.synchronize()
    path = tmp_path / "layer.npz"
    layer.save(path)
    np.save(tmp_path / "x.npy", W.activations(24, 768, 77))
    out, out8 = tmp_path / "y.npy", tmp_path / "y8.npy"
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys, numpy as np, torch; sys.path.insert(0, %r); import decode_tile_interleaved_rans_amd as ep; "
            "layer = ep.CompressedLinear.load(%r); layer8 = ep.CompressedLinear.load(%r, compute='fp8'); "
            "x = torch.from_numpy(np.load(%r).view(np.int16)).view(torch.bfloat16).cuda(); "
            "y = layer(x); y8 = layer8(x); torch.cuda.synchronize(); "
            "np.save(%r, y.cpu().view(torch.int16).numpy()); np.save(%r, y8.cpu().view(torch.int16).numpy())"
            ) % (root, str(path), str(path), str(tmp_path / "x.npy"), str(out), str(out8))
    subprocess.run([sys.executable, "-c", code], check=True, timeout=300)
    assert np.array_equal(np.load(out), y.cpu().view(torch.int16).numpy())
    assert np.array_equal(np.load(out8), y8.cpu().view(torch.int16).numpy())


# ---------------------------------------------------------------- FP8 forward
# The weight decoded to the FP8 E4M3 container with its row scales (EntroPack paper, Abstract:
# FP8 among the containers) multiplied with per-row E4M3 activations on the FP8 MFMA. Reference:
# the oracle's FP8 decode and activation quantizer, then the exact product of the dequantized
# codes in fp64. The bar, relative L2 <= 3e-3, is set by the BF16 rounding of Y (about 1.1e-3
# RMS); the fp32 accumulation of exact E4M3 products adds far less.
def e4m3(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def fp8_reference(xq, xs, wq, ws, bias=None):
    y = (e4m3(xq) @ e4m3(wq).T) * xs[:, None].astype(np.float64) * ws[None, :].astype(np.float64)
    return y if bias is None else y + bias[None, :]


@pytest.mark.parametrize("M,K", [(1, 16), (7, 784), (300, 2048), (64, 16384)])
def test_quantize_rows_fp8_matches_oracle(M, K):
    rng = np.random.default_rng(M * K)
    x = W.to_bf16_bits(rng.standard_t(3, (M, K)) * np.exp(rng.normal(0, 2, (M, 1))))
    if M > 2:
        x[1] = 0
        x[1, ::3] = 0x8000                         # a zero row with -0.0 entries: codes +0
        x[2] = 0
        x[2, 3] = 0x0001
        x[0, 1] = 0x8000                           # -0.0 in a non-zero row keeps its sign
    q, s = ep.quantize_rows_fp8(bf16_tensor(x).cuda())
    torch.cuda.synchronize()
    qo, so = oracle.quantize_rows_e4m3(x)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(s.cpu().numpy(), so)


# shapes cover every FP8 tile choice: 64 x 32 tiles for M <= 64, 64 x 64, 128 x 128 (2 x 256 of them
# or more) and 256 x 256 (256 or more), with ragged M and N and K not a multiple of the 128 K step
# (2000, 4000, 144), (4100, 4000, 272), (1024, 1000, 2064), (600, 520, 1040) and (300, 1000, 784) go
# to hipBLASLt (512 rows and more, more than 64 with K <= 4096, or 256 and more with N <= 4096)
@pytest.mark.parametrize("M,N,K", [(16, 256, 512), (64, 4100, 1040), (300, 1000, 784), (1, 8, 16),
                                   (2000, 4000, 144), (4100, 4000, 272), (33, 17, 4112), (1024, 1000, 2064),
                                   (600, 520, 1040)])
def test_gemm_fp8_matches_fp64(M, N, K):
    rng = np.random.default_rng(M + N + K)
    x = W.to_bf16_bits(rng.normal(0, 1, (M, K)))
    w = W.to_bf16_bits(rng.standard_t(5, (N, K)) * 0.02)
    xq, xs = oracle.quantize_rows_e4m3(x)
    wq, ws = oracle.quantize_rows_e4m3(w)
    b = W.to_bf16_bits(rng.normal(0, 0.1, N))
    args = (torch.from_numpy(xq).cuda(), torch.from_numpy(xs).cuda(), torch.from_numpy(wq).cuda(),
            torch.from_numpy(ws).cuda())
    y = ep.gemm_fp8(*args, bias=bf16_tensor(b).cuda())
    y2 = ep.gemm_fp8(*args, bias=bf16_tensor(b).cuda())
    torch.cuda.synchronize()
    ref = fp8_reference(xq, xs, wq, ws, W.bf16_bits_to_f32(b).astype(np.float64))
    assert rel_l2(y.float().cpu().numpy(), ref) < 3e-3
    assert torch.equal(y, y2), "two calls must give the same bits"


def fp8_linear_case(M, N, K, target, seed, bias=False, rows=None):
    rng = np.random.default_rng(seed)
    w = (0.02 * rng.standard_t(5, (N, K))).astype(np.float32)
    x = W.to_bf16_bits(rng.normal(0, 1, (M, K)))
    s, _ = ep.compress(w, target)
    b = bf16_tensor(W.to_bf16_bits(rng.normal(0, 0.1, N))).cuda() if bias else None
    layer = ep.CompressedLinear(s, bias=b, compute="fp8")
    y = layer(bf16_tensor(x).cuda())
    torch.cuda.synchronize()
    layer.handle.check()
    rows = np.arange(M) if rows is None else rows
    wq, ws = oracle.decompress(s, oracle.F8E4M3, n_threads=16)
    xq, xs = oracle.quantize_rows_e4m3(x[rows])
    ref = fp8_reference(xq, xs, wq, ws, b.float().cpu().numpy().astype(np.float64) if bias else None)
    w_bf16 = W.bf16_bits_to_f32(oracle.decompress(s, oracle.BF16, n_threads=16)[0])
    ref_bf16 = W.bf16_bits_to_f32(x[rows]) @ w_bf16.T
    if bias:
        ref_bf16 = ref_bf16 + b.float().cpu().numpy()[None, :]
    return y.float().cpu().numpy()[rows], ref, ref_bf16


@pytest.mark.parametrize("M,N,K,target", [(16, 512, 1024, 4.0), (256, 768, 2048, 4.5), (33, 300, 272, 3.0),
                                          (4, 4096, 512, 6.0)])
def test_linear_forward_fp8_matches_quantized_reference(M, N, K, target):
    y, ref, ref_bf16 = fp8_linear_case(M, N, K, target, seed=M + N)
    assert rel_l2(y, ref) < 3e-3
    # FP8 activations and weights against the BF16 path: E4M3 rounding of both operands
    assert rel_l2(y, ref_bf16) < 0.08


def test_linear_forward_fp8_with_bias_and_multi_slice():
    # 9000 x 16384 weight: 128 MiB slices of 8192 rows of E4M3 codes -> two slices, the last ragged
    y, ref, _ = fp8_linear_case(64, 9000, 16384, 4.0, seed=5, bias=True)
    assert rel_l2(y, ref) < 3e-3


def test_linear_forward_fp8_prefill_sampled_rows():
    M, N, K = 4096, 8192, 8192
    w, xb = W.prefill_case()
    s, _ = ep.compress(w, 4.5, dtype=ep.BF16)
    layer = ep.CompressedLinear(s, compute="fp8")
    y = layer(bf16_tensor(xb).cuda())
    y2 = layer(bf16_tensor(xb).cuda())              # the GEMM library's kernel: the same bits again
    torch.cuda.synchronize()
    layer.handle.check()
    assert torch.equal(y, y2)
    rows = np.random.default_rng(6).choice(M, 32, replace=False)
    wq, ws = oracle.decompress(s, oracle.F8E4M3, n_threads=16)
    xq, xs = oracle.quantize_rows_e4m3(xb[rows])
    assert rel_l2(y[rows].float().cpu().numpy(), fp8_reference(xq, xs, wq, ws)) < 3e-3


@pytest.mark.parametrize("M", [256, 512, 1024])
def test_fp8_prefill_with_bias_over_two_slices(M):
    """The FP8 forward from 512 rows (256 for this N; slices multiplied by hipBLASLt with the row scales as
    outer-vector scales): a ragged N with a bias over two slices, against the fp64 product of the
    oracle's codes and scales, repeatable bits."""
    N, K = 1000, 139264                             # 128 MiB FP8 slices of 960 rows: 960 + 40
    w = W.student_t(N, K, seed=16)
    s, _ = ep.compress(w, 4.0, dtype=ep.BF16)
    bias_bits = W.activations(1, N, 17)[0]
    layer = ep.CompressedLinear(s, bf16_tensor(bias_bits).cuda(), compute="fp8")
    xb = W.activations(M, K, 18)
    X = bf16_tensor(xb).cuda()
    y = layer(X)
    y2 = layer(X)
    torch.cuda.synchronize()
    layer.handle.check()
    assert torch.equal(y, y2)
    rows = np.random.default_rng(19).choice(M, 16, replace=False)
    wq, ws = oracle.decompress(s, oracle.F8E4M3, n_threads=16)
    xq, xs = oracle.quantize_rows_e4m3(xb[rows])
    ref = fp8_reference(xq, xs, wq, ws, W.bf16_bits_to_f32(bias_bits).astype(np.float64))
    assert rel_l2(y[rows].float().cpu().numpy(), ref) < 3e-3


def test_binding_refuses_mismatched_tensors():
    """The kernels trust the sizes they are given, so the binding checks every tensor before its
    pointer crosses the C ABI: wrong shapes, dtypes or layouts raise before anything is launched."""
    w = W.student_t(64, 256, 21)
    s, _ = ep.compress(w, 4.0, dtype=ep.BF16)
    layer = ep.CompressedLinear(s)
    with pytest.raises(ValueError):
        layer(torch.zeros((4, 255), dtype=torch.bfloat16, device="cuda"))          # wrong in_features
    x = torch.zeros((32, 256), dtype=torch.bfloat16, device="cuda")
    wt = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        ep.gemm_bf16(x, torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda"))  # K mismatch
    with pytest.raises(ValueError):
        ep.gemm_bf16(x, wt.float())                                                  # wrong dtype
    with pytest.raises(ValueError):
        ep.gemm_bf16(x.t().contiguous().t(), wt)                                      # not row-major
    xq, xs = ep.quantize_rows_fp8(x)
    wq, ws = ep.quantize_rows_fp8(wt)
    with pytest.raises(ValueError):
        ep.gemm_fp8(xq, xs[:16].contiguous(), wq, ws)                               # short scales
    h = ep.upload(s)
    with pytest.raises(ValueError):
        ep.decompress_many([h], [torch.empty((64, 128), dtype=torch.bfloat16, device="cuda")])
    with pytest.raises(ValueError):
        h.decompress_into(torch.empty((64, 256), dtype=torch.float8_e4m3fn, device="cuda"),
                          torch.empty(8, dtype=torch.float32, device="cuda"))         # short row scales
    torch.cuda.synchronize()


def test_forward_on_two_streams_at_once():
    """Each (device, stream) pair owns its forward workspace: two layers running on two HIP
    streams at the same time (decode-once slices and the fused matrix-vector path) give the same
    bits as the same calls one after the other on the default stream."""
    rng = np.random.default_rng(31)
    ws = [(0.02 * rng.standard_t(5, (1536, 2048))).astype(np.float32) for _ in range(2)]
    layers = [ep.CompressedLinear(ep.compress(w, 4.0)[0]) for w in ws]
    xs = [bf16_tensor(W.to_bf16_bits(rng.normal(0, 1, (m, 2048)))).cuda() for m in (300, 3)]
    want = [layers[i](xs[i]) for i in range(2)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [None, None]
    for _ in range(3):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                got[i] = layers[i](xs[i], stream=streams[i])
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(got[i], want[i]) or (xs[i].shape[0] <= 4 and
                                                    rel_l2(got[i].float().cpu().numpy(),
                                                           want[i].float().cpu().numpy()) < 1e-2)


def test_forward_on_a_side_stream_with_fp32_input():
    """fp32 activations need cast=True (no silent precision change); with an explicit side stream
    the conversion and the output live on that stream, which waits for the producer of x."""
    w = W.student_t(512, 1024, seed=61)
    s, _ = ep.compress(w, 4.0, dtype=ep.BF16)
    layer = ep.CompressedLinear(s)
    want, _ = oracle.decompress(s, oracle.BF16)
    xf = torch.randn(40, 1024, generator=torch.Generator().manual_seed(3))
    x = xf.cuda()                                   # fp32, produced on the current stream
    with pytest.raises(ValueError):
        layer(x)
    side = torch.cuda.Stream()
    y = layer.forward(x * 1.0, stream=side, cast=True)
    side.synchronize()
    layer.handle.check()
    xb = xf.to(torch.bfloat16).float().numpy().astype(np.float64)
    ref = xb @ W.bf16_bits_to_f32(want).astype(np.float64).T
    assert rel_l2(y.float().cpu().numpy(), ref) < 2e-2


def test_helpers_on_a_side_stream_match_the_current_stream():
    """gemm_bf16, quantize_rows_fp8, gemm_fp8 and decode_symbols with an explicit side stream:
    the side stream waits for the producer of the inputs (queued on the current stream just
    before), the outputs are allocated on it, and the results are the bits of the same calls on
    the current stream (every one of these kernels is deterministic)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(8)
    a = torch.randn(300, 1040, generator=g, device="cuda")
    wf = torch.randn(520, 1040, generator=g, device="cuda")
    s, _ = ep.compress(W.student_t(256, 1024, seed=62), 4.0, dtype=ep.BF16)
    h = ep.upload(s)
    side = torch.cuda.Stream()
    results = []
    for stream in (None, side):
        x = (a * 0.5).to(torch.bfloat16)            # produced on the current stream right before the calls
        w = (wf * 0.25).to(torch.bfloat16)
        y = ep.gemm_bf16(x, w, stream=stream)
        xq, xs = ep.quantize_rows_fp8(x, stream=stream)
        wq, ws = ep.quantize_rows_fp8(w, stream=stream)
        y8 = ep.gemm_fp8(xq, xs, wq, ws, stream=stream)
        q = h.decode_symbols(stream=stream)
        del x, w                                     # the allocator must not reuse them while `side` reads
        if stream is not None:
            stream.synchronize()
        torch.cuda.synchronize()
        results.append((y, xq, xs, y8, q))
    h.check()
    for u, v in zip(*results):
        assert torch.equal(u, v)
    qo, _ = oracle.decode_symbols(s)
    assert np.array_equal(results[1][4].cpu().numpy(), qo)


def test_matrix_vector_and_gemm_paths_agree():
    """M <= 4 on a layout-0 stream forms the products inside the decode and M >= 5 in the GEMM of
    decoded slices; both multiply the BF16-rounded weights, so the same rows differ only by the fp32
    summation order and the final rounding. The matrix-vector path stores per-pair partials added in
    column order: two calls give the same bits. Both are checked against the fp64 product of the
    oracle-decoded BF16 weights."""
    w = W.student_t(2048, 4096, seed=62)
    s, _ = ep.compress(w, 4.5, dtype=ep.BF16)
    layer = ep.CompressedLinear(s)
    xb = W.activations(5, 4096, 63)
    x = bf16_tensor(xb).cuda()
    y4a = layer(x[:4].contiguous())
    y4b = layer(x[:4].contiguous())
    y5 = layer(x).float().cpu().numpy()
    torch.cuda.synchronize()
    layer.handle.check()
    assert torch.equal(y4a, y4b)
    y4 = y4a.float().cpu().numpy()
    d = rel_l2(y4, y5[:4])
    print(f"M=4 (fused matrix-vector) vs M=5 (decode + GEMM): relative L2 {d:.2e}")
    assert d < 1e-3
    want, _ = oracle.decompress(s, oracle.BF16)
    ref = W.bf16_bits_to_f32(xb).astype(np.float64) @ W.bf16_bits_to_f32(want).astype(np.float64).T
    assert rel_l2(y4, ref[:4]) < 5e-3 and rel_l2(y5, ref) < 5e-3


@pytest.mark.parametrize("M,N,K", [(256, 8192, 2048), (300, 1000, 776), (512, 2048, 4096)])
def test_split_k_gemm_is_deterministic_and_exact_to_fp32(M, N, K):
    """Too few 256 x 256 tiles to fill the CUs: the K splits' fp32 partial tiles are added in split
    order, so two calls give the same bits, and the result stays within the fp32 reference's bar."""
    rng = np.random.default_rng(M + K)
    x = W.to_bf16_bits(rng.normal(0, 1, (M, K)))
    w = W.to_bf16_bits(rng.normal(0, 0.05, (N, K)))
    X, Wt = bf16_tensor(x).cuda(), bf16_tensor(w).cuda()
    y1 = ep.gemm_bf16(X, Wt)
    y2 = ep.gemm_bf16(X, Wt)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    ref = W.bf16_bits_to_f32(x) @ W.bf16_bits_to_f32(w).T
    assert rel_l2(y1.float().cpu().numpy(), ref) < 5e-3


@pytest.mark.parametrize("compute", ["bf16", "fp8"])
@pytest.mark.parametrize("layout", [0, ep.ROW_LAYOUT])
def test_forward_with_no_input_features(layout, compute):
    """in_features 0: every product is an empty sum, so Y = bias (or zeros) on every path (the
    matrix-vector, fused and slice paths all take M here), and X may have no storage."""
    s, _ = ep.compress(np.zeros((40, 0), np.float32), 4.0, layout=layout)
    bias_bits = W.activations(1, 40, 7)[0]
    for bias in (None, bf16_tensor(bias_bits).cuda()):
        layer = ep.CompressedLinear(s, bias, compute=compute)
        for M in (1, 5, 40, 100):
            y = layer(torch.empty((M, 0), dtype=torch.bfloat16, device="cuda"))
            torch.cuda.synchronize()
            want = torch.zeros((M, 40), dtype=torch.bfloat16) if bias is None else bias.cpu()[None, :].expand(M, 40)
            assert torch.equal(y.cpu(), want), (M, bias is None)


def test_fused_forwards_on_two_streams_and_interleaved_layers():
    """Fused forwards share nothing between calls but their stream's workspace: row-layout layers
    of different heights called in turn on one stream, and on two streams at once (each stream with
    its own workspace), give the bits of the first calls, BF16 and FP8."""
    rng = np.random.default_rng(41)
    shapes = [(2048, 1536), (520, 1024), (4096, 512)]
    layers = []
    for i, (N, K) in enumerate(shapes):
        w = (0.02 * rng.standard_t(5, (N, K))).astype(np.float32)
        s, _ = ep.compress(w, 4.0, prob_bits=ep.LAYER_PROB_BITS, layout=ep.ROW_LAYOUT)
        b = bf16_tensor(W.to_bf16_bits(rng.normal(0, 0.1, N))).cuda() if i != 1 else None
        layers += [ep.CompressedLinear(s, b), ep.CompressedLinear(s, b, compute="fp8")]
    ms = [16, 40, 64, 3, 33, 1]
    xs = [bf16_tensor(W.to_bf16_bits(rng.normal(0, 1, (m, lay.in_features)))).cuda() for m, lay in zip(ms, layers)]
    want = [lay(x) for lay, x in zip(layers, xs)]
    torch.cuda.synchronize()
    for lay in layers:
        lay.handle.check()
    for _ in range(2):                               # in turn, reversed order, one stream
        got = [lay(x) for lay, x in reversed(list(zip(layers, xs)))][::-1]
        torch.cuda.synchronize()
        assert all(torch.equal(g, w_) for g, w_ in zip(got, want))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(3):                               # two streams at once
        got = [None] * len(layers)
        for i, (lay, x) in enumerate(zip(layers, xs)):
            st = streams[i % 2]
            with torch.cuda.stream(st):
                got[i] = lay(x, stream=st)
        torch.cuda.synchronize()
        assert all(torch.equal(g, w_) for g, w_ in zip(got, want))


def test_gemm_library_plan_cache_keeps_working_past_its_limit():
    """hipBLASLt plans are cached per shape up to a fixed count, least recently used out first:
    140 distinct row counts through the plain FP8 GEMM (hipBLASLt from 512 rows), then the first
    shape again, which gets a new plan and the same bits; sampled results match the fp64 product."""
    rng = np.random.default_rng(77)
    N, K = 256, 256
    w = W.to_bf16_bits(rng.standard_t(5, (N, K)) * 0.02)
    wq, ws = oracle.quantize_rows_e4m3(w)
    wq_t, ws_t = torch.from_numpy(wq).cuda(), torch.from_numpy(ws).cuda()
    x = W.to_bf16_bits(rng.normal(0, 1, (1024 + 140, K)))
    xq, xs = oracle.quantize_rows_e4m3(x)
    xq_t, xs_t = torch.from_numpy(xq).cuda(), torch.from_numpy(xs).cuda()
    first = None
    for M in range(1024, 1024 + 140):
        y = ep.gemm_fp8(xq_t[:M].contiguous(), xs_t[:M].contiguous(), wq_t, ws_t)
        if M == 1024:
            first = y.clone()
        if M % 35 == 0:
            torch.cuda.synchronize()
            ref = fp8_reference(xq[:M], xs[:M], wq, ws, None)
            assert rel_l2(y.float().cpu().numpy(), ref) < 3e-3, M
    again = ep.gemm_fp8(xq_t[:1024].contiguous(), xs_t[:1024].contiguous(), wq_t, ws_t)
    torch.cuda.synchronize()
    assert torch.equal(again, first)


@pytest.mark.parametrize("layout", [0, ep.ROW_LAYOUT])
def test_benchmark_weight_every_forward_path(layout):
    """The 8192 x 8192 benchmark weight coded as the benchmark codes it (4.5 bpp target, the layers'
    11-bit probabilities) in each tile layout, through every forward path the benchmark times:
    M = 1 and 4 (matrix-vector kernel in layout 0, register-direct fused kernel in the row layout),
    16, 32 and 64 (fused kernels), 256 (decode-once slice + split-K GEMM) and 4096 (slice +
    hipBLASLt), BF16 and FP8. Sampled rows within 5e-3 (BF16) of the fp64 product of the oracle's
    BF16 weights and within 3e-3 (FP8) of the product of the oracle's E4M3 codes and scales."""
    w, xb = W.prefill_case()
    s, _ = ep.compress(w, 4.5, dtype=ep.BF16, prob_bits=ep.LAYER_PROB_BITS, layout=layout)
    layer, layer8 = ep.CompressedLinear(s), ep.CompressedLinear(s, compute="fp8")
    w_hat = W.bf16_bits_to_f32(oracle.decompress(s, oracle.BF16, n_threads=16)[0]).astype(np.float64)
    wq, ws = oracle.decompress(s, oracle.F8E4M3, n_threads=16)
    X = bf16_tensor(xb).cuda()
    rng = np.random.default_rng(layout + 40)
    for M in (1, 4, 16, 32, 64, 256, 4096):
        rows = np.sort(rng.choice(M, min(M, 12), replace=False))
        y = layer(X[:M].contiguous())
        y8 = layer8(X[:M].contiguous())
        torch.cuda.synchronize()
        layer.handle.check()
        ref = W.bf16_bits_to_f32(xb[rows]).astype(np.float64) @ w_hat.T
        assert rel_l2(y[rows].float().cpu().numpy(), ref) < 5e-3, ("bf16", M)
        xq, xs = oracle.quantize_rows_e4m3(xb[:M])
        ref8 = fp8_reference(xq[rows], xs[rows], wq, ws)
        assert rel_l2(y8[rows].float().cpu().numpy(), ref8) < 3e-3, ("fp8", M)
