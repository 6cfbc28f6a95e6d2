"""The decode fused into the compressed linear layer's matrix product (5 <= M <= 16 activation rows;
larger M takes the decode-then-GEMM path, which the M = 17 ... 64 cases below cover):
every tile pair decoded straight into the B operand of the BF16 MFMA through LDS, never written
out ("EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary Bitrates",
Abstract; "EntroPack PyTorch Guide", section "Replace one linear layer before a whole model").

Reference: the oracle's BF16 decode of the same stream, multiplied by the BF16 activations in
fp64 on the CPU. The fused path multiplies exactly those BF16 weights with fp32 accumulation, so
besides the 2e-2 bar it must stay at the level of the fp32 summation and the final BF16 rounding
(5e-3). Cases: every M tile count (M = 5 ... 64, ragged M), ragged N and K (K not a multiple of
512, an odd number of 256-column tiles so that the last pair holds one tile), prob_bits 10 / 11 /
12 (12 and 8 waves per CU), bias, escapes, a full-size matrix, and run-to-run determinism."""
import numpy as np
import pytest
import torch

import oracle
import decode_tile_interleaved_rans_amd as ep
from decode_tile_interleaved_rans_amd import workloads as W

pytestmark = pytest.mark.gpu


def rel_l2(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))


def bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def check(N, K, M, target=4.0, prob_bits=12, seed=0, bias=False, outliers=False):
    if outliers:
        w = W.gaussian_with_outliers(N, K, seed=seed, outlier_frac=0.003)
        s, _ = ep.compress(w, target, prob_bits=prob_bits)
    else:
        w = W.student_t(N, K, seed=seed)
        s, _ = ep.compress(w, target, dtype=ep.BF16, prob_bits=prob_bits)
    b = W.activations(1, N, seed + 1)[0] if bias else None
    layer = ep.CompressedLinear(s, bf16(b).cuda() if bias else None)
    xb = W.activations(M, K, seed + 2)
    x = bf16(xb).cuda()
    y = layer(x)
    y2 = layer(x)
    torch.cuda.synchronize()
    layer.handle.check()
    want, _ = oracle.decompress(s, oracle.BF16)
    ref = W.bf16_bits_to_f32(xb).astype(np.float64) @ W.bf16_bits_to_f32(want).astype(np.float64).T
    if bias:
        ref += W.bf16_bits_to_f32(b).astype(np.float64)[None, :]
    got = y.float().cpu().numpy()
    err = rel_l2(got, ref)
    assert err < 5e-3, (N, K, M, prob_bits, err)
    assert torch.equal(y, y2), "two calls must give the same bits"
    return s, layer, err


@pytest.mark.parametrize("M", [5, 16, 17, 32, 33, 48, 64])
def test_every_m_tile_count(M):
    check(256, 1024, M, seed=M)


@pytest.mark.parametrize("N,K", [(200, 776), (48, 520), (17, 256), (1000, 3072), (64, 8)])
def test_ragged_shapes(N, K):
    check(N, K, 24, seed=N + K, bias=True)


@pytest.mark.parametrize("prob_bits", [10, 11, 12])
def test_probability_precisions(prob_bits):
    check(512, 2048, 16, prob_bits=prob_bits, seed=prob_bits)


def test_escapes():
    s, _, _ = check(128, 1024, 40, target=8.0, seed=5, outliers=True)
    assert ep.stream_info(s)["n_escapes"] > 0


def test_full_size_layer_against_the_gemm_path():
    """The 8192 x 8192 benchmark weight at M = 16: the fused result equals, within the fp32
    summation order, the decode-then-GEMM result on the same BF16 weight (M = 65 takes the slice
    path; its first 16 rows are computed from the same weights)."""
    wb, xb = W.prefill_case()
    s, _ = ep.compress(wb, 4.5, dtype=ep.BF16)
    layer = ep.CompressedLinear(s)
    x = bf16(xb[:65]).cuda()
    y16 = layer(x[:16].contiguous())
    y65 = layer(x)
    torch.cuda.synchronize()
    layer.handle.check()
    assert rel_l2(y16.float().cpu().numpy(), y65[:16].float().cpu().numpy()) < 3e-3
    want, _ = oracle.decompress(s, oracle.BF16)
    rows = [0, 7, 15]
    ref = W.bf16_bits_to_f32(xb[rows]).astype(np.float64) @ W.bf16_bits_to_f32(want).astype(np.float64).T
    assert rel_l2(y16[rows].float().cpu().numpy(), ref) < 5e-3


def e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


@pytest.mark.parametrize("N,K,M,prob_bits", [(256, 1024, 16, 12), (200, 784, 12, 11), (48, 528, 9, 10),
                                             (1000, 2048, 5, 11), (64, 1040, 40, 11)])
def test_fp8_fused_matches_oracle_codes(N, K, M, prob_bits):
    """The FP8 forward for M <= 16 (the weight decoded into E4M3 codes straight into the B operand of
    the FP8 MFMA): within 3e-3 of the fp64 product of the oracle's E4M3 weight codes and row scales
    and the oracle's per-row activation codes and scales (K = 784 and 528: the last 32-code chunk
    of a lane half past K; M = 40 takes the decode-then-GEMM path)."""
    w = W.student_t(N, K, seed=N + K)
    s, _ = ep.compress(w, 4.5, dtype=ep.BF16, prob_bits=prob_bits)
    bias_bits = W.activations(1, N, 3)[0]
    layer = ep.CompressedLinear(s, bf16(bias_bits).cuda(), compute="fp8")
    xb = W.activations(M, K, N + M)
    x = bf16(xb).cuda()
    y = layer(x)
    y2 = layer(x)
    torch.cuda.synchronize()
    layer.handle.check()
    wq, ws = oracle.decompress(s, oracle.F8E4M3)
    xq, xs = oracle.quantize_rows_e4m3(xb)
    ref = (e4m3(xq) @ e4m3(wq).T) * xs[:, None].astype(np.float64) * ws[None, :].astype(np.float64)
    ref += W.bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
    assert rel_l2(y.float().cpu().numpy(), ref) < 3e-3
    assert torch.equal(y, y2)
