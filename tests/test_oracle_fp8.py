"""Pins of the oracle's FP8 activation quantizer (the FP8 linear forward: weights decoded to the
FP8 container, "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary
Bitrates", Abstract, multiplied with FP8 activations). Reading: per-row scale s = amax / 448,
codes E4M3(x * (448 / amax)) with the saturating round-to-nearest-even cast.

Pins: hand-worked codes; torch's float8_e4m3fn cast applied to the same fp32 products; the row
maximum maps to +-448; dequantized values within the E4M3 half-step of the input; zero rows."""
import numpy as np
import pytest
import torch

import oracle
from decode_tile_interleaved_rans_amd import workloads as W


def e4m3_values(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def test_hand_worked_row():
    # [1, -2, 4]: amax 4, scaled values 112, -224, 448 are all exact E4M3 numbers:
    # 112 = 1.75 * 2^6 -> (13 << 3) | 6 = 110; -224 -> 0x80 | (14 << 3) | 6 = 246; 448 -> 0x7E
    x = np.array([[0x3F80, 0xC000, 0x4080]], np.uint16)
    q, s = oracle.quantize_rows_e4m3(x)
    assert list(q[0]) == [110, 246, 126]
    assert s[0] == np.float32(4.0) / np.float32(448.0)


def test_matches_torch_cast_of_the_scaled_rows():
    rng = np.random.default_rng(3)
    x = W.to_bf16_bits(rng.normal(0, 1, (64, 777)) * np.exp(rng.normal(0, 3, (64, 1))))
    q, s = oracle.quantize_rows_e4m3(x)
    xf = W.bf16_bits_to_f32(x)
    amax = np.abs(xf).max(1).astype(np.float32)
    assert np.array_equal(s, amax / np.float32(448.0))
    inv = (np.float32(448.0) / amax).astype(np.float32)
    prod = (xf * inv[:, None]).astype(np.float32)
    want = torch.from_numpy(prod).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, want)


def test_row_maximum_and_error_bound():
    rng = np.random.default_rng(4)
    x = W.to_bf16_bits(rng.standard_t(3, (32, 512)))
    q, s = oracle.quantize_rows_e4m3(x)
    xf = W.bf16_bits_to_f32(x).astype(np.float64)
    v = e4m3_values(q).astype(np.float64)
    assert np.all(np.abs(v).max(1) == 448.0)
    deq = v * s[:, None].astype(np.float64)
    scaled = xf * (448.0 / np.abs(xf).max(1))[:, None]
    # normal E4M3 range: relative error <= 2^-4 (half of the 3-bit mantissa step); below 2^-6
    # the subnormal grid of 2^-9 bounds the absolute error by 2^-10 in scaled units
    big = np.abs(scaled) >= 2.0 ** -6
    assert np.all(np.abs(v - scaled)[big] <= np.abs(scaled)[big] * 2.0 ** -4 * (1 + 1e-6))
    assert np.all(np.abs(v - scaled)[~big] <= 2.0 ** -10 * (1 + 1e-6))
    assert np.allclose(deq, xf, rtol=2.0 ** -4 * 1.01, atol=float(s.max()) * 2.0 ** -10 * 1.01)


def test_zero_and_tiny_rows():
    x = np.zeros((3, 40), np.uint16)
    x[1, 5] = 0x0001                              # smallest bf16 subnormal, 2^-133
    x[2, :] = 0x8000                              # -0.0 everywhere
    q, s = oracle.quantize_rows_e4m3(x)
    assert s[0] == 0.0 and not q[0].any()
    # amax below 2^-100 is raised to 2^-100 (448 / amax stays finite): 2^-133 scales to
    # 448 * 2^-33, below half the smallest E4M3 subnormal, so every code is 0
    assert s[1] == np.float32(2.0 ** -100) / np.float32(448.0) and not q[1].any()
    assert s[2] == 0.0 and not q[2].any()
    x[1, 6] = 0x0D80                              # 2^-100: now the row maximum, code 448
    q, s = oracle.quantize_rows_e4m3(x)
    assert q[1, 6] == 126 and q[1, 5] == 0


def test_non_finite_input_is_rejected():
    x = np.zeros((1, 8), np.uint16)
    x[0, 3] = 0x7F80
    with pytest.raises(oracle.OracleError) as e:
        oracle.quantize_rows_e4m3(x)
    assert e.value.rc == -4
