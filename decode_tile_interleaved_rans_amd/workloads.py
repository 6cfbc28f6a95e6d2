"""Seeded synthetic inputs for the tile-rANS weight codec.

This module only draws random numbers and casts them to the stored element types: it holds none
of the codec's arithmetic, and both the GPU path's tests and the oracle's tests take their inputs
from it. The pages' only workload is a trained image generator whose weights are not available,
so these recipes stand in for it (shapes of a 30-block DiT-like denoiser with hidden size 3840;
heavy-tailed Student-t weights with per-row scale spread; 0.1% large outliers).

Every generator returns numpy arrays. BF16 tensors are returned as uint16 bit patterns (fp64 draw
-> fp32 -> bf16 round-to-nearest-even via torch on the CPU).
"""
from __future__ import annotations

import numpy as np

DIT_BLOCK_SHAPES = [  # [out_features, in_features] of one DiT-like block
    (11520, 3840),    # fused QKV projection
    (3840, 3840),     # attention output projection
    (10240, 3840),    # FFN gate
    (10240, 3840),    # FFN up
    (3840, 10240),    # FFN down
]
DIT_BLOCKS = 30


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def gaussian_with_outliers(rows: int = 1024, cols: int = 1024, seed: int = 1, sigma: float = 0.02,
                           outlier_frac: float = 0.001) -> np.ndarray:
    """fp32 [rows, cols]: N(0, sigma^2), with round(outlier_frac * numel) entries (chosen without
    replacement) replaced by +-U(0.1, 0.3) with random signs."""
    rng = np.random.default_rng(seed)
    w = rng.normal(0.0, sigma, (rows, cols))
    k = int(round(outlier_frac * rows * cols))
    idx = rng.choice(rows * cols, size=k, replace=False)
    sign = np.where(rng.random(k) < 0.5, -1.0, 1.0)
    w.reshape(-1)[idx] = sign * rng.uniform(0.1, 0.3, k)
    return w.astype(np.float32)


def student_t_rowscaled(rows: int = 4096, cols: int = 4096, seed: int = 2, scale: float = 0.015,
                        row_sigma: float = 0.5) -> np.ndarray:
    """bf16 bits [rows, cols]: scale * t(nu=5), each row multiplied by exp(N(0, row_sigma^2))."""
    rng = np.random.default_rng(seed)
    w = scale * rng.standard_t(5, (rows, cols))
    w *= np.exp(rng.normal(0.0, row_sigma, rows))[:, None]
    return to_bf16_bits(w)


def student_t(rows: int, cols: int, seed: int, scale: float = 0.02) -> np.ndarray:
    """bf16 bits [rows, cols]: scale * t(nu=5)."""
    rng = np.random.default_rng(seed)
    return to_bf16_bits(scale * rng.standard_t(5, (rows, cols)))


def activations(rows: int, cols: int, seed: int) -> np.ndarray:
    """bf16 bits [rows, cols]: N(0, 1)."""
    rng = np.random.default_rng(seed)
    return to_bf16_bits(rng.normal(0.0, 1.0, (rows, cols)))


def dit_matrix(block: int, m: int) -> np.ndarray:
    """Matrix m of block b of the 30-block DiT-like model (seed 3000 + 5b + m)."""
    R, Cc = DIT_BLOCK_SHAPES[m]
    return student_t(R, Cc, 3000 + 5 * block + m, 0.02)


def mixed_rate_set(count: int = 64, seed: int = 5):
    """The mixed-rate stress set: per matrix (rows, cols, target_bpp, weight seed, activation seed)
    with rows, cols drawn from {2048, 4096, 8192} and the target uniform in [2.5, 6.0]."""
    rng = np.random.default_rng(seed)
    sizes = np.array([2048, 4096, 8192])
    out = []
    for i in range(count):
        R = int(rng.choice(sizes))
        Cc = int(rng.choice(sizes))
        t = float(rng.uniform(2.5, 6.0))
        out.append((R, Cc, t, 100000 + i, 500 + i))
    return out


def gpu_student_t(rows: int, cols: int, seed: int, scale: float = 0.02):
    """scale * t(nu=5) as a BF16 torch tensor drawn on the current GPU: z / sqrt(chi2_5 / 5) from six
    normals of torch's generator seeded with `seed`, so that large weight sets need no host
    generation (the benchmark's full-model and mixed-rate sets, and their parity tests)."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    z = torch.randn((rows, cols), generator=g, device="cuda")
    v = torch.zeros((rows, cols), device="cuda")
    for _ in range(5):
        v += torch.randn((rows, cols), generator=g, device="cuda").square()
    return (scale * z / torch.sqrt(v / 5.0)).to(torch.bfloat16)


def prefill_case(seed_w: int = 4, seed_x: int = 4004, n: int = 8192, k: int = 8192, m: int = 4096):
    """Fused-GEMM prefill case: W bf16 [n, k] = 0.02 t5 and X bf16 [m, k] ~ N(0, 1)."""
    return student_t(n, k, seed_w, 0.02), activations(m, k, seed_x)
