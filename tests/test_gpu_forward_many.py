"""The grouped compressed linear forward (ep_linear_forward_many): layers that take the same input
are decoded into the BF16 MFMA by one launch when they are row-layout streams with one prob_bits
and M <= 64; above 64 rows, when every layer would be one whole-layer slice multiplied by
hipBLASLt, their slices are decoded by one grouped launch and multiplied one by one. Either way
each layer must give the same bits as its own forward (the same partial sums added in the same
order, or the same slices and GEMMs); other groups run the layers one by one. Cases: ragged shapes
and biases at M = 1, 16, 33, 64 (one to four M tiles), grouped slices at 100 and 600 rows with
mixed tile layouts, the DiT-like gate and up projections at 16 and 256 rows, the fallbacks (a
layout-0 layer, mixed prob_bits, M = 65 with K > 4096 rows for the own GEMM), the fp64 product of
the oracle's weights, and the C ABI refusing layers of different input widths before any launch."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import decode_tile_interleaved_rans_amd as ep
from decode_tile_interleaved_rans_amd import workloads as W

pytestmark = pytest.mark.gpu


def bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def layer(N, K, seed, layout=ep.ROW_LAYOUT, prob_bits=11, bias=True, target=4.5):
    w = W.student_t(N, K, seed)
    s, _ = ep.compress(w, target, dtype=ep.BF16, layout=layout, prob_bits=prob_bits)
    b = bf16(W.activations(1, N, seed + 1)[0]).cuda() if bias else None
    return ep.CompressedLinear(s, b), s, b


def same_as_own_forwards(layers, x):
    ys = ep.linear_forward_many(layers, x)
    want = [l(x) for l in layers]
    torch.cuda.synchronize()
    for l in layers:
        l.handle.check()
    for i, (y, w_) in enumerate(zip(ys, want)):
        assert y.shape == w_.shape
        assert torch.equal(y, w_), f"layer {i}"
    return ys


@pytest.mark.parametrize("M", [1, 16, 33, 64])
def test_group_equals_each_layer(M):
    K = 768                                       # one and a half tile pairs per tile row
    layers = [layer(N, K, sd, bias=sd % 2 == 1)[0] for N, sd in [(300, 1), (1000, 2), (512, 3), (16, 4)]]
    same_as_own_forwards(layers, bf16(W.activations(M, K, 9)).cuda())


def test_group_against_the_oracle():
    K, M = 1024, 24
    built = [layer(N, K, sd) for N, sd in [(200, 11), (96, 12)]]
    xb = W.activations(M, K, 13)
    ys = same_as_own_forwards([b[0] for b in built], bf16(xb).cuda())
    x64 = W.bf16_bits_to_f32(xb).astype(np.float64)
    for y, (_, s, b) in zip(ys, built):
        wq, _ = oracle.decompress(s, oracle.BF16)
        ref = x64 @ W.bf16_bits_to_f32(wq).astype(np.float64).T + b.float().cpu().numpy().astype(np.float64)
        got = y.float().cpu().numpy()
        assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 5e-3


@pytest.mark.parametrize("M", [16, 256])
def test_dit_like_gate_and_up(M):
    R, K = W.DIT_BLOCK_SHAPES[2]                  # [10240, 3840] twice: 4800 tile pairs each
    layers = [layer(R, K, sd, bias=False, target=4.0)[0] for sd in (21, 22)]
    same_as_own_forwards(layers, bf16(W.activations(M, K, 23)).cuda())


@pytest.mark.parametrize("M", [100, 600])
def test_prefill_group_slices(M):
    K = 1024
    layers = [layer(N, K, sd, bias=sd % 2 == 0, layout=lay)[0]
              for N, sd, lay in [(700, 51, ep.ROW_LAYOUT), (256, 52, 0), (1000, 53, ep.ROW_LAYOUT)]]
    same_as_own_forwards(layers, bf16(W.activations(M, K, 54)).cuda())


@pytest.mark.parametrize("case", ["layout0", "prob_bits", "M65", "one"])
def test_groups_that_run_layer_by_layer(case):
    K = 512
    a = layer(160, K, 31)[0]
    if case == "layout0":
        layers, M = [a, layer(96, K, 32, layout=0)[0]], 16
    elif case == "prob_bits":
        layers, M = [a, layer(96, K, 33, prob_bits=12)[0]], 8
    elif case == "M65":
        K = 4608                                  # above 4096: the own GEMM, layer by layer
        layers, M = [layer(160, K, 36)[0], layer(96, K, 34)[0]], 65
    else:
        layers, M = [a], 5
    same_as_own_forwards(layers, bf16(W.activations(M, K, 35)).cuda())


def test_abi_refuses_different_input_widths():
    a, b = layer(64, 512, 41)[0], layer(64, 768, 42)[0]
    x = bf16(W.activations(4, 512, 43)).cuda()
    ys = [torch.empty((4, 64), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    hs = (C.c_void_p * 2)(a.handle.ptr.value, b.handle.ptr.value)
    os_ = (C.c_void_p * 2)(*[y.data_ptr() for y in ys])
    rc = ep.lib().ep_linear_forward_many(hs, 2, C.c_void_p(x.data_ptr()), 4, None, os_,
                                         C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == -1 and b"widths" in ep.lib().ep_last_error()
    with pytest.raises(ValueError):
        ep.linear_forward_many([a, b], x)


@pytest.mark.parametrize("M", [1, 16, 64, 80])
def test_fp8_group_equals_each_layer(M):
    """ep_linear_forward_fp8_many: the activations quantized once for the group, every layer the
    same bits as its own FP8 forward (one launch up to 64 rows, layer by layer above)."""
    K = 768
    built = [layer(N, K, sd, bias=sd % 2 == 1) for N, sd in [(300, 61), (512, 62), (40, 63)]]
    layers = [ep.CompressedLinear(s, b, compute="fp8") for _, s, b in built]
    same_as_own_forwards(layers, bf16(W.activations(M, K, 64)).cuda())
