"""The no-allocation linear forward (ep_linear_forward_noalloc, for callers that cannot allocate
device memory) against the pool-workspace forward (ep_linear_forward), both called through the C
ABI, on two calls in a row with the second smaller than the first, on every forward path: for a
layout-0 stream the fused matrix-vector products (M <= 4), the transposing fused decode + MFMA
kernel (5 <= M <= 16) and decode slices + GEMM above; for a row-layout stream the register-direct
fused kernel (M <= 64, one to four M tiles) and the slices above. Collected last: it runs after
every other GPU test and also alone."""
import ctypes as C

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle
import decode_tile_interleaved_rans_amd as ep
from decode_tile_interleaved_rans_amd import workloads as W

pytestmark = pytest.mark.gpu


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def call(fn, h, x, bias):
    M = x.shape[0]
    y = torch.full((M, h.shape[0]), float("nan"), dtype=torch.bfloat16, device="cuda")
    bp = C.c_void_p(bias.data_ptr()) if bias is not None else None
    rc = fn(h.ptr, C.c_void_p(x.data_ptr()), M, bp, C.c_void_p(y.data_ptr()),
            C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, ep.lib().ep_last_error()
    return y


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def pool_slices_use_gemm_library(M, N, K):
    """Slices (more than 64 rows) that the pool forward multiplies with hipBLASLt; the
    no-allocation forward always uses the library's own GEMM kernel."""
    return M > 64 and (M >= 512 or K <= 4096 or (M >= 256 and N <= 4096))


@pytest.mark.parametrize("layout", [0, ep.ROW_LAYOUT])
@pytest.mark.parametrize("N,K,Ms", [(2048, 3072, (96, 40)), (2048, 3072, (4, 1)), (2048, 3072, (300, 3)),
                                    (1024, 5120, (200, 100)), (1024, 5120, (300, 70))])
def test_noalloc_forward_matches_pool_forward(N, K, Ms, layout):
    w = W.student_t(N, K, seed=71)
    s, _ = ep.compress(w, 4.0, dtype=ep.BF16, layout=layout)
    h = ep.upload(s)
    want, _ = oracle.decompress(s, oracle.BF16)
    w_hat = W.bf16_bits_to_f32(want).astype(np.float64)
    bias_bits = W.activations(1, N, 9)[0]
    bias = bf16(bias_bits)
    L = ep.lib()
    for M in Ms:                                       # the second call is smaller than the first
        xb = W.activations(M, K, 100 + M)
        x = bf16(xb)
        y_pool = call(L.ep_linear_forward, h, x, bias)
        y_fixed = call(L.ep_linear_forward_noalloc, h, x, bias)
        torch.cuda.synchronize()
        h.check()
        a = y_fixed.float().cpu().numpy()
        b = y_pool.float().cpu().numpy()
        assert np.isfinite(a).all()
        if pool_slices_use_gemm_library(M, N, K):
            # the pool forward multiplies these slices with hipBLASLt (the no-allocation one with
            # the library's own kernel): the fp32 summation order differs
            assert rel_l2(a, b) < 3e-3, M
        elif M > 4 or layout != 0:
            assert torch.equal(y_fixed, y_pool), M        # same kernels, deterministic order
        else:
            assert rel_l2(a, b) < 1e-3, M                 # fp32 atomics: summation order varies
        ref = W.bf16_bits_to_f32(xb).astype(np.float64) @ w_hat.T + W.bf16_bits_to_f32(bias_bits)[None, :]
        assert rel_l2(a, ref) < 2e-2, M
    h.release()


def test_noalloc_forwards_captured_in_a_hip_graph():
    """What the no-allocation entry point is for: forwards captured into a HIP graph (after one
    warm-up call per path, which resolves the static scratch), here the row-layout fused kernel
    (40 rows), the layout-0 matrix-vector kernel (3 rows) and decode slices + GEMM (96 rows) in
    one graph on one stream. Three replays, with eager work on the stream between them, each give
    the eager calls' results (the same bits; the matrix-vector kernel's float atomics within 1e-3)."""
    L = ep.lib()
    cases = []
    for layout, M, seed in ((ep.ROW_LAYOUT, 40, 81), (0, 3, 82), (0, 96, 83)):
        w = W.student_t(1024, 2048, seed=seed)
        s, _ = ep.compress(w, 4.0, dtype=ep.BF16, layout=layout)
        h = ep.upload(s)
        x = bf16(W.activations(M, 2048, seed + 10))
        bias = bf16(W.activations(1, 1024, seed + 20)[0])
        y = torch.empty((M, 1024), dtype=torch.bfloat16, device="cuda")
        cases.append((h, x, bias, y))
    st = torch.cuda.Stream()

    def run_all():
        for h, x, bias, y in cases:
            rc = L.ep_linear_forward_noalloc(h.ptr, C.c_void_p(x.data_ptr()), x.shape[0], C.c_void_p(bias.data_ptr()),
                                             C.c_void_p(y.data_ptr()), C.c_void_p(st.cuda_stream))
            assert rc == 0, L.ep_last_error()

    with torch.cuda.stream(st):
        run_all()
    torch.cuda.synchronize()
    want = [y.clone() for *_, y in cases]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        run_all()
    for _ in range(3):
        for *_, y in cases:
            y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for (h, x, bias, y), w_ in zip(cases, want):
            if x.shape[0] <= 4:
                assert rel_l2(y.float().cpu().numpy(), w_.float().cpu().numpy()) < 1e-3
            else:
                assert torch.equal(y, w_), x.shape[0]
        with torch.cuda.stream(st):                  # eager work between replays
            torch.matmul(cases[2][1], cases[2][1].T)
        torch.cuda.synchronize()
    for h, *_ in cases:
        h.check()
        h.release()
