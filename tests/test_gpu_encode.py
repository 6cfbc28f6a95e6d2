"""The device encoder (ep_compress_device: row scales, sampled rate search, E8 quantization, the
coordinate model and the tile rANS coding as gfx950 kernels; the method's fast encoding, EntroPack
paper, Abstract) against the host encoder, whose streams equal the oracle's (tests/test_host.py):
the streams must be byte-identical. Cases: the seeded workloads, ragged shapes with every tile
option, FP16 and BF16 inputs, escapes, zero rows, degenerate and empty matrices."""
import numpy as np
import pytest
import torch

import oracle
import decode_tile_interleaved_rans_amd as ep
from decode_tile_interleaved_rans_amd import workloads as W

pytestmark = pytest.mark.gpu


def device_tensor(w: np.ndarray, dt: int):
    if dt == ep.F32:
        return torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).cuda()
    return t.view(torch.bfloat16 if dt == ep.BF16 else torch.float16)


def same_stream(w, dt, target, **kw):
    sh, bh = ep.compress(w, target, dtype=dt, **kw)
    sd, bd = ep.compress_device(device_tensor(w, dt), target, **kw)
    if sd != sh:
        dh, dd = ep.stream_info(sh), ep.stream_info(sd)
        raise AssertionError(f"device stream differs: host {dh}, device {dd}, first differing byte "
                             f"{next(i for i in range(min(len(sh), len(sd))) if sh[i] != sd[i]) if len(sh) == len(sd) else 'length'}")
    assert bd == bh
    return sh


def test_c1_gaussian_outliers():
    s = same_stream(W.gaussian_with_outliers(), ep.F32, 4.0)
    assert s == oracle.compress(W.gaussian_with_outliers(), 4.0)[0]


@pytest.mark.parametrize("target", [3.0, 4.5])
def test_c2_student_t_bf16(target):
    same_stream(W.student_t_rowscaled(4096, 4096, 2), ep.BF16, target)


@pytest.mark.parametrize("shape,prob_bits,tile_rows", [((17, 300), 12, 16), ((1, 1), 12, 16), ((33, 513), 11, 32),
                                                       ((5, 7), 10, 16), ((130, 1000), 11, 16), ((48, 2304), 10, 32)])
def test_ragged_shapes_and_options(shape, prob_bits, tile_rows):
    rng = np.random.default_rng(sum(shape))
    w = (0.02 * rng.standard_t(5, shape)).astype(np.float32)
    same_stream(w, ep.F32, 4.0, prob_bits=prob_bits, tile_rows=tile_rows)


def test_fp16_input_escapes_and_zero_rows():
    rng = np.random.default_rng(5)
    w = rng.normal(0, 0.01, (64, 512)).astype(np.float32)
    w[rng.random(w.shape) < 0.002] = 3.0
    w[11] = 0.0
    s = same_stream(w.astype(np.float16).view(np.uint16), ep.F16, 7.0)
    assert ep.stream_info(s)["n_escapes"] > 0


@pytest.mark.parametrize("target", [2.5, 6.0])
def test_low_and_high_rates(target):
    same_stream(W.bf16_bits_to_f32(W.student_t(256, 1024, 8)).copy(), ep.F32, target)


def test_degenerate_and_empty():
    same_stream(np.zeros((40, 300), np.float32), ep.F32, 4.0)
    same_stream(np.full((16, 256), 0.5, np.float32), ep.F32, 4.0)
    same_stream(np.zeros((0, 16), np.float32), ep.F32, 4.0)


def test_non_finite_input_is_an_error():
    w = np.ones((16, 256), np.float32)
    w[3, 7] = np.inf
    with pytest.raises(ep.EPError) as e:
        ep.compress_device(device_tensor(w, ep.F32), 4.0)
    assert e.value.status == -4


def test_prefill_weight_8192():
    w, _ = W.prefill_case()
    s = same_stream(w, ep.BF16, 4.5)
    h = ep.upload(s)
    out = h.decompress(torch.bfloat16)
    torch.cuda.synchronize()
    h.check()
