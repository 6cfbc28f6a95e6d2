"""Parity on the inputs the benchmark times, built exactly as it builds them.

- The device encoder against the oracle encoder, byte for byte, on the 4096 x 4096 row-scaled
  Student-t matrix at 3.0 and 4.5 bpp and on a full-size matrix of the DiT-like model drawn on the
  GPU (the oracle encodes the same BF16 values copied to the host).
- All 150 matrices of the DiT-like model (drawn on the GPU with seeds 3000 + 5 b + m and coded by
  the device encoder) in the benchmark's five grouped launches of 30 to BF16, then sampled tiles
  of every matrix against the oracle's decode of the same streams.
- All 64 matrices of the mixed-rate set drawn and coded as the benchmark does, decoded to FP8
  E4M3, INT8 and BF16 by one grouped call each (launches of 32, as timed), sampled tiles and row
  scales of every matrix against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import decode_tile_interleaved_rans_amd as ep
from decode_tile_interleaved_rans_amd import workloads as W

pytestmark = pytest.mark.gpu


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def tiles_of(out: torch.Tensor, tiles, tile_rows: int = 16) -> np.ndarray:
    """[n, tile_rows, 256] container bits of the listed tiles of a decoded matrix, gathered on the
    GPU so that whole matrices never cross to the host."""
    R, C = out.shape
    tc = C // 256
    o = torch.stack([out[(t // tc) * tile_rows:(t // tc + 1) * tile_rows, (t % tc) * 256:(t % tc + 1) * 256]
                     for t in tiles.tolist()]).cpu()
    return o.view(torch.int16).numpy().view(np.uint16) if o.element_size() == 2 else o.view(torch.uint8).numpy()


def sample_tiles(rng, n_tiles: int, k: int) -> np.ndarray:
    return np.unique(np.r_[0, n_tiles - 1, rng.choice(n_tiles, k, replace=False)]).astype(np.uint32)


@pytest.mark.parametrize("target", [3.0, 4.5])
def test_device_encoder_equals_oracle_on_4096sq(target):
    w = W.student_t_rowscaled(4096, 4096, 2)
    t = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    sd, _ = ep.compress_device(t, target)
    so, _ = oracle.compress(w, target, dtype=oracle.BF16)
    assert sd == so


def test_dit_model_launches_as_benched():
    """Every matrix of the benchmark's step: blocks 0-29 in five grouped launches of 30."""
    rng = np.random.default_rng(30)
    for g in range(W.DIT_BLOCKS // 6):
        streams, hs, outs = [], [], []
        for b in range(6 * g, 6 * g + 6):
            for m, (R, Cc) in enumerate(W.DIT_BLOCK_SHAPES):
                w = W.gpu_student_t(R, Cc, 3000 + 5 * b + m, 0.02)
                st, _ = ep.compress_device(w, 4.0)
                if b == 0 and m == 0:        # one full-size matrix: the oracle encoder gives the same bytes
                    assert st == oracle.compress(host_bits(w), 4.0, dtype=oracle.BF16)[0]
                del w
                streams.append(st)
                hs.append(ep.upload(st))
                outs.append(torch.empty((R, Cc), dtype=torch.bfloat16, device="cuda"))
        ep.decompress_many(hs, outs)           # the benchmark's launch: 30 matrices, one kernel
        torch.cuda.synchronize()
        for i, (st, h, out) in enumerate(zip(streams, hs, outs)):
            h.check()
            tiles = sample_tiles(rng, h.info["n_tiles"], 8)
            want = oracle.decompress_tiles(st, tiles, oracle.BF16)
            assert np.array_equal(tiles_of(out, tiles), want), f"launch {g}, matrix {i}"
            h.release()
        del outs


@pytest.mark.parametrize("container", ["fp8", "int8", "bf16"])
def test_mixed_set_as_benched(container):
    """Every matrix of the mixed-rate set, decoded by one grouped call (two launches of 32)."""
    specs = W.mixed_rate_set()
    dt = {"fp8": torch.float8_e4m3fn, "int8": torch.int8, "bf16": torch.bfloat16}[container]
    oc = {"fp8": oracle.F8E4M3, "int8": oracle.I8, "bf16": oracle.BF16}[container]
    streams, hs, outs, scs = [], [], [], []
    for R, Cc, tgt, seed, _ in specs:
        w = W.gpu_student_t(R, Cc, seed, 0.02)
        st, _ = ep.compress_device(w, tgt)
        del w
        streams.append(st)
        hs.append(ep.upload(st))
        outs.append(torch.empty((R, Cc), dtype=dt, device="cuda"))
        scs.append(torch.empty(R, dtype=torch.float32, device="cuda") if container != "bf16" else None)
    ep.decompress_many(hs, outs, scs if container != "bf16" else None)
    torch.cuda.synchronize()
    rng = np.random.default_rng(64)
    for k, (st, h, out, sc) in enumerate(zip(streams, hs, outs, scs)):
        h.check()
        tiles = sample_tiles(rng, h.info["n_tiles"], 6)
        if sc is None:
            want = oracle.decompress_tiles(st, tiles, oc)
        else:
            want, want_sc = oracle.decompress_tiles(st, tiles, oc, want_scale=True)
            tc = out.shape[1] // 256
            rows = np.concatenate([np.arange((t // tc) * 16, (t // tc + 1) * 16) for t in tiles])
            got_sc = sc.cpu().numpy()[rows].reshape(len(tiles), 16)
            assert np.array_equal(got_sc.view(np.uint32), want_sc.view(np.uint32)), f"matrix {k} scales"
        assert np.array_equal(tiles_of(out, tiles), want), f"matrix {k}"
        h.release()
