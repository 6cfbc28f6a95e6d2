"""GPU parity of the gfx950 decode kernels against the oracle (bit-exact: symbols, container
bytes and row scales), through the C ABI.

Inputs are the seeded synthetic workloads: a 1024x1024 fp32 Gaussian matrix with 0.1% outliers
at 4.0 bpp; 4096x4096 bf16 Student-t(5) rows with log-normal row scales at 3.0 / 4.0 / 4.5 bpp
plus the lossless bf16 round trip; ragged shapes, escapes, degenerate matrices; sampled tiles of
8192x8192 at 4.5 bpp; the DiT-like model (one block in a grouped launch, two matrices in full,
sampled tiles of the rest and of other blocks); the 64-matrix mixed-rate set in FP8, INT8 and
BF16."""
import numpy as np
import pytest
import torch

import oracle
import decode_tile_interleaved_rans_amd as ep
from decode_tile_interleaved_rans_amd import workloads as W

pytestmark = pytest.mark.gpu

CONTAINERS = {"bf16": (torch.bfloat16, oracle.BF16), "f16": (torch.float16, oracle.F16),
              "f8": (torch.float8_e4m3fn, oracle.F8E4M3), "i8": (torch.int8, oracle.I8)}


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.element_size() == 1:
        return t.view(torch.uint8).numpy()
    return t.view(torch.int32).numpy().view(np.uint32)


def gpu_decode(stream: bytes, dtype):
    h = ep.upload(stream)
    out = h.decompress(dtype)
    torch.cuda.synchronize()
    h.check()
    return out


def mismatch_report(name, got, want, q=None):
    bad = np.argwhere(got != want)
    msg = f"{name}: {len(bad)} of {got.size} elements differ"
    for r, c in bad[:6]:
        msg += f"\n  [{r},{c}] gpu={int(got[r, c]):#x} oracle={int(want[r, c]):#x}"
        if q is not None:
            msg += f" q={int(q[r, c])}"
    return msg


def assert_parity(stream: bytes, names=("bf16", "f16", "f8", "i8"), threads=16):
    h = ep.upload(stream)
    q = h.decode_symbols()
    qo, _ = oracle.decode_symbols(stream, n_threads=threads)
    torch.cuda.synchronize()
    h.check()
    assert np.array_equal(q.cpu().numpy(), qo), mismatch_report("symbols", q.cpu().numpy(), qo)
    errors = []
    for name in names:
        tdt, odt = CONTAINERS[name]
        res = h.decompress(tdt)
        torch.cuda.synchronize()
        h.check()
        want, wscale = oracle.decompress(stream, odt, n_threads=threads)
        if isinstance(res, tuple):
            out, scale = res
            if not np.array_equal(scale.cpu().numpy(), wscale):
                errors.append(mismatch_report(f"{name} row scales", scale.cpu().numpy()[:, None], wscale[:, None]))
        else:
            out = res
        got = bits(out)
        if not np.array_equal(got, want):
            errors.append(mismatch_report(f"{name} container", got, want, qo))
    h.release()
    assert not errors, "\n".join(errors)


def test_c1_gaussian_outliers_all_containers():
    w = W.gaussian_with_outliers()
    s, bpp = ep.compress(w, 4.0)
    assert bpp >= 4.0
    assert_parity(s)


@pytest.mark.parametrize("target", [3.0, 4.0, 4.5])
def test_c2_student_t_4096(target):
    w = W.student_t_rowscaled(4096, 4096, 2)
    s, _ = ep.compress(w, target, dtype=ep.BF16)
    assert_parity(s, names=("bf16", "f16"))


def test_c2_bench_step_as_one_grouped_launch():
    # the launch the benchmark times: the 4096^2 matrix at 3.0 / 4.0 / 4.5 bpp to BF16 and FP16
    # plus its lossless BF16 stream, seven matrices in one grouped decode, each output bit-exact
    w = W.student_t_rowscaled(4096, 4096, 2)
    items = []
    for t in (3.0, 4.0, 4.5):
        s, _ = ep.compress(w, t, dtype=ep.BF16)
        items += [(s, torch.bfloat16, oracle.BF16), (s, torch.float16, oracle.F16)]
    ll, _ = ep.lossless_compress(w, dtype=ep.BF16)
    items.append((ll, torch.bfloat16, None))
    hs = [ep.upload(s) for s, _, _ in items]
    outs = [torch.empty((4096, 4096), dtype=tdt, device="cuda") for _, tdt, _ in items]
    ep.decompress_many(hs, outs)
    torch.cuda.synchronize()
    for h, (s, _, odt), o in zip(hs, items, outs):
        h.check()
        want = w if odt is None else oracle.decompress(s, odt, n_threads=16)[0]
        assert np.array_equal(bits(o), want), mismatch_report("bench-step output", bits(o), want)


def test_c2_lossless_bf16_roundtrip():
    w = W.student_t_rowscaled(4096, 4096, 2)
    s, bpp = ep.lossless_compress(w, dtype=ep.BF16)
    out = gpu_decode(s, torch.bfloat16)
    assert np.array_equal(bits(out), w)
    assert bpp < 16.0


def test_c2_lossless_exponent_coded_roundtrip():
    """The guide's DFloat11 config for lossless BF16 ("Choose a compression contract"), read as
    exponent by tile rANS + uncoded sign/mantissa bytes: bit-exact on the 4096 x 4096 matrix."""
    w = W.student_t_rowscaled(4096, 4096, 2)
    s, bpp = ep.lossless_compress(w, exponent_coded=True, dtype=ep.BF16)
    out = gpu_decode(s, torch.bfloat16)
    assert np.array_equal(bits(out), w)
    want, _ = oracle.decompress(s, oracle.BF16, n_threads=16)
    assert np.array_equal(want, w)
    assert bpp < 12.0


@pytest.mark.parametrize("case", ["ragged_17x300", "one", "ragged_33x513_t32_n11", "ragged_5x7_n10",
                                  "all_bit_patterns", "zeros", "ragged_130x1000_n11"])
def test_lossless_exponent_coded_shapes(case):
    rng = np.random.default_rng(len(case))
    opts = {"prob_bits": 12, "tile_rows": 16}
    if case == "all_bit_patterns":
        x = np.arange(1 << 16, dtype=np.uint16).reshape(64, 1024)
    elif case == "zeros":
        x = np.zeros((40, 300), np.uint16)
    elif case == "one":
        x = np.array([[0xBF80]], np.uint16)
    else:
        R, Cc = (int(v) for v in case.split("_")[1].split("x"))
        x = W.to_bf16_bits(rng.standard_t(4, (R, Cc)) * 0.03)
        opts["tile_rows"] = 32 if "_t32" in case else 16
        opts["prob_bits"] = 11 if "_n11" in case else 10 if "_n10" in case else 12
    s, _ = ep.lossless_compress(x, exponent_coded=True, dtype=ep.BF16, **opts)
    out = gpu_decode(s, torch.bfloat16)
    assert np.array_equal(bits(out), x)


@pytest.mark.parametrize("shape,prob_bits,tile_rows", [((17, 300), 12, 16), ((1, 1), 12, 16), ((33, 513), 11, 32),
                                                       ((5, 7), 10, 16), ((16, 768), 12, 16), ((48, 2304), 10, 32),
                                                       ((130, 1000), 11, 16)])
def test_ragged_shapes_and_options(shape, prob_bits, tile_rows):
    rng = np.random.default_rng(sum(shape))
    w = (0.02 * rng.standard_t(5, shape)).astype(np.float32)
    s, _ = ep.compress(w, 4.0, prob_bits=prob_bits, tile_rows=tile_rows)
    assert_parity(s)


def test_escapes_and_small_rows():
    rng = np.random.default_rng(5)
    w = rng.normal(0, 0.01, (64, 512)).astype(np.float32)
    w[rng.random(w.shape) < 0.002] = 3.0
    w[10] *= 1e-30                       # tiny row scale: FP16 subnormal outputs
    w[11] = 0.0
    s, _ = ep.compress(w, 7.0)
    assert ep.stream_info(s)["n_escapes"] > 0
    assert_parity(s)


def test_escapes_in_some_tables_only():
    # outliers only at column position 3 of every 8-block: only the coordinate tables of position 3
    # (tables 7 and 8) can decode the escape symbol, so the kernel takes its escape test at that
    # step alone and skips it at the other seven; several tiles and a ragged tail
    rng = np.random.default_rng(9)
    w = rng.normal(0, 0.01, (80, 1000)).astype(np.float32)
    m = np.zeros(w.shape, bool)
    m[:, 3::8] = rng.random((80, 125)) < 0.01
    w[m] = 3.0 * np.sign(rng.normal(size=int(m.sum())))
    s, _ = ep.compress(w, 4.0)
    assert ep.stream_info(s)["n_escapes"] > 0
    _, _, f = oracle.tables(s)
    esc = [t for t in range(1, 17) if f[t, 255] > 0]
    assert esc and set(esc) <= {7, 8}, esc
    assert_parity(s)


def test_degenerate_matrices():
    for w in [np.zeros((40, 300), np.float32), np.full((16, 256), 0.5, np.float32)]:
        s, _ = ep.compress(w, 4.0)
        assert_parity(s)
    s, _ = ep.compress(np.zeros((0, 16), np.float32), 4.0)
    h = ep.upload(s)
    out = torch.empty((0, 16), dtype=torch.bfloat16, device="cuda")
    h.decompress_into(out)
    torch.cuda.synchronize()
    h.check()


@pytest.mark.parametrize("dt", ["f16", "f32", "u8", "f8e4m3", "i8", "zeros"])
def test_lossless_other_dtypes(dt):
    rng = np.random.default_rng(6)
    shape = (37, 600)
    if dt == "f8e4m3":          # every E4M3 bit pattern occurs, NaN codes included
        x, code, tdt = rng.integers(0, 256, shape).astype(np.uint8), ep.F8E4M3, torch.float8_e4m3fn
    elif dt == "i8":
        x, code, tdt = rng.integers(-128, 128, shape).astype(np.int8).view(np.uint8), ep.I8, torch.int8
    elif dt == "f16":
        x, code, tdt = rng.normal(0, 1, shape).astype(np.float16).view(np.uint16), ep.F16, torch.float16
    elif dt == "f32":
        x, code, tdt = rng.normal(0, 1, shape).astype(np.float32).view(np.uint32), ep.F32, torch.float32
    elif dt == "u8":
        x, code, tdt = rng.integers(0, 9, shape).astype(np.uint8), ep.U8, torch.uint8
    else:
        x, code, tdt = np.zeros(shape, np.uint16), ep.BF16, torch.bfloat16
    s, _ = ep.lossless_compress(x, dtype=code)
    out = gpu_decode(s, tdt)
    assert np.array_equal(bits(out), x)


def test_grouped_decode_matches_single():
    """One grouped call over lossy matrices in four containers, lossless BF16 / U8 / FP32
    matrices and an exponent-coded BF16 matrix: the kernel balances the kinds of tiles by cost
    within one launch."""
    rng = np.random.default_rng(7)
    streams, conts = [], []
    for i, (R, Cc, t) in enumerate([(256, 512, 3.0), (128, 1024, 6.0), (300, 700, 2.5), (64, 256, 4.5)]):
        w = (0.02 * rng.standard_t(5, (R, Cc))).astype(np.float32)
        streams.append(ep.compress(w, t)[0])
        conts.append([torch.bfloat16, torch.float8_e4m3fn, torch.int8, torch.float16][i])
    lossless = [W.student_t(200, 600, 71), rng.integers(0, 255, (40, 300)).astype(np.uint8),
                rng.normal(0, 1, (33, 257)).astype(np.float32), W.student_t(300, 1000, 72)]
    for x, code, tdt in zip(lossless, (ep.BF16, ep.U8, ep.F32, ep.BF16),
                            (torch.bfloat16, torch.uint8, torch.float32, torch.bfloat16)):
        streams.append(ep.lossless_compress(x, dtype=code, exponent_coded=len(streams) == 7)[0])
        conts.append(tdt)
    hs = [ep.upload(s) for s in streams]
    outs = [torch.empty(h.shape, dtype=c, device="cuda") for h, c in zip(hs, conts)]
    scales = [torch.empty(h.shape[0], dtype=torch.float32, device="cuda") if c in (torch.float8_e4m3fn, torch.int8)
              else None for h, c in zip(hs, conts)]
    ep.decompress_many(hs, outs, scales)
    torch.cuda.synchronize()
    for i, (h, s, o, sc, c) in enumerate(zip(hs, streams, outs, scales, conts)):
        h.check()
        if i >= 4:
            x = lossless[i - 4]
            assert np.array_equal(bits(o), x.view(np.uint32) if x.dtype == np.float32 else x)
            continue
        odt = {torch.bfloat16: oracle.BF16, torch.float16: oracle.F16, torch.float8_e4m3fn: oracle.F8E4M3,
               torch.int8: oracle.I8}[c]
        want, wsc = oracle.decompress(s, odt, n_threads=8)
        assert np.array_equal(bits(o), want)
        if sc is not None:
            assert np.array_equal(sc.cpu().numpy(), wsc)


def test_device_flag_on_inconsistent_stream():
    """A stream that passes host validation (CRCs recomputed) but whose lane state was altered:
    the kernel's bounded reads keep it in range and the final-state check raises the flag."""
    import zlib
    w = W.gaussian_with_outliers(64, 512, seed=8)
    s, _ = ep.compress(w, 4.0)
    off_pay = int.from_bytes(s[72:80], "little")
    bad = bytearray(s)
    bad[off_pay + 4 * 3 + 1] ^= 0x10                       # tile 0, lane 3 state
    bad[88:92] = zlib.crc32(bytes(bad[off_pay:])).to_bytes(4, "little")
    bad[112:116] = zlib.crc32(bytes(bad[:112] + bad[116:off_pay])).to_bytes(4, "little")   # the header changed
    h = ep.upload(bytes(bad))
    h.decompress(torch.bfloat16)
    with pytest.raises(ep.EPError) as e:
        h.check()
    assert e.value.status == -7
    h.check()                                              # the flag was cleared


@pytest.mark.parametrize("exponent_coded", [False, True])
def test_unsupported_container_is_an_error(exponent_coded):
    x = np.zeros((16, 256), np.uint16)
    s, _ = ep.lossless_compress(x, dtype=ep.BF16, exponent_coded=exponent_coded)
    h = ep.upload(s)
    with pytest.raises(ep.EPError) as e:
        h.decompress(torch.float16)
    assert e.value.status == -3


def sampled_tile_parity(stream: bytes, n_sample: int, seed: int, dtype=torch.bfloat16, odt=oracle.BF16):
    """Decode the full matrix on the GPU, then compare randomly chosen tiles with the oracle's
    decode of just those tiles."""
    info = ep.stream_info(stream)
    h = ep.upload(stream)
    out = h.decompress(dtype)
    torch.cuda.synchronize()
    h.check()
    rng = np.random.default_rng(seed)
    tiles = np.sort(rng.choice(info["n_tiles"], size=min(n_sample, info["n_tiles"]), replace=False))
    want = oracle.decompress_tiles(stream, tiles, odt)
    tr_rows, tiles_c = info["tile_rows"], -(-info["cols"] // 256)
    got = bits(out)
    for k, t in enumerate(tiles):
        r0, c0 = (t // tiles_c) * tr_rows, (t % tiles_c) * 256
        blk = got[r0:r0 + tr_rows, c0:c0 + 256]
        assert np.array_equal(blk, want[k][: blk.shape[0], : blk.shape[1]]), f"tile {t}"


def test_c4_8192_sampled_tiles():
    w = W.student_t(8192, 8192, 4, 0.02)
    s, bpp = ep.compress(w, 4.5, dtype=ep.BF16)
    sampled_tile_parity(s, 400, 1)


def test_c3_dit_block_grouped_full_and_sampled():
    """DiT-like model at 4.0 bpp: block 0's five matrices decoded to BF16 in one grouped launch;
    the attention output projection and the FFN down projection compared in full, 1% of the
    tiles of the other three; then 1% of the tiles of one matrix from each of five other
    blocks (all 150 matrices would take minutes of host-side generation)."""
    streams = [ep.compress(W.dit_matrix(0, m), 4.0, dtype=ep.BF16)[0] for m in range(5)]
    hs = [ep.upload(s) for s in streams]
    outs = [torch.empty(h.shape, dtype=torch.bfloat16, device="cuda") for h in hs]
    ep.decompress_many(hs, outs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(30)
    for m, (h, s, o) in enumerate(zip(hs, streams, outs)):
        h.check()
        got = bits(o)
        if m in (1, 4):
            want, _ = oracle.decompress(s, oracle.BF16, n_threads=16)
            assert np.array_equal(got, want), mismatch_report(f"block 0 matrix {m}", got, want)
        else:
            info = ep.stream_info(s)
            tiles = np.sort(rng.choice(info["n_tiles"], size=info["n_tiles"] // 100, replace=False))
            want = oracle.decompress_tiles(s, tiles, oracle.BF16)
            tiles_c = -(-info["cols"] // 256)
            for k, t in enumerate(tiles):
                r0, c0 = (t // tiles_c) * 16, (t % tiles_c) * 256
                assert np.array_equal(got[r0:r0 + 16, c0:c0 + 256], want[k]), f"block 0 matrix {m} tile {t}"
        h.release()
    for b in (6, 12, 18, 24, 29):
        s, _ = ep.compress(W.dit_matrix(b, b % 5), 4.0, dtype=ep.BF16)
        sampled_tile_parity(s, ep.stream_info(s)["n_tiles"] // 100, b)


def test_c5_mixed_rate_set_all_containers():
    """The 64-matrix mixed-rate set (rows, cols in {2048, 4096, 8192}, targets U[2.5, 6.0]), each
    decoded to FP8 E4M3 (+ row scale), INT8 (+ row scale) and BF16 by grouped launches over all
    64 matrices; every matrix is checked on 8 tiles (first, last and 6 random ones) against the
    oracle's decode of those tiles, container bytes and row scales."""
    items = W.mixed_rate_set()
    streams = []
    for R, Cc, t, wseed, _ in items:
        s, bpp = ep.compress(W.student_t(R, Cc, wseed, 0.02), t, dtype=ep.BF16)
        assert bpp > t                                  # metadata included: the target is a floor
        streams.append(s)
    hs = [ep.upload(s) for s in streams]
    rng = np.random.default_rng(64)
    for name in ("f8", "i8", "bf16"):
        tdt, odt = CONTAINERS[name]
        outs = [torch.empty(h.shape, dtype=tdt, device="cuda") for h in hs]
        scales = [torch.empty(h.shape[0], dtype=torch.float32, device="cuda") for h in hs] if name != "bf16" else None
        ep.decompress_many(hs, outs, scales)
        torch.cuda.synchronize()
        for i, (h, s) in enumerate(zip(hs, streams)):
            h.check()
            info = ep.stream_info(s)
            n = info["n_tiles"]
            tiles = np.unique(np.r_[0, n - 1, rng.choice(n, 6, replace=False)])
            got = bits(outs[i])
            tiles_c = -(-info["cols"] // 256)
            if scales is None:
                want = oracle.decompress_tiles(s, tiles, odt)
            else:
                want, wsc = oracle.decompress_tiles(s, tiles, odt, want_scale=True)
                gsc = scales[i].cpu().numpy()
            for k, t in enumerate(tiles):
                r0, c0 = (t // tiles_c) * 16, (t % tiles_c) * 256
                assert np.array_equal(got[r0:r0 + 16, c0:c0 + 256], want[k]), f"matrix {i} {name} tile {t}"
                if scales is not None:
                    assert np.array_equal(gsc[r0:r0 + 16], wsc[k]), f"matrix {i} {name} row scales, tile {t}"
        del outs, scales
    for h in hs:
        h.release()


def test_fp8_container_saturates_on_very_wide_rows():
    """A row's normalized values reach sqrt(C) (one non-zero entry in a unit-RMS row), so with
    C = 2^18 the FP8 values q * step / 2 pass 448 and must saturate to the largest E4M3 code."""
    R, Cc = 16, 1 << 18
    rng = np.random.default_rng(12)
    w = np.zeros((R, Cc), np.float32)
    w[:, 5] = rng.choice([-1.0, 1.0], R)
    w[:, 1000:1008] = rng.normal(0, 1e-3, (R, 8))
    s, _ = ep.compress(w, 4.0)
    want, wscale = oracle.decompress(s, oracle.F8E4M3, n_threads=16)
    assert np.all((want[:, 5] & 0x7F) == 0x7E), "the oracle saturates at 448"
    h = ep.upload(s)
    out, scale = h.decompress(torch.float8_e4m3fn)
    torch.cuda.synchronize()
    h.check()
    assert np.array_equal(bits(out), want)
    assert np.array_equal(scale.cpu().numpy(), wscale)
