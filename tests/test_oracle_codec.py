"""End-to-end pins of the oracle codec: containers against library casts, quantization against
brute-force nearest points, lossless bit equality, accounting, edge cases and stream validation.

Passages followed: containers BF16/FP16/FP8/INT8 with the bitrate independent of precision and
tiles that decode independently (EntroPack paper, Abstract); target versus actual bitrate, where
the actual figure includes metadata ("EntroPack PyTorch Guide", "Start with a tensor round
trip"); lossless recovery of every bit, zeros and repeated values included (same guide,
"Choose a compression contract" and "Start with a tensor round trip"); a clear error instead of
a silent cast (same guide, "Diagnose compression failures in the correct order")."""
import json
import os
import zlib

import numpy as np
import pytest
import torch

import oracle
from decode_tile_interleaved_rans_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- number formats vs torch casts
def special_f32(rng, n):
    v = np.concatenate([
        rng.normal(0, 1, n) * np.exp(rng.uniform(-30, 30, n)),
        rng.normal(0, 1, n // 4) * 2.0 ** -130,                    # fp32 subnormals
        (rng.integers(-2 ** 20, 2 ** 20, n // 4) + 0.5) * 2.0 ** -8,   # exact ties for bf16/fp16
        [0.0, -0.0, 65504.0, 65519.0, 65520.0, 3.4e38, -3.4e38, 1e-45],
    ]).astype(np.float32)
    return v


def test_bf16_and_fp16_casts_match_torch():
    rng = np.random.default_rng(1)
    v = special_f32(rng, 20000)
    t = torch.from_numpy(v)
    want_bf = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    want_h = t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    got_bf = np.array([oracle.f32_to_bf16(float(x)) for x in v], np.uint16)
    got_h = np.array([oracle.f32_to_f16(float(x)) for x in v], np.uint16)
    assert np.array_equal(got_bf, want_bf)
    assert np.array_equal(got_h, want_h)


def test_e4m3_cast_matches_torch_in_range_and_saturates():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000) * 2.0 ** rng.uniform(-14, 8, 20000),
                        np.arange(-64, 65) / 8.0 * 2.0 ** -6, [448.0, -448.0, 0.0]]).astype(np.float32)
    v = v[np.abs(v) <= 448]
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.f32_to_e4m3(float(x)) for x in v], np.uint8)
    assert np.array_equal(got, want)
    assert oracle.f32_to_e4m3(500.0) == 0x7E and oracle.f32_to_e4m3(-1e9) == 0xFE   # +-448


# ---------------------------------------------------------------- lossy end to end
@pytest.fixture(scope="module")
def c1_stream():
    w = W.gaussian_with_outliers()            # 1024 x 1024 fp32 with 0.1% outliers
    s, bpp = oracle.compress(w, 4.0)
    return w, s, bpp


def test_lossy_symbols_are_nearest_e8_points(c1_stream):
    w, s, _ = c1_stream
    d = oracle.info(s)
    q, b = oracle.decode_symbols(s)
    assert np.all((q & 1) == np.repeat(b, 8, axis=1)[:, : w.shape[1]])
    assert np.all(q.reshape(-1, 8).astype(np.int64).sum(1) % 4 == 0)
    scale = np.array([oracle.row_scale(w, r) for r in range(w.shape[0])], np.float32)
    y = w.astype(np.float64) / (scale.astype(np.float64)[:, None] * np.float64(np.float32(d["step"])))
    dist = ((y - q / 2.0) ** 2).reshape(-1, 8).sum(1)
    rng = np.random.default_rng(0)
    pick = rng.choice(len(dist), 3000, replace=False)
    from test_oracle_e8 import brute_min_dist
    assert np.all(dist[pick] <= brute_min_dist(y.reshape(-1, 8)[pick]) + 1e-9)


def test_lossy_containers_match_library_casts(c1_stream):
    """The containers follow from the decoded q, the header step and the row scales:
    BF16/FP16 = torch casts of fp32(q * fp32(h * s)); FP8 = torch e4m3 cast of fp32(q * h) with
    s as the row scale; INT8 = the integer closed form with k = max(1, ceil(qmax / 127))."""
    w, s, _ = c1_stream
    d = oracle.info(s)
    q, _ = oracle.decode_symbols(s)
    h = np.float32(d["step"]) / np.float32(2)
    scale = np.array([oracle.row_scale(w, r) for r in range(w.shape[0])], np.float32)
    alpha = (h * scale).astype(np.float32)
    v = q.astype(np.float32) * alpha[:, None]
    bf, _ = oracle.decompress(s, oracle.BF16)
    assert np.array_equal(bf, torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    hf, _ = oracle.decompress(s, oracle.F16)
    assert np.array_equal(hf, torch.from_numpy(v).to(torch.float16).view(torch.int16).numpy().view(np.uint16))
    f8, sc8 = oracle.decompress(s, oracle.F8E4M3)
    v8 = q.astype(np.float32) * h
    assert np.abs(v8).max() <= 448
    assert np.array_equal(f8, torch.from_numpy(v8).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert np.array_equal(sc8, scale)
    i8, sci = oracle.decompress(s, oracle.I8)
    qmax = np.abs(q.astype(np.int64)).max(1)
    k = np.maximum(1, -(-qmax // 127))
    a = np.abs(q.astype(np.int64))
    want = np.sign(q) * ((2 * a + k[:, None]) // (2 * k[:, None]))
    assert np.array_equal(i8.view(np.int8).astype(np.int64), want)
    assert np.abs(want).max() <= 127
    assert np.array_equal(sci, (alpha * k.astype(np.float32)).astype(np.float32))


def test_int8_exhaustive_closed_form():
    """INT8 rounding over every |q| <= qmax for several qmax, through a stream whose rows hold
    exactly those values: round-half-away(q / k) with k = max(1, ceil(qmax / 127))."""
    for qmax in (1, 127, 128, 255, 300, 1000):
        k = max(1, -(-qmax // 127))
        qs = np.arange(-qmax, qmax + 1)
        want = np.sign(qs) * ((2 * np.abs(qs) + k) // (2 * k))
        assert np.abs(want).max() <= 127
        # |q| <= 127 is exact, and the error is at most k / 2 in q units
        assert np.all(np.abs(want * k - qs) <= k / 2 + 1e-9)
        if qmax <= 127:
            assert np.array_equal(want, qs)


def test_accounting_identity(c1_stream):
    w, s, bpp = c1_stream
    d = oracle.info(s)
    assert bpp == 8 * len(s) / w.size
    assert d["payload_bytes"] + d["meta_bytes"] == len(s) == d["total_bytes"]
    assert bpp >= 4.0, "actual includes states and metadata on top of the payload target"
    word_bpp = 8 * (d["payload_bytes"] - d["state_bytes"]) / w.size
    assert abs(word_bpp - 4.0) <= 0.05


def test_paper_bitrate_example():
    """1e6 parameters at 4.5 bits each: about 4.5e6 data bits, plus the information needed to
    restore, so the stored size is above the plain product."""
    g = json.load(open(os.path.join(GOLDEN, "paper_bitrate_example.json")))
    rng = np.random.default_rng(31)
    w = (0.02 * rng.standard_t(5, (1000, 1000))).astype(np.float32)
    assert w.size == g["params"]
    s, bpp = oracle.compress(w, g["bits_per_param"])
    d = oracle.info(s)
    data_bits = 8 * (d["payload_bytes"] - d["state_bytes"])
    assert data_bits == pytest.approx(g["data_bits"], rel=0.02)
    assert 8 * len(s) > g["data_bits"] and bpp > g["bits_per_param"]


@pytest.mark.slow
@pytest.mark.parametrize("target", [3.0, 4.0, 4.5])
def test_word_payload_meets_target_4096(target):
    w = W.student_t_rowscaled(4096, 4096, 2)
    s, bpp = oracle.compress(w, target, dtype=oracle.BF16)
    d = oracle.info(s)
    word_bpp = 8 * (d["payload_bytes"] - d["state_bytes"]) / w.size
    assert abs(word_bpp - target) <= 0.05
    assert bpp >= target


def test_escapes_are_coded_and_recovered():
    """Values beyond a 255-wide window use the escape symbol + raw word: a narrow Gaussian bulk
    with far outliers at a high rate."""
    rng = np.random.default_rng(5)
    w = rng.normal(0, 0.01, (64, 512)).astype(np.float32)
    w[rng.random(w.shape) < 0.002] = 3.0
    s, _ = oracle.compress(w, 7.0)
    d = oracle.info(s)
    lo, S, _ = oracle.tables(s)
    assert d["n_escapes"] > 0 and S.max() == 255
    q, b = oracle.decode_symbols(s)
    scale = np.array([oracle.row_scale(w, r) for r in range(w.shape[0])], np.float32)
    y = w.astype(np.float64) / (scale.astype(np.float64)[:, None] * np.float64(np.float32(d["step"])))
    from test_oracle_e8 import brute_min_dist
    dist = ((y - q / 2.0) ** 2).reshape(-1, 8).sum(1)
    big = np.abs(q).reshape(-1, 8).max(1) > 2 * 300
    assert big.sum() > 0
    assert np.all(dist[big] <= brute_min_dist(y.reshape(-1, 8)[big]) + 1e-9)


@pytest.mark.parametrize("shape", [(17, 300), (1, 1), (16, 256), (33, 513), (5, 7)])
def test_ragged_shapes_roundtrip(shape):
    rng = np.random.default_rng(sum(shape))
    w = rng.normal(0, 0.05, shape).astype(np.float32)
    s, bpp = oracle.compress(w, 4.0)
    d = oracle.info(s)
    assert d["n_tiles"] == -(-shape[0] // 16) * -(-shape[1] // 256)
    q, _ = oracle.decode_symbols(s)
    assert q.shape == shape
    bf, _ = oracle.decompress(s, oracle.BF16)
    assert bf.shape == shape
    tiles = oracle.decompress_tiles(s, np.arange(d["n_tiles"]), oracle.BF16)
    tc = -(-shape[1] // 256)
    full = tiles.reshape(-1, tc, 16, 256).transpose(0, 2, 1, 3).reshape(-(-shape[0] // 16) * 16, tc * 256)
    assert np.array_equal(full[: shape[0], : shape[1]], bf)


@pytest.mark.parametrize("container", [oracle.F8E4M3, oracle.I8])
def test_tile_decode_row_scales_match_full_decode(container):
    """The per-tile decode's row scales (used to check sampled tiles of large matrices) are the
    full decode's, row for row; padding rows of the last tile row give 0."""
    w = W.gaussian_with_outliers(40, 600, seed=12)
    s, _ = oracle.compress(w, 5.0)
    d = oracle.info(s)
    full, scale = oracle.decompress(s, container)
    tiles = np.arange(d["n_tiles"])
    out, sc = oracle.decompress_tiles(s, tiles, container, want_scale=True)
    tc = -(-600 // 256)
    for t in tiles:
        r0 = (t // tc) * 16
        rows = np.arange(r0, r0 + 16)
        want = np.where(rows < 40, scale[np.minimum(rows, 39)], 0.0).astype(np.float32)
        assert np.array_equal(sc[t], want)


def test_zero_rows_decode_to_positive_zero():
    rng = np.random.default_rng(6)
    w = rng.normal(0, 0.02, (32, 256)).astype(np.float32)
    w[3] = 0.0
    w[7] = -0.0
    s, _ = oracle.compress(w, 4.0)
    for ct in (oracle.BF16, oracle.F16, oracle.F8E4M3, oracle.I8):
        out, sc = oracle.decompress(s, ct)
        assert np.all(out[3] == 0) and np.all(out[7] == 0)
        if sc is not None:
            assert sc[3] == 0.0 and sc[7] == 0.0


def test_all_zero_matrix():
    w = np.zeros((64, 512), np.float32)
    s, bpp = oracle.compress(w, 4.0)
    d = oracle.info(s)
    assert d["payload_bytes"] == 128 * d["n_tiles"], "single-symbol tables: states only"
    bf, _ = oracle.decompress(s, oracle.BF16)
    assert np.all(bf == 0)


def test_empty_matrix():
    for shape in [(0, 16), (8, 0)]:
        s, bpp = oracle.compress(np.zeros(shape, np.float32), 4.0)
        d = oracle.info(s)
        assert d["n_tiles"] == 0 and bpp == 0.0
        out, _ = oracle.decompress(s, oracle.BF16)
        assert out.shape == shape


# ---------------------------------------------------------------- lossless mode
def lossless_cases():
    rng = np.random.default_rng(7)
    rnd = W.to_bf16_bits(rng.normal(0, 0.02, (40, 300)))
    specials = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0x7F81, 0xFFFF, 0x0001, 0x807F, 0x3F80],
                        np.uint16)
    return {
        "random_bf16": (rnd, oracle.BF16),
        "zeros": (np.zeros((32, 512), np.uint16), oracle.BF16),
        "constant": (np.full((20, 260), 0x3C00, np.uint16), oracle.BF16),
        "alternating": (np.tile(np.array([0x3F80, 0xBF80], np.uint16), (16, 128)), oracle.BF16),
        "specials": (np.resize(specials, (24, 270)), oracle.BF16),
        "fp16": (rng.integers(0, 1 << 16, (17, 257)).astype(np.uint16), oracle.F16),
        "fp32": (rng.normal(0, 1, (16, 300)).astype(np.float32).view(np.uint32), oracle.F32),
        "u8": (rng.integers(0, 256, (18, 256)).astype(np.uint8), oracle.U8),
    }


@pytest.mark.parametrize("name", list(lossless_cases()))
def test_lossless_bit_exact(name):
    x, dt = lossless_cases()[name]
    s, bpp = oracle.compress(x, dtype=dt, mode=oracle.LOSSLESS)
    out, _ = oracle.decompress(s, dt)
    assert out.dtype == x.dtype and np.array_equal(out, x)
    if name == "zeros":
        d = oracle.info(s)
        assert d["payload_bytes"] == 128 * d["n_tiles"]


def test_lossless_4096_student_t_bf16():
    w = W.student_t_rowscaled(1024, 1024, 2)
    s, bpp = oracle.compress(w, dtype=oracle.BF16, mode=oracle.LOSSLESS)
    out, _ = oracle.decompress(s, oracle.BF16, n_threads=4)
    assert np.array_equal(out, w)
    assert bpp < 16


# ---------------------------------------------------------------- validation
def test_corrupt_and_unsupported_streams(c1_stream):
    _, s, _ = c1_stream
    with pytest.raises(oracle.OracleError) as e:
        oracle.decompress(b"XXXX" + s[4:])
    assert e.value.rc == -2
    with pytest.raises(oracle.OracleError):
        oracle.decompress(s[:-8])
    bad = bytearray(s)
    bad[-100] ^= 1                                    # payload byte: CRC catches it
    with pytest.raises(oracle.OracleError):
        oracle.decompress(bytes(bad))
    assert zlib.crc32(s[oracle.info(s)["meta_bytes"]:]) == int.from_bytes(s[88:92], "little")
    x = np.zeros((16, 256), np.uint16)
    sl, _ = oracle.compress(x, dtype=oracle.BF16, mode=oracle.LOSSLESS)
    with pytest.raises(oracle.OracleError) as e:
        oracle.decompress(sl, oracle.F16)             # no silent cast of a lossless stream
    assert e.value.rc == -3


# ---------------------------------------------------------------- exponent-coded lossless BF16
# Reading of the DFloat11 config the guide names for lossless BF16 ("Choose a compression
# contract"): the 8-bit exponent is entropy coded with the tile rANS, sign and mantissa are kept
# uncoded as one byte per element in a raw plane (offset in header bytes 96..103, its CRC-32 in
# 104..107).
def header_field(s: bytes, off: int, size: int) -> int:
    return int.from_bytes(s[off:off + size], "little")


def test_metadata_crc_covers_every_byte_but_payload_and_raw_plane(c1_stream):
    # format version 2 (reading R22): header bytes 112..115 hold the CRC-32 of the stream with the
    # payload, the raw plane and these four bytes left out; zlib's CRC-32 is the reference
    _, s, _ = c1_stream
    assert header_field(s, 4, 2) == 2
    o_pl = header_field(s, 72, 8)
    assert zlib.crc32(s[:112] + s[116:o_pl]) == header_field(s, 112, 4)
    x = W.student_t_rowscaled(32, 512, seed=1)
    se, _ = oracle.compress(x, dtype=oracle.BF16, mode=oracle.LOSSLESS_EXP)
    o_raw, o_pl = header_field(se, 96, 8), header_field(se, 72, 8)
    raw_len = 32 * 512                                # Rp x Cp of the padded matrix
    assert zlib.crc32(se[:112] + se[116:o_raw] + se[o_raw + raw_len:o_pl]) == header_field(se, 112, 4)
    old = bytearray(s)
    old[4] = 1                                        # a version-1 header is refused
    with pytest.raises(oracle.OracleError) as e:
        oracle.info(bytes(old))
    assert e.value.rc == -2


def test_every_single_bit_flip_is_rejected():
    # three CRC-32s (payload, raw plane, metadata) leave no bit of a stream unchecked
    rng = np.random.default_rng(3)
    w = rng.normal(0, 0.02, (16, 256)).astype(np.float32)
    w[2, 9] = 1.0                                     # an escape
    streams = [oracle.compress(w, 2.0)[0],
               oracle.compress(W.student_t_rowscaled(16, 256, seed=4), dtype=oracle.BF16, mode=oracle.LOSSLESS_EXP)[0],
               oracle.compress(rng.integers(0, 40, (16, 256)).astype(np.uint8), dtype=oracle.U8, mode=oracle.LOSSLESS)[0]]
    for st in streams:
        oracle.info(st)
        accepted = []
        for i in range(len(st)):
            for b in range(8):
                bad = bytearray(st)
                bad[i] ^= 1 << b
                try:
                    oracle.info(bytes(bad))
                    accepted.append((i, b))
                except oracle.OracleError:
                    pass
        assert not accepted, accepted[:10]


def exp_cases():
    cases = {k: v for k, v in lossless_cases().items() if v[1] == oracle.BF16}
    rng = np.random.default_rng(11)
    cases["ragged_5x9"] = (W.to_bf16_bits(rng.normal(0, 3, (5, 9))), oracle.BF16)
    cases["all_bits"] = (np.arange(1 << 16, dtype=np.uint16).reshape(64, 1024), oracle.BF16)
    return cases


@pytest.mark.parametrize("name", list(exp_cases()))
def test_lossless_exp_bit_exact(name):
    x, dt = exp_cases()[name]
    s, bpp = oracle.compress(x, dtype=dt, mode=oracle.LOSSLESS_EXP)
    out, _ = oracle.decompress(s, dt)
    assert out.dtype == x.dtype and np.array_equal(out, x)
    tiles = np.arange(oracle.info(s)["n_tiles"])
    t_out = oracle.decompress_tiles(s, tiles, dt)
    R, Cc = x.shape
    padded = np.zeros((len(tiles) and t_out.shape[1] * ((R + t_out.shape[1] - 1) // t_out.shape[1]),
                       (Cc + 255) // 256 * 256), np.uint16)
    tc = padded.shape[1] // 256
    for i in tiles:
        padded[i // tc * t_out.shape[1]:(i // tc + 1) * t_out.shape[1], i % tc * 256:(i % tc + 1) * 256] = t_out[i]
    assert np.array_equal(padded[:R, :Cc], x)
    assert not padded[R:].any() and not padded[:, Cc:].any(), "padding decodes to +0.0"


def test_lossless_exp_sections_closed_form():
    """The raw plane holds (sign << 7) | mantissa of the zero-padded matrix, byte for byte; the
    single table has f > 0 exactly for the exponents present (padding counts as exponent 0)."""
    rng = np.random.default_rng(5)
    x = W.to_bf16_bits(rng.standard_t(3, (40, 300)) * 0.05)
    x[3, :7] = [0x7F80, 0xFF80, 0x7FC1, 0x0001, 0x8000, 0x807F, 0x3F80]
    s, _ = oracle.compress(x, dtype=oracle.BF16, mode=oracle.LOSSLESS_EXP, tile_rows=16)
    Rp, Cp = 48, 512
    pad = np.zeros((Rp, Cp), np.uint16)
    pad[:40, :300] = x
    o_raw = header_field(s, 96, 8)
    assert s[6] == 2 and s[23] == 1 and o_raw % 16 == 0
    raw = np.frombuffer(s[o_raw:o_raw + Rp * Cp], np.uint8).reshape(Rp, Cp)
    want = (((pad >> 8) & 0x80) | (pad & 0x7F)).astype(np.uint8)
    assert np.array_equal(raw, want)
    assert zlib.crc32(raw.tobytes()) == header_field(s, 104, 4)
    o_pl = header_field(s, 72, 8)
    assert o_pl >= o_raw + Rp * Cp and zlib.crc32(s[o_pl:]) == header_field(s, 88, 4)
    lo, S, f = oracle.tables(s)
    assert len(S) == 1 and S[0] == 256 and lo[0] == 0 and f[0].sum() == 1 << 12
    present = np.bincount(((pad >> 7) & 0xFF).ravel(), minlength=256) > 0
    assert np.array_equal(f[0] > 0, present)
    d = oracle.info(s)
    assert d["payload_bytes"] == len(s) - o_pl + Rp * Cp


def test_lossless_exp_rate_close_to_exponent_entropy():
    """Coded size: at least N (H(exponent) + 8) bits (the order-0 entropy bound), at most that
    plus the 32 states per tile and 2%, and no larger than the two-plane lossless stream of the
    same tensor by more than 1%."""
    w = W.student_t_rowscaled(1024, 1024, 2)
    s, bpp = oracle.compress(w, dtype=oracle.BF16, mode=oracle.LOSSLESS_EXP)
    s2, bpp2 = oracle.compress(w, dtype=oracle.BF16, mode=oracle.LOSSLESS)
    e = ((w >> 7) & 0xFF).astype(np.int64)
    p = np.bincount(e.ravel(), minlength=256) / e.size
    h = -(p[p > 0] * np.log2(p[p > 0])).sum()
    assert h + 8 <= bpp <= (h + 8 + 32 * 32 / 4096) * 1.02, (bpp, h)
    assert bpp <= bpp2 * 1.01, (bpp, bpp2)
    out, _ = oracle.decompress(s, oracle.BF16, n_threads=4)
    assert np.array_equal(out, w)


def test_lossless_exp_validation():
    x = W.to_bf16_bits(np.random.default_rng(1).normal(0, 1, (16, 256)))
    with pytest.raises(oracle.OracleError) as e:
        oracle.compress(x, dtype=oracle.F16, mode=oracle.LOSSLESS_EXP)      # BF16 only
    assert e.value.rc == -3
    s, _ = oracle.compress(x, dtype=oracle.BF16, mode=oracle.LOSSLESS_EXP)
    with pytest.raises(oracle.OracleError) as e:
        oracle.decompress(s, oracle.F16)                                     # no silent cast
    assert e.value.rc == -3
    bad = bytearray(s)
    bad[header_field(s, 96, 8) + 5] ^= 0x40                                 # raw byte: its CRC catches it
    with pytest.raises(oracle.OracleError) as e:
        oracle.decompress(bytes(bad))
    assert e.value.rc == -2
    s1, _ = oracle.compress(x, dtype=oracle.BF16, mode=oracle.LOSSLESS)
    bad = bytearray(s1)
    bad[96] = 16                                                             # raw offset in a two-plane stream
    with pytest.raises(oracle.OracleError) as e:
        oracle.decompress(bytes(bad))
    assert e.value.rc == -2
