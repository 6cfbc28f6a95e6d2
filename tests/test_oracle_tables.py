"""Pins of two format readings of the oracle that its round trips cannot catch, because encoder and
decoder would share any mistake in them.

1. The window rule of the symbol model (the conditional model of the lattice coordinates, EntroPack
   paper, Abstract; reading R8): a table covers the whole observed range of its values when that
   range has at most 255 values, else the 255-wide window holding the most occurrences, the smallest
   start winning ties; other values are escaped. Pinned by a brute-force search over every window
   start, on constructed histograms (ties, a best window ending exactly at the largest value or
   starting at the smallest) and random heavy-tailed ones, and end to end on real streams, whose
   tables must equal the rule applied to histograms counted here from the decoded coordinates.

2. The lossy tile layout (tiles that decode on their own, same passage; readings R7, R10, R12, R13):
   an independent Python reader, written from the byte layout alone, decodes every tile of oracle
   streams (escapes included) and must give the oracle decoder's doubled coordinates and cosets:
   step 9s codes the coset bit of each lane's block with table 0, steps 9s + 1 + j code coordinate
   j with table 1 + 2j + b chosen by the coset just decoded, refill words then escape words in
   ascending lane order; in layout 0 lane l codes the 8-column block l of tile row s, in layout 1
   (reading R27) the block of tile row l mod tile_rows at block column (32 / tile_rows) s +
   l // tile_rows. Both layouts deal the same symbols to the states, so their streams must decode
   to the same weights."""
import struct

import numpy as np
import pytest

import oracle
from decode_tile_interleaved_rans_amd import workloads as W

L = 1 << 16
LANES = 32


def window_brute(values):
    """(start, width, escaped) by trying every window start."""
    v = np.asarray(values, np.int64)
    vmin, vmax = int(v.min()), int(v.max())
    if vmax - vmin + 1 <= 255:
        return vmin, vmax - vmin + 1, 0
    hist = np.bincount(v - vmin)
    best_lo, best = None, -1
    for lo in range(vmin, vmax - 254 + 1):
        mass = int(hist[lo - vmin:lo - vmin + 255].sum())
        if mass > best:                      # strictly greater: the first (smallest) start keeps ties
            best, best_lo = mass, lo
    return best_lo, 255, len(v) - best


CONSTRUCTED = {
    "range_255": list(range(0, 255)),
    "range_1": [7] * 5,
    "two_equal_windows": [0] * 10 + [600] * 10,
    "best_window_ends_at_max": list(range(0, 1000)) + list(range(745, 1000)) * 3,
    "best_window_starts_at_min": list(range(-500, 500)) + list(range(-500, -245)) * 3,
    "densest_strictly_inside": [-1000, 1000] + list(range(40, 295)) * 2 + list(range(0, 40)),
    "tie_across_shift": list(range(-3, 254)) + [100] * 4,
    "off_by_one_window": [0] * 3 + [255] * 3 + [254] * 2,
}


@pytest.mark.parametrize("name", sorted(CONSTRUCTED))
def test_window_rule_constructed(name):
    vals = CONSTRUCTED[name]
    assert oracle.choose_window(vals) == window_brute(vals)


def test_window_rule_constructed_values():
    """The same cases with the answers written out by hand."""
    assert oracle.choose_window(CONSTRUCTED["range_255"]) == (0, 255, 0)
    assert oracle.choose_window(CONSTRUCTED["range_1"]) == (7, 1, 0)
    assert oracle.choose_window(CONSTRUCTED["two_equal_windows"]) == (0, 255, 10)      # not 346
    assert oracle.choose_window(CONSTRUCTED["best_window_ends_at_max"]) == (745, 255, 745)
    assert oracle.choose_window(CONSTRUCTED["best_window_starts_at_min"]) == (-500, 255, 745)
    assert oracle.choose_window(CONSTRUCTED["tie_across_shift"]) == (-3, 255, 2)
    # values {0, 254, 255}: [0, 254] holds 5, [1, 255] holds 5 -> the smaller start
    assert oracle.choose_window(CONSTRUCTED["off_by_one_window"]) == (0, 255, 3)


def test_window_rule_random_heavy_tails():
    rng = np.random.default_rng(11)
    for k in range(60):
        n = int(rng.integers(1, 3000))
        scale = float(rng.choice([3.0, 30.0, 120.0, 400.0]))
        vals = np.round(rng.standard_t(2 + k % 4, n) * scale).astype(np.int64)
        vals = np.clip(vals, -16384, 16383)
        assert oracle.choose_window(vals) == window_brute(vals), k


def table_histograms(q, b):
    """Per table the list of coded values, counted from doubled coordinates q [R, C] and cosets
    b [R, C/8] (the tables are built from every coded block)."""
    R, C = q.shape
    blocks = q.reshape(R, C // 8, 8).astype(np.int64)
    cos = b.astype(np.int64)
    vals = [cos.ravel()]
    for j in range(8):
        x = (blocks[:, :, j] - cos) // 2
        for bb in (0, 1):
            vals.append(x[cos == bb])
    # order: table 0, then 1 + 2j + b
    return [vals[0]] + [vals[1 + 2 * j + bb] for j in range(8) for bb in (0, 1)]


@pytest.mark.parametrize("target", [4.0, 7.0, 9.0])
def test_stream_tables_follow_the_window_rule(target):
    """End to end: at high rates the outliers spread the coordinates over more than 255 values, so
    windows and escapes occur; each table's window and escape count equal the brute-force rule on
    the histogram of the decoded coordinates."""
    w = W.gaussian_with_outliers(64, 1024, seed=21, outlier_frac=0.004)
    s, _ = oracle.compress(w, target)
    q, b = oracle.decode_symbols(s)
    lo, S, f = oracle.tables(s)
    vals = table_histograms(q, b)
    total_esc = 0
    for t in range(17):
        if len(vals[t]) == 0:
            continue
        blo, bS, besc = window_brute(vals[t])
        assert (lo[t], S[t]) == (blo, bS), t
        assert (f[t][255] > 0) == (besc > 0) or t == 0, t
        total_esc += besc if t > 0 else 0
    assert oracle.info(s)["n_escapes"] == total_esc
    if target >= 7.0:
        assert total_esc > 0 and (S[1:] == 255).any(), "the case must exercise windows and escapes"


# ------------------------------------------------------------------------------- lossy stream reader
def u16(s, o):
    return struct.unpack_from("<H", s, o)[0]


def u32(s, o):
    return struct.unpack_from("<I", s, o)[0]


def u64(s, o):
    return struct.unpack_from("<Q", s, o)[0]


def read_lossy_stream(s: bytes):
    """Doubled coordinates [Rp, Cp] and cosets [Rp, Cp / 8] of a lossy stream, read from its bytes
    with the layout: 128-byte header, tables (i16 window start, u16 width, u16 escape frequency,
    u16 frequencies), tile index of u32 offsets in 4-byte units, tiles of 32 u32 states then u16
    words. Header byte 116 says how a tile's 32 x tile_rows blocks are dealt to the states: 0, by
    rows (block step = tile row, lane = block column); 1, by columns of lanes (lane l stays on
    row l mod tile_rows and walks its blocks left to right, interleaved with the other lanes of
    that row)."""
    assert s[:4] == b"EPK1" and s[6] == 0
    R, C, tr = u32(s, 8), u32(s, 12), u16(s, 16)
    layout = s[116]
    assert layout in (0, 1)
    per_row = LANES // tr                                   # lanes sharing a row in layout 1

    def block(bs, l):
        """(tile row, block column) coded by lane l at block step bs."""
        if layout == 0:
            return bs, l
        return l % tr, bs * per_row + l // tr
    assert u16(s, 18) == 256 and u16(s, 20) == LANES
    n, nt, ntiles = s[22], s[23], u32(s, 32)
    o_tb, o_ix, o_pl = u64(s, 56), u64(s, 64), u64(s, 72)
    M = 1 << n
    lo, freqs = [], []
    pos = o_tb
    for _ in range(nt):
        start, width, esc = struct.unpack_from("<hHH", s, pos)
        pos += 6
        f = np.zeros(256, np.int64)
        f[:width] = struct.unpack_from("<%dH" % width, s, pos)
        pos += 2 * width
        f[255] += esc
        assert f.sum() == M
        lo.append(start)
        freqs.append(f)
    cum = [np.concatenate([[0], np.cumsum(f)[:-1]]) for f in freqs]
    slot_sym = [np.repeat(np.arange(256), f) for f in freqs]        # slot -> symbol
    Rp, Cp = -(-R // tr) * tr, -(-C // 256) * 256
    tiles_c = Cp // 256
    assert ntiles == (Rp // tr) * tiles_c
    index = struct.unpack_from("<%dI" % (ntiles + 1), s, o_ix)
    q = np.zeros((Rp, Cp), np.int64)
    cos = np.zeros((Rp, Cp // 8), np.int64)
    for t in range(ntiles):
        a, e = o_pl + 4 * index[t], o_pl + 4 * index[t + 1]
        tile = s[a:e]
        x = list(struct.unpack_from("<32I", tile, 0))
        words = struct.unpack_from("<%dH" % ((len(tile) - 128) // 2), tile, 128)
        k = 0
        r0, c0 = (t // tiles_c) * tr, (t % tiles_c) * 256
        b = [0] * LANES
        for step in range(9 * tr):
            bs, m = divmod(step, 9)
            syms = [0] * LANES
            tabs = [0 if m == 0 else 1 + 2 * (m - 1) + b[l] for l in range(LANES)]
            for l in range(LANES):
                T = tabs[l]
                slot = x[l] % M
                sym = int(slot_sym[T][slot])
                x[l] = int(freqs[T][sym]) * (x[l] // M) + slot - int(cum[T][sym])
                syms[l] = sym
            for l in range(LANES):                          # refills, ascending lanes
                if x[l] < L:
                    x[l] = (x[l] << 16) | words[k]
                    k += 1
            for l in range(LANES):                          # then escapes, ascending lanes
                rr, kk = block(bs, l)
                if m == 0:
                    b[l] = lo[0] + syms[l]
                    cos[r0 + rr, c0 // 8 + kk] = b[l]
                    continue
                if syms[l] == 255:
                    v = struct.unpack("<h", struct.pack("<H", words[k]))[0]
                    k += 1
                else:
                    v = lo[tabs[l]] + syms[l]
                q[r0 + rr, c0 + 8 * kk + (m - 1)] = 2 * v + b[l]
        assert all(v == L for v in x), f"tile {t}: final states"
        assert len(words) - k in (0, 1), f"tile {t}: words left over"
    return q, cos, (R, C)


@pytest.mark.parametrize("shape,target,prob_bits,tile_rows", [
    ((32, 512), 8.0, 12, 16),        # escapes (outliers at a high rate)
    ((40, 300), 4.0, 10, 16),        # ragged: padding rows and columns
    ((64, 256), 6.0, 11, 32),        # 32-row tiles
])
@pytest.mark.parametrize("layout", [0, 1])
def test_python_reader_matches_oracle_decoder(shape, target, prob_bits, tile_rows, layout):
    w = W.gaussian_with_outliers(*shape, seed=31, outlier_frac=0.003)
    s, _ = oracle.compress(w, target, prob_bits=prob_bits, tile_rows=tile_rows, layout=layout)
    assert oracle.info(s)["layout"] == layout
    q, cos, (R, C) = read_lossy_stream(s)
    qo, bo = oracle.decode_symbols(s)
    assert np.array_equal(q[:R, :C], qo.astype(np.int64))
    assert np.array_equal(cos[:R, :(C + 7) // 8], bo.astype(np.int64))
    assert not q[R:].any() and not q[:, C:].any(), "zero padding quantizes to the origin"
    if target >= 8.0:
        assert oracle.info(s)["n_escapes"] > 0


def test_window_range_rule_rejects_out_of_range_tables():
    """A coordinate table whose window leaves [-16384, 16383] (its doubled coordinates would not fit
    int16) is refused by the oracle's validator even with every checksum made consistent."""
    import zlib
    w = W.gaussian_with_outliers(16, 256, seed=5)
    s, _ = oracle.compress(w, 4.0)
    o_tb, o_pl = u64(s, 56), u64(s, 72)
    # the window start of table 1 (after table 0: 6 bytes + 2 per symbol)
    S0 = u16(s, o_tb + 2)
    t1 = o_tb + 6 + 2 * S0
    for start in (-16385, 16383 - u16(s, t1 + 2) + 2):
        bad = bytearray(s)
        struct.pack_into("<h", bad, t1, start)
        struct.pack_into("<I", bad, 112, zlib.crc32(bytes(bad[:112] + bad[116:o_pl])))
        with pytest.raises(oracle.OracleError) as e:
            oracle.info(bytes(bad))
        assert e.value.rc == -2
    ok = bytearray(s)
    struct.pack_into("<h", ok, t1, -16384)
    struct.pack_into("<I", ok, 112, zlib.crc32(bytes(ok[:112] + ok[116:o_pl])))
    oracle.info(bytes(ok))


@pytest.mark.parametrize("shape,tile_rows,target", [
    ((48, 776), 16, 4.0),            # ragged rows and columns
    ((64, 512), 32, 3.0),            # 32-row tiles: one lane per row
    ((32, 1024), 16, 8.0),           # escapes
])
def test_layouts_decode_to_the_same_weights(shape, tile_rows, target):
    """Reading R27: the layout changes only which state codes a block, so both layouts give the
    same step, tables, escapes and decoded weights in every container (BF16, FP8 with its row
    scales), and payloads of about the same size (the same symbols, coded by other states)."""
    w = W.gaussian_with_outliers(*shape, seed=sum(shape), outlier_frac=0.002)
    s0, _ = oracle.compress(w, target, tile_rows=tile_rows, layout=0)
    s1, _ = oracle.compress(w, target, tile_rows=tile_rows, layout=1)
    i0, i1 = oracle.info(s0), oracle.info(s1)
    assert (i0["layout"], i1["layout"]) == (0, 1)
    for k in ("step", "n_escapes", "n_tiles", "meta_bytes"):
        assert i0[k] == i1[k], k
    t0, t1 = oracle.tables(s0), oracle.tables(s1)
    for a, b in zip(t0, t1):
        assert np.array_equal(a, b)
    assert abs(i0["payload_bytes"] - i1["payload_bytes"]) <= 0.01 * i0["payload_bytes"] + 64
    assert np.array_equal(oracle.decompress(s0, oracle.BF16)[0], oracle.decompress(s1, oracle.BF16)[0])
    f0, sc0 = oracle.decompress(s0, oracle.F8E4M3)
    f1, sc1 = oracle.decompress(s1, oracle.F8E4M3)
    assert np.array_equal(f0, f1) and np.array_equal(sc0, sc1)
    if target >= 8.0:
        assert i1["n_escapes"] > 0


def test_layout_byte_is_validated():
    """The layout byte (header byte 116) takes 0 or 1, and 1 only in the lossy mode: other values
    are refused as corrupt even with the metadata checksum made consistent, and the encoder refuses
    layout 1 for the lossless modes."""
    import zlib
    w = W.gaussian_with_outliers(16, 256, seed=9)
    s, _ = oracle.compress(w, 4.0, layout=1)
    bits = np.frombuffer(np.float32(w).astype(np.float32).tobytes(), np.uint32)
    sl, _ = oracle.compress((bits >> 16).astype(np.uint16).reshape(w.shape), dtype=oracle.BF16,
                            mode=oracle.LOSSLESS)
    for stream, value in ((s, 2), (s, 255), (sl, 1)):
        o_pl = u64(stream, 72)
        bad = bytearray(stream)
        bad[116] = value
        struct.pack_into("<I", bad, 112, zlib.crc32(bytes(bad[:112] + bad[116:o_pl])))
        with pytest.raises(oracle.OracleError) as e:
            oracle.info(bytes(bad))
        assert e.value.rc == -2
    with pytest.raises(oracle.OracleError) as e:
        oracle.compress((bits >> 16).astype(np.uint16).reshape(w.shape), dtype=oracle.BF16,
                        mode=oracle.LOSSLESS, layout=1)
    assert e.value.rc == -1
