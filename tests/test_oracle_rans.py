"""Pins of the oracle's tile rANS coder (entropy coding in tiles that decode on their own,
EntroPack paper, Abstract; rANS after Duda arXiv:1311.2540, interleaved states after Giesen
arXiv:1402.3392).

Pins: exact round trips over extreme tables (one symbol with f = M; f = 1 and M - 1; 256
symbols; n = 10, 11, 12), escapes, the final decoder state L in every lane, the coded size
against the ideal code length, and a separate pure-Python decoder written from the byte layout
that must read the oracle encoder's bytes back to the same symbols."""
import struct

import numpy as np
import pytest

import oracle

L = 1 << 16
LANES = 32


def random_freqs(rng, n, nsym, min_f=1):
    """Frequencies over the first nsym symbols summing to 2^n, each >= min_f."""
    M = 1 << n
    cuts = np.sort(rng.choice(np.arange(1, M - nsym * min_f + nsym), nsym - 1, replace=False))
    parts = np.diff(np.r_[0, cuts, M - nsym * min_f + nsym]) - 1 + min_f
    f = np.zeros(256, np.uint32)
    f[:nsym] = parts
    assert f.sum() == M and f[:nsym].min() >= min_f
    return f


def draw(rng, f, shape):
    p = f / f.sum()
    return rng.choice(256, size=shape, p=p).astype(np.uint8)


def py_decode(tile: bytes, freqs, n, tab, esc_sym=-1):
    """Independent reader of one tile: 32 u32 LE states (lane 0 first), then u16 LE words; per
    step every lane decodes, then lanes with state < 2^16 take a refill word in ascending lane
    order, then escape lanes take a raw word in ascending lane order."""
    M = 1 << n
    cum = [np.concatenate([[0], np.cumsum(f.astype(np.int64))[:-1]]) for f in freqs]
    x = list(struct.unpack("<32I", tile[:128]))
    words = struct.unpack("<%dH" % ((len(tile) - 128) // 2), tile[128:])
    k = 0
    syms = np.zeros(tab.shape, np.uint8)
    escs = np.zeros(tab.shape, np.uint16)
    for t in range(tab.shape[0]):
        for lane in range(LANES):
            T = tab[t, lane]
            slot = x[lane] % M
            s = int(np.searchsorted(cum[T], slot, side="right") - 1)
            while freqs[T][s] == 0:          # zero-frequency symbols share a cumulative value
                s -= 1
            x[lane] = int(freqs[T][s]) * (x[lane] // M) + slot - int(cum[T][s])
            syms[t, lane] = s
        for lane in range(LANES):
            if x[lane] < L:
                x[lane] = (x[lane] << 16) | words[k]
                k += 1
        for lane in range(LANES):
            if esc_sym >= 0 and syms[t, lane] == esc_sym:
                escs[t, lane] = words[k]
                k += 1
    return syms, escs, x, k, len(words)


def roundtrip(freqs, n, tab, sym, esc=None, esc_sym=-1):
    tile = oracle.rans_encode(freqs, n, tab, sym, esc, esc_sym)
    rc, s2, e2, fin = oracle.rans_decode(freqs, n, tab, tile, esc_sym)
    assert rc == 0
    assert np.array_equal(s2, sym)
    if esc is not None:
        m = sym == esc_sym
        assert np.array_equal(e2[m], esc[m])
    assert np.all(fin == L), "every lane ends at the initial encoder state"
    return tile


@pytest.mark.parametrize("n", [10, 11, 12])
def test_single_symbol_table_costs_no_words(n):
    f = np.zeros((1, 256), np.uint32)
    f[0, 7] = 1 << n
    tab = np.zeros((144, LANES), np.uint8)
    sym = np.full((144, LANES), 7, np.uint8)
    tile = roundtrip(f, n, tab, sym)
    assert len(tile) == 128
    assert struct.unpack("<32I", tile) == (L,) * 32


@pytest.mark.parametrize("n", [10, 11, 12])
def test_extreme_two_symbol_table(n):
    rng = np.random.default_rng(n)
    M = 1 << n
    f = np.zeros((1, 256), np.uint32)
    f[0, 0], f[0, 1] = 1, M - 1
    tab = np.zeros((300, LANES), np.uint8)
    sym = (rng.random((300, LANES)) < 0.05).astype(np.uint8) ^ 1      # rare symbol 0 overrepresented
    roundtrip(f, n, tab, sym)


@pytest.mark.parametrize("n", [10, 11, 12])
def test_full_alphabet_and_many_tables(n):
    rng = np.random.default_rng(100 + n)
    freqs = np.stack([random_freqs(rng, n, 256), random_freqs(rng, n, 40), random_freqs(rng, n, 3)])
    tab = rng.integers(0, 3, (144, LANES)).astype(np.uint8)
    sym = np.zeros((144, LANES), np.uint8)
    for T in range(3):
        m = tab == T
        sym[m] = draw(rng, freqs[T], m.sum())
    tile = roundtrip(freqs, n, tab, sym)
    s2, _, x, k, nw = py_decode(tile, freqs, n, tab)
    assert np.array_equal(s2, sym) and all(v == L for v in x)
    assert k in (nw, nw - 1), "all words read, except one trailing pad word"


def test_escapes_roundtrip_and_word_order():
    rng = np.random.default_rng(7)
    n = 12
    f = random_freqs(rng, n, 20)
    f[255] = 37                               # escape symbol
    f[int(np.argmax(f[:20]))] -= 37
    freqs = f[None]
    tab = np.zeros((144, LANES), np.uint8)
    sym = draw(rng, f, (144, LANES))
    esc = rng.integers(0, 1 << 16, (144, LANES)).astype(np.uint16)
    assert (sym == 255).sum() > 0
    tile = roundtrip(freqs, n, tab, sym, esc, 255)
    s2, e2, x, k, nw = py_decode(tile, freqs, n, tab, 255)
    m = sym == 255
    assert np.array_equal(s2, sym) and np.array_equal(e2[m], esc[m])
    assert all(v == L for v in x)
    assert k == nw or (k == nw - 1 and struct.unpack("<H", tile[-2:])[0] == 0)
    assert len(tile) % 4 == 0


def test_code_length_near_ideal():
    """sum_l log2(X_l / L) + 16 W equals the ideal code length sum -log2(f_s / M) up to the rANS
    rounding, which stays within 32 bits + 1% of a bit per symbol here."""
    rng = np.random.default_rng(8)
    n = 12
    M = 1 << n
    f = random_freqs(rng, n, 60)
    tab = np.zeros((288, LANES), np.uint8)
    sym = draw(rng, f, (288, LANES))
    tile = roundtrip(f[None], n, tab, sym)
    X = np.array(struct.unpack("<32I", tile[:128]), np.float64)
    nw = (len(tile) - 128) // 2
    coded = np.log2(X / L).sum() + 16 * nw
    ideal = -np.log2(f[sym].astype(np.float64) / M).sum()
    assert abs(coded - ideal) <= 32 + 0.01 * sym.size + 16      # +16: the optional pad word


def test_corrupt_tiles_are_rejected():
    rng = np.random.default_rng(9)
    n = 12
    f = random_freqs(rng, n, 30)[None]
    tab = np.zeros((144, LANES), np.uint8)
    sym = draw(rng, f[0], (144, LANES))
    tile = oracle.rans_encode(f, n, tab, sym)
    rc, *_ = oracle.rans_decode(f, n, tab, tile[:-4])           # truncated
    assert rc == -2
    rc, *_ = oracle.rans_decode(f, n, tab, tile + b"\0\0\0\0")  # trailing words
    assert rc == -2
    bad = bytearray(tile)
    bad[5] ^= 0x40                                              # damaged state of lane 1
    rc, *_ = oracle.rans_decode(f, n, tab, bytes(bad))
    assert rc == -2


def test_exponent_coded_tiles_read_back_by_the_python_reader():
    """The exponent-coded lossless BF16 stream (the guide's DFloat11 config, "Choose a
    compression contract", read as exponent by tile rANS + raw sign/mantissa plane): every tile
    of the oracle's stream, read by py_decode with the stream's single table (one step per
    element, row -> element order, lane l on columns 8l..8l+7), joined with the raw plane, gives
    the input bits."""
    rng = np.random.default_rng(3)
    R, C = 33, 520
    x = (rng.standard_t(4, (R, C)) * 0.02).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)      # truncation is fine: any bit pattern
    s, _ = oracle.compress(bits, dtype=oracle.BF16, mode=oracle.LOSSLESS_EXP, prob_bits=11)
    info = oracle.info(s)
    _, _, f = oracle.tables(s)
    Rp, Cp, tr = 48, 768, 16
    o_ix = int.from_bytes(s[64:72], "little")
    o_pl = int.from_bytes(s[72:80], "little")
    o_raw = int.from_bytes(s[96:104], "little")
    raw = np.frombuffer(s[o_raw:o_raw + Rp * Cp], np.uint8).reshape(Rp, Cp).astype(np.uint16)
    index = np.frombuffer(s[o_ix:o_ix + 4 * (info["n_tiles"] + 1)], np.uint32)
    out = np.zeros((Rp, Cp), np.uint16)
    tab = np.zeros((tr * 8, LANES), np.uint8)
    for t in range(info["n_tiles"]):
        tile = s[o_pl + 4 * int(index[t]):o_pl + 4 * int(index[t + 1])]
        syms, _, fin, used, nwords = py_decode(tile, f, 11, tab)
        assert all(v == L for v in fin) and nwords - used in (0, 1)
        r0, c0 = t // 3 * tr, t % 3 * 256
        for rr in range(tr):
            for e in range(8):
                for lane in range(LANES):
                    r, c = r0 + rr, c0 + 8 * lane + e
                    rb = raw[r, c]
                    out[r, c] = ((rb & 0x80) << 8) | (int(syms[rr * 8 + e, lane]) << 7) | (rb & 0x7F)
    assert np.array_equal(out[:R, :C], bits)
    assert not out[R:].any() and not out[:, C:].any()
