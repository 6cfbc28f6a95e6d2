"""Host-side tests of the product library (no GPU): the C ABI exports, the threaded host encoder
against the oracle encoder (byte-identical streams), and stream validation errors.

Encoder parity: both encoders implement the same stream definition independently (the oracle in
plain C, the product in threaded C++), so equal bytes on varied inputs pin the product's
quantizer, model, rate search and tile coder to the oracle, whose own pins live in the
test_oracle_* files."""
import os
import re

import numpy as np
import pytest

import oracle
import decode_tile_interleaved_rans_amd as ep
from decode_tile_interleaved_rans_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(ep_\w+)\s*\(", src, re.M))
    return names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"ep_compress", "ep_upload", "ep_decompress", "ep_linear_forward"} <= names
    L = ep.lib()
    for n in sorted(names):
        assert hasattr(L, n), n
    assert set(ep.EXPORTS) == names
    assert b"gfx950" in L.ep_version()


def test_every_declaration_cites_its_passage():
    """Each exported call's comment names the page and section (or the reading) that defines it."""
    src = open(os.path.join(ROOT, "include", "entropack.h")).read()
    decls = list(re.finditer(r"^(?:const\s+)?\w+\*?\s+\**(ep_\w+)\s*\(", src, re.M))
    assert len(decls) == len(declared_functions())
    for m in decls:
        before = src[:m.start()]
        comment = before[before.rfind("/*"):]
        assert comment.rstrip().endswith("*/"), m.group(1)
        assert "Source:" in comment and ('"EntroPack' in comment or "reading R" in comment), m.group(1)


def test_header_is_plain_c():
    # the C ABI header compiles as C11 on its own, warnings as errors (no C++ constructs leak)
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-x", "c",
                        os.path.join(root, "include", "entropack.h")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def oracle_and_product(w, target, dtype=None, mode=0, prob_bits=12, tile_rows=16, threads=4, layout=0):
    so, bo = oracle.compress(w, target, dtype=dtype, mode=mode, prob_bits=prob_bits, tile_rows=tile_rows,
                             layout=layout)
    sp, bp = ep.compress(w, target, dtype=dtype, mode=mode, prob_bits=prob_bits, tile_rows=tile_rows,
                         n_threads=threads, layout=layout)
    return so, sp, bo, bp


@pytest.mark.parametrize("target", [2.5, 4.0, 6.0])
def test_encoder_matches_oracle_gaussian_outliers(target):
    w = W.gaussian_with_outliers(1024, 1024, seed=1)
    so, sp, bo, bp = oracle_and_product(w, target)
    assert so == sp and bo == bp


@pytest.mark.parametrize("shape,prob_bits,tile_rows", [((100, 300), 10, 16), ((33, 513), 11, 32), ((16, 256), 12, 16),
                                                       ((1, 9), 12, 16), ((257, 1000), 12, 32)])
def test_encoder_matches_oracle_shapes(shape, prob_bits, tile_rows):
    rng = np.random.default_rng(sum(shape) + prob_bits)
    w = (0.02 * rng.standard_t(5, shape)).astype(np.float32)
    w[rng.random(shape) < 0.003] *= 40
    so, sp, *_ = oracle_and_product(w, 4.5, prob_bits=prob_bits, tile_rows=tile_rows, threads=3)
    assert so == sp


def test_encoder_matches_oracle_bf16_rowscaled():
    w = W.student_t_rowscaled(512, 768, 2)
    so, sp, *_ = oracle_and_product(w, 3.0, dtype=ep.BF16, threads=8)
    assert so == sp


def test_encoder_matches_oracle_fp16_and_escapes():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 0.01, (64, 512)).astype(np.float32)
    x[rng.random(x.shape) < 0.002] = 3.0
    h = x.astype(np.float16).view(np.uint16)
    so, sp, *_ = oracle_and_product(h, 7.0, dtype=ep.F16)
    assert so == sp
    assert oracle.info(so)["n_escapes"] > 0


@pytest.mark.parametrize("shape,target,prob_bits,tile_rows", [
    ((100, 300), 4.5, 10, 16), ((33, 513), 4.0, 11, 32), ((64, 512), 8.0, 12, 16), ((1, 9), 4.0, 11, 16),
    ((0, 7), 4.0, 12, 16)])
def test_encoder_matches_oracle_row_layout(shape, target, prob_bits, tile_rows):
    """The row layout (each rANS state on one tile row, reading R27): the same bytes as the
    oracle, ragged shapes, 32-row tiles, escapes and an empty matrix included."""
    w = W.gaussian_with_outliers(*shape, seed=sum(shape), outlier_frac=0.003) if shape[0] else np.zeros(shape, np.float32)
    so, sp, *_ = oracle_and_product(w, target, prob_bits=prob_bits, tile_rows=tile_rows, threads=3,
                                    layout=ep.ROW_LAYOUT)
    assert so == sp
    assert ep.stream_info(sp)["layout"] == ep.ROW_LAYOUT == oracle.info(so)["layout"]
    if target >= 8.0:
        assert oracle.info(so)["n_escapes"] > 0


def test_encoder_matches_oracle_degenerate():
    for w in [np.zeros((40, 300), np.float32), np.zeros((0, 7), np.float32), np.full((16, 256), 0.5, np.float32)]:
        so, sp, *_ = oracle_and_product(w, 4.0)
        assert so == sp


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32", "u8"])
def test_lossless_encoder_matches_oracle(dt):
    rng = np.random.default_rng(4)
    shape = (37, 600)
    if dt == "bf16":
        x, code = W.student_t_rowscaled(*shape, seed=9), ep.BF16
    elif dt == "f16":
        x, code = rng.normal(0, 1, shape).astype(np.float16).view(np.uint16), ep.F16
    elif dt == "f32":
        x, code = rng.normal(0, 1, shape).astype(np.float32).view(np.uint32), ep.F32
    else:
        x, code = rng.integers(0, 7, shape).astype(np.uint8), ep.U8
    so, sp, *_ = oracle_and_product(x, 0.0, dtype=code, mode=ep.LOSSLESS)
    assert so == sp


@pytest.mark.parametrize("shape,prob_bits,tile_rows", [((37, 600), 12, 16), ((5, 9), 10, 16), ((64, 1024), 11, 32),
                                                      ((0, 256), 12, 16)])
def test_exponent_coded_encoder_matches_oracle(shape, prob_bits, tile_rows):
    rng = np.random.default_rng(sum(shape))
    x = W.student_t_rowscaled(*shape, seed=9) if shape[0] else np.zeros(shape, np.uint16)
    if x.size:
        x.ravel()[rng.choice(x.size, min(7, x.size), replace=False)] = [0x7F80, 0xFF80, 0x7FC1, 0x0001, 0x8000,
                                                                      0x807F, 0xFFFF][:min(7, x.size)]
    so, sp, *_ = oracle_and_product(x, 0.0, dtype=ep.BF16, mode=ep.LOSSLESS_EXP, prob_bits=prob_bits,
                                    tile_rows=tile_rows)
    assert so == sp
    a, b = ep.stream_info(sp), oracle.info(so)
    assert a["payload_bytes"] == b["payload_bytes"] and a["meta_bytes"] == b["meta_bytes"] and a["mode"] == 2


def test_exponent_coded_validation():
    x = W.student_t_rowscaled(32, 512, seed=1)
    s, _ = ep.lossless_compress(x, exponent_coded=True, dtype=ep.BF16)
    o_raw = int.from_bytes(s[96:104], "little")
    bad = bytearray(s)
    bad[o_raw + 100] ^= 4                           # raw plane byte: its CRC-32 catches it
    with pytest.raises(ep.EPError) as e:
        ep.stream_info(bytes(bad))
    assert e.value.status == -2
    bad = bytearray(s)
    bad[96:104] = (o_raw + 16).to_bytes(8, "little")   # raw plane overlapping the payload
    with pytest.raises(ep.EPError) as e:
        ep.stream_info(bytes(bad))
    assert e.value.status == -2
    bad = bytearray(s)
    bad[7] = ep.F16                                  # exponent coding is defined for BF16 only
    with pytest.raises(ep.EPError) as e:
        ep.stream_info(bytes(bad))
    assert e.value.status == -2
    with pytest.raises(ep.EPError) as e:
        ep.compress(x.view(np.uint16), 0.0, mode=ep.LOSSLESS_EXP, dtype=ep.F16)
    assert e.value.status == -3
    s1, _ = ep.lossless_compress(x, dtype=ep.BF16)
    bad = bytearray(s1)
    bad[104] = 1                                     # raw plane CRC in a two-plane stream
    with pytest.raises(ep.EPError) as e:
        ep.stream_info(bytes(bad))
    assert e.value.status == -2


@pytest.mark.slow
def test_encoder_matches_oracle_4096_student_t():
    w = W.student_t_rowscaled(4096, 4096, 2)
    for t in (3.0, 4.0, 4.5):
        so, sp, *_ = oracle_and_product(w, t, dtype=ep.BF16, threads=8)
        assert so == sp
    so, sp, *_ = oracle_and_product(w, 0.0, dtype=ep.BF16, mode=ep.LOSSLESS, threads=8)
    assert so == sp
    so, sp, *_ = oracle_and_product(w, 0.0, dtype=ep.BF16, mode=ep.LOSSLESS_EXP, threads=8)
    assert so == sp


def test_stream_info_matches_oracle():
    w = W.gaussian_with_outliers(256, 512, seed=2)
    s, bpp = ep.compress(w, 4.0)
    a, b = ep.stream_info(s), oracle.info(s)
    assert a["rows"] == b["rows"] and a["payload_bytes"] == b["payload_bytes"] and a["n_tiles"] == b["n_tiles"]
    assert a["actual_bpp"] == bpp == 8 * len(s) / w.size
    assert a["meta_bytes"] + a["payload_bytes"] == len(s)


def test_every_single_bit_flip_is_rejected():
    # the payload, raw-plane and metadata CRC-32s leave no bit of a stream unchecked; the host
    # validator must refuse every single-bit corruption (a flipped row scale, step, shape or table
    # window would otherwise decode to a wrong tensor without an error)
    rng = np.random.default_rng(3)
    w = rng.normal(0, 0.02, (16, 256)).astype(np.float32)
    w[2, 9] = 1.0
    streams = [ep.compress(w, 2.0)[0],
               ep.lossless_compress(W.student_t_rowscaled(16, 256, seed=4), dtype=ep.BF16, exponent_coded=True)[0],
               ep.lossless_compress(rng.integers(0, 40, (16, 256)).astype(np.uint8))[0]]
    for st in streams:
        ep.stream_info(st)
        accepted = []
        for i in range(len(st)):
            for b in range(8):
                bad = bytearray(st)
                bad[i] ^= 1 << b
                try:
                    ep.stream_info(bytes(bad))
                    accepted.append((i, b))
                except ep.EPError as e:
                    assert e.status == -2
        assert not accepted, accepted[:10]


def test_validation_errors():
    w = W.gaussian_with_outliers(64, 512, seed=3)
    s, _ = ep.compress(w, 4.0)
    cases = {
        "magic": b"EPK2" + s[4:],
        "truncated": s[:-4],
        "header": s[:100],
        "crc": s[:-10] + bytes([s[-10] ^ 1]) + s[-9:],
        "table_sum": s[:0x200] + s[0x200:],  # placeholder replaced below
    }
    info = oracle.info(s)
    off_tables = int.from_bytes(s[56:64], "little")
    bad = bytearray(s)
    bad[off_tables + 6] ^= 1                       # first frequency of table 0
    cases["table_sum"] = bytes(bad)
    bad = bytearray(s)
    off_index = int.from_bytes(s[64:72], "little")
    bad[off_index + 4:off_index + 8] = (10).to_bytes(4, "little")   # tile 0 shorter than its states
    cases["index"] = bytes(bad)
    for name, blob in cases.items():
        with pytest.raises(ep.EPError) as e:
            ep.stream_info(blob)
        assert e.value.status == -2, name
    assert info["n_tiles"] == 8


def wide_lossless_u8_stream(cols: int) -> bytes:
    """An intact one-row lossless U8 stream of `cols` columns with an all-zero payload (every tile
    holding just its 32 states), put together from a small encoder-written stream: the shape,
    section offsets, tile index and both CRC-32s rewritten (the validator does not decode)."""
    import zlib
    base, _ = ep.lossless_compress(np.zeros((1, 256), np.uint8))
    r64 = lambda o: int.from_bytes(base[o:o + 8], "little")
    off_tables, off_index = r64(56), r64(64)
    tables = base[off_tables:off_index]
    n_tiles = -(-cols // 256)
    index = (np.arange(n_tiles + 1, dtype=np.uint32) * 32).tobytes()
    off_payload = -(-(off_index + len(index)) // 16) * 16
    payload = bytes(128 * n_tiles)
    total = off_payload + len(payload)
    h = bytearray(base[:128])
    h[12:16] = cols.to_bytes(4, "little")
    h[32:36] = n_tiles.to_bytes(4, "little")
    h[64:72] = off_index.to_bytes(8, "little")
    h[72:80] = off_payload.to_bytes(8, "little")
    h[80:88] = total.to_bytes(8, "little")
    h[88:92] = zlib.crc32(payload).to_bytes(4, "little")
    body = bytes(h[:off_tables]) + tables + index + bytes(off_payload - off_index - len(index))
    meta = zlib.crc32(body[:112] + body[116:])
    body = body[:112] + meta.to_bytes(4, "little") + body[116:]
    return body + payload


def test_stream_wider_than_the_encoders_write_is_refused():
    """The encoders refuse 2^28 or more columns (the decode kernels address an output row with 32-bit
    byte offsets); an intact stream that wide is refused by the validator with EP_ERANGE, and one
    tile narrower passes (so the refusal is the width rule, not a flaw of the constructed stream)."""
    ok = wide_lossless_u8_stream((1 << 28) - 256)
    assert ep.stream_info(ok)["cols"] == (1 << 28) - 256
    del ok
    with pytest.raises(ep.EPError) as e:
        ep.stream_info(wide_lossless_u8_stream(1 << 28))
    assert e.value.status == -4


def test_bad_arguments():
    w = np.zeros((4, 4), np.float32)
    with pytest.raises(ep.EPError) as e:
        ep.compress(w, 0.0)
    assert e.value.status == -1
    with pytest.raises(ep.EPError) as e:
        ep.compress(w, 4.0, prob_bits=9)
    assert e.value.status == -1
    with pytest.raises(ep.EPError) as e:
        ep.compress(np.zeros((4, 4), np.uint8), 4.0, dtype=ep.U8)
    assert e.value.status == -3
    bad = np.ones((4, 4), np.float32)
    bad[1, 1] = np.inf
    with pytest.raises(ep.EPError) as e:
        ep.compress(bad, 4.0)
    assert e.value.status == -4


def test_saved_stream_reloads_in_a_fresh_process(tmp_path):
    """Save / reload ("EntroPack PyTorch Guide", section "Test saved artifacts"): a stream and its
    bias written to disk are read back by a new Python process, which decodes the stream with
    the oracle; the result equals the oracle's decode of the original stream bit for bit."""
    import subprocess
    import sys
    w = W.gaussian_with_outliers(96, 700, seed=21)
    s, _ = ep.compress(w, 4.5)
    bias = W.to_bf16_bits(np.linspace(-1, 1, 96))
    path = tmp_path / "layer.npz"
    ep.save(path, s, bias)
    out = tmp_path / "decoded.npy"
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys, numpy as np; sys.path.insert(0, %r); import oracle, decode_tile_interleaved_rans_amd as ep; "
            "s, b = ep.load(%r); q, _ = oracle.decompress(s, oracle.BF16); "
            "np.save(%r, np.concatenate([q.ravel(), b]))") % (root, str(path), str(out))
    subprocess.run([sys.executable, "-c", code], check=True, timeout=120)
    got = np.load(out)
    want, _ = oracle.decompress(s, oracle.BF16)
    assert np.array_equal(got, np.concatenate([want.ravel(), bias]))


def test_load_rejects_a_damaged_file(tmp_path):
    w = W.gaussian_with_outliers(32, 256, seed=22)
    s, _ = ep.compress(w, 4.0)
    bad = bytearray(s)
    bad[-3] ^= 0x5A                                        # payload byte: the CRC no longer matches
    path = tmp_path / "bad.npz"
    ep.save(path, bytes(bad))
    with pytest.raises(ep.EPError) as e:
        ep.load(path)
    assert e.value.status == -2


def test_new_entry_points_reject_bad_arguments_before_any_device_work():
    """Argument checks of the FP8 forward, the quantizer, the BF16 and FP8 GEMMs and the device
    encoder return EP_EINVAL / EP_EUNSUPPORTED / EP_ERANGE without touching a device."""
    import ctypes as C
    L = ep.lib()
    out = C.POINTER(C.c_uint8)()
    n = C.c_size_t()
    assert L.ep_linear_forward_fp8(None, None, 4, None, None, None) == -1           # null handle
    assert L.ep_quantize_rows_fp8(None, 4, 32, None, None, None) == -1              # null pointers
    assert L.ep_quantize_rows_fp8(C.c_void_p(16), 4, 24, C.c_void_p(16), C.c_void_p(16), None) == -1   # K % 16
    assert L.ep_gemm_fp8(C.c_void_p(16), C.c_void_p(16), C.c_void_p(16), C.c_void_p(16), 4, 4, 24, None,
                         C.c_void_p(16), None) == -1                                  # K % 16
    assert L.ep_gemm_fp8(None, None, None, None, 0, 4, 16, None, None, None) == 0    # empty: nothing to do
    p16 = C.c_void_p(16)
    assert L.ep_gemm_fp8(p16, p16, p16, p16, 4, 1 << 31, 16, None, p16, None) == -4  # N past 32-bit sizes
    assert L.ep_quantize_rows_fp8(p16, 1 << 31, 32, p16, p16, None) == -4           # M past 32-bit sizes
    assert L.ep_gemm_bf16(p16, p16, 4, 4, 12, p16, None) == -1                      # K % 8
    assert L.ep_gemm_bf16(p16, p16, 1 << 31, 4, 16, p16, None) == -4                # M past 32-bit sizes
    assert L.ep_compress_device(None, ep.F32, 4, 4, None, None, C.byref(out), C.byref(n), None) == -1
    opts = ep.EncodeOpts(ep.LOSSLESS, 0.0, 12, 16, 0)
    assert L.ep_compress_device(C.c_void_p(16), ep.BF16, 4, 4, C.byref(opts), None, C.byref(out), C.byref(n),
                                None) == -3                                           # lossless: host encoder only
    opts = ep.EncodeOpts(ep.LOSSY, 4.0, 12, 16, 0)
    assert L.ep_compress_device(C.c_void_p(16), ep.U8, 4, 4, C.byref(opts), None, C.byref(out), C.byref(n),
                                None) == -3                                           # lossy takes float input
    assert L.ep_compress_device(C.c_void_p(16), ep.F32, 4, 1 << 28, C.byref(opts), None, C.byref(out), C.byref(n),
                                None) == -4                                           # too wide
    opts = ep.EncodeOpts(ep.LOSSY, 0.0, 12, 16, 0)
    assert L.ep_compress_device(C.c_void_p(16), ep.F32, 4, 4, C.byref(opts), None, C.byref(out), C.byref(n),
                                None) == -1                                           # target must be > 0
    opts = ep.EncodeOpts(ep.LOSSY, 4.0, 12, 16, 0, 2)
    assert L.ep_compress_device(C.c_void_p(16), ep.F32, 4, 4, C.byref(opts), None, C.byref(out), C.byref(n),
                                None) == -1                                           # layout 0 or 1
    w = np.zeros((4, 4), np.float32)
    assert L.ep_compress(w.ctypes.data_as(C.c_void_p), ep.F32, 4, 4, C.byref(opts), C.byref(out), C.byref(n),
                         None) == -1
    opts = ep.EncodeOpts(ep.LOSSLESS, 0.0, 12, 16, 0, 1)                               # layout 1 is lossy only
    assert L.ep_compress(w.ctypes.data_as(C.c_void_p), ep.F32, 4, 4, C.byref(opts), C.byref(out), C.byref(n),
                         None) == -1


def test_concurrent_compress_calls_from_threads():
    # the host encoder and the error-message store are per call / per thread: four threads
    # compressing different matrices at once give the same bytes as one after the other, and an
    # error in one thread leaves the others' messages alone
    import threading
    mats = [W.gaussian_with_outliers(96, 512, seed=20 + i) for i in range(4)]
    want = [ep.compress(m, 3.0 + 0.5 * i, n_threads=2)[0] for i, m in enumerate(mats)]
    got, errs = [None] * 4, []

    def work(i):
        try:
            for _ in range(3):
                got[i] = ep.compress(mats[i], 3.0 + 0.5 * i, n_threads=2)[0]
                with pytest.raises(ep.EPError):
                    ep.stream_info(b"EPK1" + bytes(200))
        except Exception as e:   # surfaced below
            errs.append(e)

    ts = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errs, errs
    assert got == want
