"""Python access to the EPK1 oracle (plain scalar C in ``ep_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline leg
are the only users. The product package never imports this module, and this module imports
nothing from the product package.

The functions below only marshal arguments (numpy arrays <-> pointers); every step of the method
runs in the C file, whose header lists the pages and passages each part follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ep_oracle.c")
LIB = os.path.join(HERE, "libep_oracle.so")

# element type codes shared by the stream header
F32, BF16, F16, F8E4M3, I8, U8 = 0, 1, 2, 3, 4, 5
LOSSY, LOSSLESS, LOSSLESS_EXP = 0, 1, 2
STATUS = {0: "ok", -1: "invalid argument", -2: "corrupt stream", -3: "unsupported", -4: "out of range",
          -6: "out of memory"}


class OracleError(RuntimeError):
    def __init__(self, rc: int, what: str):
        super().__init__(f"oracle {what}: {STATUS.get(rc, rc)} ({rc})")
        self.rc = rc


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        cmd = ["gcc", "-O2", "-std=gnu11", "-Wall", "-fPIC", "-shared", "-ffp-contract=off",
               "-o", LIB + ".tmp", SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(LIB + ".tmp", LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = C.CDLL(LIB)
        vp, i64, sz = C.c_void_p, C.c_int64, C.c_size_t
        L.or_compress.argtypes = [vp, C.c_int, i64, i64, C.c_int, C.c_double, C.c_int, C.c_int, C.c_int,
                                  C.POINTER(C.POINTER(C.c_uint8)), C.POINTER(sz), C.POINTER(C.c_double)]
        L.or_free.argtypes = [vp]
        L.or_decompress.argtypes = [vp, sz, C.c_int, vp, vp, C.c_int]
        L.or_decode_symbols.argtypes = [vp, sz, vp, vp, C.c_int]
        L.or_decompress_tiles.argtypes = [vp, sz, C.c_int, vp, C.c_int, vp, vp, vp]
        L.or_stream_info.argtypes = [vp, sz, vp, vp]
        L.or_stream_tables.argtypes = [vp, sz, vp, vp, vp]
        L.or_e8_nearest_batch.argtypes = [vp, i64, vp, vp]
        L.or_e8_nearest_batch.restype = None
        L.or_normalize.argtypes = [vp, C.c_int, vp]
        L.or_choose_window.argtypes = [vp, i64, vp, vp, vp]
        L.or_estimate_bpp.argtypes = [vp, C.c_int, i64, i64, C.c_double]
        L.or_estimate_bpp.restype = C.c_double
        L.or_select_step.argtypes = [vp, C.c_int, i64, i64, C.c_double]
        L.or_select_step.restype = C.c_float
        L.or_row_scale.argtypes = [vp, C.c_int, i64, i64, i64]
        L.or_row_scale.restype = C.c_float
        L.or_f32_to_bf16.argtypes = [C.c_float]
        L.or_f32_to_bf16.restype = C.c_uint16
        L.or_f32_to_f16.argtypes = [C.c_float]
        L.or_f32_to_f16.restype = C.c_uint16
        L.or_f32_to_e4m3.argtypes = [C.c_float]
        L.or_f32_to_e4m3.restype = C.c_uint8
        L.or_rans_encode.argtypes = [C.c_int, vp, C.c_int, C.c_int, vp, vp, vp, C.c_int, vp, sz, C.POINTER(sz)]
        L.or_rans_decode.argtypes = [C.c_int, vp, C.c_int, C.c_int, vp, C.c_int, vp, sz, vp, vp, vp]
        L.or_quantize_rows_e4m3.argtypes = [vp, i64, i64, vp, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _dtype_code(a: np.ndarray, dtype: int | None) -> int:
    if dtype is not None:
        return dtype
    if a.dtype == np.float32:
        return F32
    raise ValueError("pass dtype= for 16-bit or 8-bit inputs (given as uint16/uint8 bit patterns)")


def compress(w: np.ndarray, target_bpp: float = 4.0, *, dtype: int | None = None, mode: int = LOSSY,
             prob_bits: int = 12, tile_rows: int = 16, layout: int = 0) -> tuple[bytes, float]:
    """Encode a [R, C] matrix. 16-bit sources are passed as uint16 bit patterns with dtype=BF16/F16.
    layout (lossy only): which block of a tile each of its 32 interleaved states codes per block
    step; 0 = lane l takes block column l of each tile row in turn, 1 = lane l takes tile row
    l mod tile_rows, block columns (32 / tile_rows) s + l // tile_rows (block_of in ep_oracle.c)."""
    w = np.ascontiguousarray(w)
    R, Cc = w.shape
    out = C.POINTER(C.c_uint8)()
    n = C.c_size_t()
    bpp = C.c_double()
    rc = lib().or_compress(_ptr(w), _dtype_code(w, dtype), R, Cc, mode, target_bpp, prob_bits, tile_rows,
                           layout, C.byref(out), C.byref(n), C.byref(bpp))
    if rc != 0:
        raise OracleError(rc, "compress")
    data = C.string_at(out, n.value)
    lib().or_free(out)
    return data, bpp.value


def info(stream: bytes) -> dict:
    v = np.zeros(13, np.int64)
    f = np.zeros(2, np.float32)
    rc = lib().or_stream_info(stream, len(stream), _ptr(v), _ptr(f))
    if rc != 0:
        raise OracleError(rc, "stream_info")
    keys = ["rows", "cols", "mode", "dtype", "tile_rows", "prob_bits", "n_tiles", "n_escapes",
            "payload_bytes", "meta_bytes", "state_bytes", "total_bytes", "layout"]
    d = {k: int(x) for k, x in zip(keys, v)}
    d["step"], d["target_bpp"] = float(f[0]), float(f[1])
    return d


def tables(stream: bytes):
    lo = np.zeros(17, np.int32)
    S = np.zeros(17, np.int32)
    f = np.zeros((17, 256), np.uint32)
    n = lib().or_stream_tables(stream, len(stream), _ptr(lo), _ptr(S), _ptr(f))
    if n < 0:
        raise OracleError(n, "stream_tables")
    return lo[:n], S[:n], f[:n]


_EB = {F32: 4, BF16: 2, F16: 2, F8E4M3: 1, I8: 1, U8: 1}
_NP = {F32: np.uint32, BF16: np.uint16, F16: np.uint16, F8E4M3: np.uint8, I8: np.uint8, U8: np.uint8}


def decompress(stream: bytes, container: int = BF16, n_threads: int = 1):
    """Returns the container bit patterns [R, C] (uint16 / uint8 / uint32) and, for FP8 / INT8,
    the per-row scale (else None)."""
    d = info(stream)
    R, Cc = d["rows"], d["cols"]
    out = np.zeros((R, Cc), _NP[container])
    scale = np.zeros(max(R, 1), np.float32) if container in (F8E4M3, I8) and d["mode"] == LOSSY else None
    rc = lib().or_decompress(stream, len(stream), container, _ptr(out), _ptr(scale), n_threads)
    if rc != 0:
        raise OracleError(rc, "decompress")
    return out, (scale[:R] if scale is not None else None)


def decode_symbols(stream: bytes, n_threads: int = 1):
    """Doubled coordinates q [R, C] (int16) and cosets [R, ceil(C/8)] (uint8)."""
    d = info(stream)
    R, Cc = d["rows"], d["cols"]
    q = np.zeros((R, Cc), np.int16)
    b = np.zeros((R, (Cc + 7) // 8), np.uint8)
    rc = lib().or_decode_symbols(stream, len(stream), _ptr(q), _ptr(b), n_threads)
    if rc != 0:
        raise OracleError(rc, "decode_symbols")
    return q, b


def decompress_tiles(stream: bytes, tiles, container: int = BF16, want_q: bool = False, want_scale: bool = False):
    """Decode only the listed tiles: returns [n, tile_rows, 256] container bits, plus q
    [n, tile_rows, 256] if want_q and the rows' output scales [n, tile_rows] (FP8 / INT8) if
    want_scale, in that order."""
    d = info(stream)
    tiles = np.ascontiguousarray(np.asarray(tiles, np.uint32))
    n = len(tiles)
    out = np.zeros((n, d["tile_rows"], 256), _NP[container])
    q = np.zeros((n, d["tile_rows"], 256), np.int16) if want_q else None
    sc = np.zeros((n, d["tile_rows"]), np.float32) if want_scale else None
    rc = lib().or_decompress_tiles(stream, len(stream), container, _ptr(tiles), n, _ptr(out), _ptr(q), _ptr(sc))
    if rc != 0:
        raise OracleError(rc, "decompress_tiles")
    res = (out,) + ((q,) if want_q else ()) + ((sc,) if want_scale else ())
    return res if len(res) > 1 else out


def e8_nearest(y: np.ndarray):
    """Nearest E8 points of y [n, 8] (fp64): doubled coordinates [n, 8] int32 and cosets [n]."""
    y = np.ascontiguousarray(y, np.float64).reshape(-1, 8)
    q = np.zeros(y.shape, np.int32)
    b = np.zeros(len(y), np.int32)
    lib().or_e8_nearest_batch(_ptr(y), len(y), _ptr(q), _ptr(b))
    return q, b


def normalize(counts, prob_bits: int = 12) -> np.ndarray:
    c = np.zeros(256, np.uint64)
    c[: len(counts)] = counts
    f = np.zeros(256, np.uint32)
    rc = lib().or_normalize(_ptr(c), prob_bits, _ptr(f))
    if rc != 0:
        raise OracleError(rc, "normalize")
    return f


def choose_window(values) -> tuple[int, int, int]:
    """The oracle's window rule applied to a list of coordinate values: (window start, width,
    number of values outside the window)."""
    v = np.ascontiguousarray(np.asarray(values, np.int32))
    lo, S, ne = C.c_int32(), C.c_int32(), C.c_uint64()
    rc = lib().or_choose_window(_ptr(v), len(v), C.byref(lo), C.byref(S), C.byref(ne))
    if rc != 0:
        raise OracleError(rc, "choose_window")
    return lo.value, S.value, ne.value


def estimate_bpp(w: np.ndarray, delta: float, dtype: int | None = None) -> float:
    w = np.ascontiguousarray(w)
    return lib().or_estimate_bpp(_ptr(w), _dtype_code(w, dtype), w.shape[0], w.shape[1], delta)


def select_step(w: np.ndarray, target: float, dtype: int | None = None) -> float:
    w = np.ascontiguousarray(w)
    return lib().or_select_step(_ptr(w), _dtype_code(w, dtype), w.shape[0], w.shape[1], target)


def row_scale(w: np.ndarray, r: int, dtype: int | None = None) -> float:
    w = np.ascontiguousarray(w)
    return lib().or_row_scale(_ptr(w), _dtype_code(w, dtype), w.shape[0], w.shape[1], r)


def f32_to_bf16(v: float) -> int:
    return lib().or_f32_to_bf16(v)


def f32_to_f16(v: float) -> int:
    return lib().or_f32_to_f16(v)


def f32_to_e4m3(v: float) -> int:
    return lib().or_f32_to_e4m3(v)


def rans_encode(freqs: np.ndarray, prob_bits: int, tab: np.ndarray, sym: np.ndarray,
                esc: np.ndarray | None = None, esc_sym: int = -1) -> bytes:
    """Encode one tile: freqs [n_tables, 256]; tab/sym [n_steps, 32]; esc [n_steps, 32] words."""
    freqs = np.ascontiguousarray(freqs, np.uint32)
    tab = np.ascontiguousarray(tab, np.uint8)
    sym = np.ascontiguousarray(sym, np.uint8)
    n_steps = tab.shape[0]
    esc = np.ascontiguousarray(np.zeros_like(tab, np.uint16) if esc is None else esc, np.uint16)
    cap = 128 + 4 * 32 * n_steps + 4
    out = np.zeros(cap, np.uint8)
    n = C.c_size_t()
    rc = lib().or_rans_encode(freqs.shape[0], _ptr(freqs), prob_bits, n_steps, _ptr(tab), _ptr(sym), _ptr(esc),
                              esc_sym, _ptr(out), cap, C.byref(n))
    if rc != 0:
        raise OracleError(rc, "rans_encode")
    return out[: n.value].tobytes()


def rans_decode(freqs: np.ndarray, prob_bits: int, tab: np.ndarray, tile: bytes, esc_sym: int = -1):
    """Decode one tile; returns (rc, symbols [n_steps, 32], escape words, final states [32])."""
    freqs = np.ascontiguousarray(freqs, np.uint32)
    tab = np.ascontiguousarray(tab, np.uint8)
    sym = np.zeros(tab.shape, np.uint8)
    esc = np.zeros(tab.shape, np.uint16)
    fin = np.zeros(32, np.uint32)
    buf = np.frombuffer(tile, np.uint8).copy() if len(tile) else np.zeros(1, np.uint8)
    rc = lib().or_rans_decode(freqs.shape[0], _ptr(freqs), prob_bits, tab.shape[0], _ptr(tab), esc_sym,
                              _ptr(buf), len(tile), _ptr(sym), _ptr(esc), _ptr(fin))
    return rc, sym, esc, fin


def quantize_rows_e4m3(x_bf16: np.ndarray):
    """Per-row FP8 E4M3 codes [M, K] (uint8) and scales [M] (fp32) of BF16 activations given as
    uint16 bit patterns."""
    x = np.ascontiguousarray(x_bf16, np.uint16)
    M, K = x.shape
    q = np.zeros((M, K), np.uint8)
    s = np.zeros(max(M, 1), np.float32)
    rc = lib().or_quantize_rows_e4m3(_ptr(x), M, K, _ptr(q), _ptr(s))
    if rc != 0:
        raise OracleError(rc, "quantize_rows_e4m3")
    return q, s[:M]
