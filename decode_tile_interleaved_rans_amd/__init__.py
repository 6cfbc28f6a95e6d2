"""MI355X (gfx950) tile-rANS weight codec: Python binding of ``libentropack.so``.

The functions mirror the C ABI in ``include/entropack.h`` and only marshal arguments: the host
encoder, the stream validator and every GPU step run in the compiled library. PyTorch provides
device memory and the current HIP stream. There is no fallback path: if the library is missing,
every call raises.

    stream, bpp = compress(weight, target_bpp=4.0)       # host encoder
    w_hat = decompress(stream, torch.bfloat16)           # GPU decode into a container
    layer = CompressedLinear.from_linear(linear, 4.0)    # fused decode + BF16 MFMA GEMM
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libentropack.so")

F32, BF16, F16, F8E4M3, I8, U8 = 0, 1, 2, 3, 4, 5
# Probability precision of the streams CompressedLinear.from_linear codes: with 2^11-slot tables
# (64 KiB in LDS instead of 96 KiB) the fused decode + MFMA forward runs 12 waves per CU instead of
# 8; the stream is about 1% larger and the plain decode runs at the same speed.
LAYER_PROB_BITS = 11
LOSSY, LOSSLESS, LOSSLESS_EXP = 0, 1, 2
# Lossy tile layouts (ep_encode_opts.layout): ROW_LAYOUT keeps each of a tile's 32 rANS states on
# one tile row, so that every block step of a 16-row tile pair yields a 16 x 32 weight block, the B
# operand of one BF16 MFMA, in the decoder's own registers.
BLOCK_ROW_LAYOUT, ROW_LAYOUT = 0, 1
# Tile layout of the streams CompressedLinear.from_linear codes: the row layout, whose forward for
# up to 64 activation rows multiplies the weight straight from the decoder's registers (at 8192 x
# 8192, 4.5 bpp: 80 us for M = 16 against 121 us in layout 0); a plain decode of it (the forward
# above 64 rows) takes about 10% longer.
LAYER_LAYOUT = ROW_LAYOUT
STATUS = {0: "EP_OK", -1: "EP_EINVAL", -2: "EP_ECORRUPT", -3: "EP_EUNSUPPORTED", -4: "EP_ERANGE",
          -5: "EP_EHIP", -6: "EP_ENOMEM", -7: "EP_EDEVICE"}
EXPORTS = ["ep_compress", "ep_free", "ep_stream_info", "ep_upload", "ep_handle_info", "ep_decompress",
           "ep_decompress_many", "ep_decode_symbols", "ep_linear_forward", "ep_gemm_bf16", "ep_handle_check",
           "ep_release", "ep_last_error", "ep_version", "ep_linear_forward_fp8", "ep_quantize_rows_fp8",
           "ep_gemm_fp8", "ep_compress_device", "ep_linear_forward_noalloc", "ep_linear_forward_many",
           "ep_linear_forward_fp8_many"]


class EPError(RuntimeError):
    def __init__(self, status: int, call: str, msg: str):
        super().__init__(f"{call}: {STATUS.get(status, status)}: {msg}")
        self.status = status


class EncodeOpts(C.Structure):
    _fields_ = [("mode", C.c_int), ("target_bpp", C.c_double), ("prob_bits", C.c_int), ("tile_rows", C.c_int),
                ("n_threads", C.c_int), ("layout", C.c_int)]


class Info(C.Structure):
    _fields_ = [("rows", C.c_int64), ("cols", C.c_int64), ("mode", C.c_int32), ("src_dtype", C.c_int32),
                ("tile_rows", C.c_int32), ("prob_bits", C.c_int32), ("n_tiles", C.c_uint32),
                ("n_escapes", C.c_uint32), ("step", C.c_float), ("target_bpp", C.c_float),
                ("actual_bpp", C.c_double), ("total_bytes", C.c_uint64), ("payload_bytes", C.c_uint64),
                ("state_bytes", C.c_uint64), ("meta_bytes", C.c_uint64), ("layout", C.c_int32)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}


_lib = None


def lib() -> C.CDLL:
    """Load the compiled library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m decode_tile_interleaved_rans_amd.build")
        L = C.CDLL(LIB_PATH)
        vp, i64, sz = C.c_void_p, C.c_int64, C.c_size_t
        L.ep_compress.argtypes = [vp, C.c_int, i64, i64, C.POINTER(EncodeOpts), C.POINTER(C.POINTER(C.c_uint8)),
                                  C.POINTER(sz), C.POINTER(C.c_double)]
        L.ep_compress_device.argtypes = [vp, C.c_int, i64, i64, C.POINTER(EncodeOpts), vp,
                                         C.POINTER(C.POINTER(C.c_uint8)), C.POINTER(sz), C.POINTER(C.c_double)]
        L.ep_free.argtypes = [vp]
        L.ep_free.restype = None
        L.ep_stream_info.argtypes = [C.c_char_p, sz, C.POINTER(Info)]
        L.ep_upload.argtypes = [C.c_char_p, sz, vp, C.POINTER(vp)]
        L.ep_handle_info.argtypes = [vp, C.POINTER(Info)]
        L.ep_decompress.argtypes = [vp, C.c_int, vp, vp, vp]
        L.ep_decompress_many.argtypes = [vp, vp, vp, vp, C.c_int, vp]
        L.ep_decode_symbols.argtypes = [vp, vp, vp]
        L.ep_linear_forward.argtypes = [vp, vp, i64, vp, vp, vp]
        L.ep_linear_forward_noalloc.argtypes = [vp, vp, i64, vp, vp, vp]
        L.ep_linear_forward_many.argtypes = [vp, C.c_int, vp, i64, vp, vp, vp]
        L.ep_linear_forward_fp8_many.argtypes = [vp, C.c_int, vp, i64, vp, vp, vp]
        L.ep_gemm_bf16.argtypes = [vp, vp, i64, i64, i64, vp, vp]
        L.ep_linear_forward_fp8.argtypes = [vp, vp, i64, vp, vp, vp]
        L.ep_quantize_rows_fp8.argtypes = [vp, i64, i64, vp, vp, vp]
        L.ep_gemm_fp8.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, vp]
        L.ep_handle_check.argtypes = [vp, vp]
        L.ep_release.argtypes = [vp]
        L.ep_release.restype = None
        L.ep_last_error.restype = C.c_char_p
        L.ep_version.restype = C.c_char_p
        for name in EXPORTS:
            if name not in ("ep_free", "ep_release", "ep_last_error", "ep_version"):
                getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def _check(rc: int, call: str):
    if rc != 0:
        raise EPError(rc, call, lib().ep_last_error().decode(errors="replace"))


def _torch():
    import torch
    return torch


_DT_OF_TORCH = None


def _dtype_code(t) -> int:
    torch = _torch()
    table = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16, torch.float8_e4m3fn: F8E4M3,
             torch.int8: I8, torch.uint8: U8}
    if t not in table:
        raise ValueError(f"unsupported dtype {t}")
    return table[t]


def _torch_dtype(code: int):
    torch = _torch()
    return {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16, F8E4M3: torch.float8_e4m3fn,
            I8: torch.int8, U8: torch.uint8}[code]


def _stream_ptr(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _run_on(stream):
    """(s, other) for a call that runs on `stream` (default: the current stream). With another
    stream, s first waits for the work queued on the current stream (which produced the inputs);
    the caller allocates its outputs under torch.cuda.stream(s) and, after the call, marks the
    input tensors as used on s (_used_on), so that the caching allocator does not hand their
    memory to other work while s may still read them."""
    torch = _torch()
    cur = torch.cuda.current_stream()
    s = stream if stream is not None else cur
    other = s.cuda_stream != cur.cuda_stream
    if other:
        s.wait_stream(cur)
    return s, other


def _used_on(s, other, *tensors):
    if other:
        for t in tensors:
            if t is not None:
                t.record_stream(s)


# ------------------------------------------------------------------------------------ host side
def compress(w, target_bpp: float = 4.0, *, mode: int = LOSSY, prob_bits: int = 12, tile_rows: int = 16,
             n_threads: int = 0, dtype: int | None = None, layout: int = 0) -> tuple[bytes, float]:
    """Compress a 2-D weight (torch tensor on any device, or numpy array) on the host.
    Returns (stream bytes, actual bits per weight including every byte of metadata).
    layout (lossy only; ep_encode_opts.layout): 0 codes each tile row by row, 1 keeps every rANS
    state on one tile row (ROW_LAYOUT), which the compressed linear forward multiplies straight
    from the decoder's registers; both decode to the same weights."""
    if hasattr(w, "detach"):
        torch = _torch()
        code = _dtype_code(w.dtype)
        t = w.detach().contiguous().cpu()
        view = t.view(torch.int16) if t.element_size() == 2 else (t.view(torch.uint8) if t.element_size() == 1 else t)
        arr = view.numpy()
    else:
        arr = np.ascontiguousarray(w)
        code = dtype if dtype is not None else {np.dtype(np.float32): F32, np.dtype(np.uint8): U8}.get(arr.dtype)
        if code is None:
            raise ValueError("numpy inputs other than float32/uint8 need dtype= (16-bit data as uint16 bits)")
    if arr.ndim != 2:
        raise ValueError("compress takes a 2-D [out_features, in_features] matrix")
    R, Cc = arr.shape
    opts = EncodeOpts(mode, float(target_bpp), prob_bits, tile_rows, n_threads, layout)
    out = C.POINTER(C.c_uint8)()
    n = C.c_size_t()
    bpp = C.c_double()
    _check(lib().ep_compress(arr.ctypes.data_as(C.c_void_p), code, R, Cc, C.byref(opts), C.byref(out), C.byref(n),
                             C.byref(bpp)), "ep_compress")
    data = C.string_at(out, n.value)
    lib().ep_free(out)
    return data, bpp.value


def compress_device(w, target_bpp: float = 4.0, *, prob_bits: int = 12, tile_rows: int = 16,
                    stream=None, layout: int = 0) -> tuple[bytes, float]:
    """Lossy compression on the GPU of a 2-D weight in device memory (torch tensor: float32,
    bfloat16 or float16); the same bytes as compress() on the same values."""
    if w.dim() != 2:
        raise ValueError("compress_device takes a 2-D [out_features, in_features] matrix")
    t = w.detach().contiguous()
    if not t.is_cuda:
        raise ValueError("compress_device takes a tensor in device memory")
    _need(t, "w", t.dtype)
    R, Cc = t.shape
    opts = EncodeOpts(LOSSY, float(target_bpp), prob_bits, tile_rows, 0, layout)
    out = C.POINTER(C.c_uint8)()
    n = C.c_size_t()
    bpp = C.c_double()
    _check(lib().ep_compress_device(C.c_void_p(t.data_ptr()), _dtype_code(t.dtype), R, Cc, C.byref(opts),
                                    _stream_ptr(stream), C.byref(out), C.byref(n), C.byref(bpp)), "ep_compress_device")
    data = C.string_at(out, n.value)
    lib().ep_free(out)
    return data, bpp.value


def lossless_compress(w, *, exponent_coded: bool = False, **kw) -> tuple[bytes, float]:
    """Bit-exact compression. exponent_coded=True (BF16 only) codes the exponent byte with the
    tile rANS and keeps sign and mantissa as uncoded bytes; otherwise every byte plane is coded."""
    return compress(w, 0.0, mode=LOSSLESS_EXP if exponent_coded else LOSSLESS, **kw)


def stream_info(stream: bytes) -> dict:
    info = Info()
    _check(lib().ep_stream_info(stream, len(stream), C.byref(info)), "ep_stream_info")
    return info.as_dict()


def save(path, stream: bytes, bias=None) -> None:
    """Write a stream (and an optional bias vector) to a file. The stream is the whole artifact:
    it is self-describing and versioned, and holds everything the decoder needs ("EntroPack
    PyTorch Guide", sections "Test saved artifacts" and "Diagnose the common failure cases").
    The file is a numpy .npz archive without pickled objects."""
    import numpy as np
    arrays = {"stream": np.frombuffer(stream, np.uint8)}
    if bias is not None:
        if isinstance(bias, np.ndarray):                 # BF16 bit patterns
            arrays["bias_bf16"] = np.asarray(bias, np.uint16)
        else:                                            # a torch tensor of any float dtype
            torch = _torch()
            b = bias.detach().to("cpu", torch.bfloat16).contiguous()
            arrays["bias_bf16"] = b.view(torch.int16).numpy().view(np.uint16)
    with open(path, "wb") as f:
        np.savez(f, **arrays)


def load(path):
    """Read a file written by save(): returns (stream bytes, bias bf16 bits as uint16 or None).
    The stream is validated before it is returned."""
    import numpy as np
    with np.load(path, allow_pickle=False) as z:
        stream = z["stream"].tobytes()
        bias = z["bias_bf16"].copy() if "bias_bf16" in z.files else None
    stream_info(stream)
    return stream, bias


def _need(t, name: str, dtype, shape=None, min_numel: int | None = None):
    """Argument check before a device pointer crosses the C ABI: the kernels trust sizes, so a
    tensor of the wrong shape, dtype, layout or device would be read or written out of bounds."""
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous tensor on the GPU")
    if t.device.index != _torch().cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, but the current device is cuda:{_torch().cuda.current_device()}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} needs at least {min_numel} elements")


# ------------------------------------------------------------------------------------ device side
class Handle:
    """A validated stream resident on the current GPU."""

    def __init__(self, stream: bytes, hip_stream=None):
        self._h = C.c_void_p()
        _check(lib().ep_upload(stream, len(stream), _stream_ptr(hip_stream), C.byref(self._h)), "ep_upload")
        info = Info()
        _check(lib().ep_handle_info(self._h, C.byref(info)), "ep_handle_info")
        self.info = info.as_dict()
        self.shape = (self.info["rows"], self.info["cols"])

    @property
    def ptr(self):
        return self._h

    def decompress_into(self, out, row_scale=None, stream=None):
        torch = _torch()
        code = _dtype_code(out.dtype) if out.dtype != torch.int16 else None
        if code is None:
            raise ValueError("use decode_symbols_into for int16 outputs")
        if tuple(out.shape) != self.shape or not out.is_contiguous() or not out.is_cuda:
            raise ValueError(f"output must be a contiguous CUDA tensor of shape {self.shape}")
        if row_scale is not None:
            _need(row_scale, "row_scale", torch.float32, min_numel=self.shape[0])
        sp = C.c_void_p(row_scale.data_ptr()) if row_scale is not None else None
        _check(lib().ep_decompress(self._h, code, C.c_void_p(out.data_ptr()), sp, _stream_ptr(stream)),
               "ep_decompress")
        return out

    def decompress(self, dtype=None, stream=None):
        """Decode into a new tensor. FP8 / INT8 return (values, per-row fp32 scale). The outputs
        are allocated on the stream the decode runs on."""
        torch = _torch()
        if dtype is None:
            dtype = _torch_dtype(self.info["src_dtype"]) if self.info["mode"] != LOSSY else torch.bfloat16
        s = stream if stream is not None else torch.cuda.current_stream()
        with torch.cuda.stream(s):
            out = torch.empty(self.shape, dtype=dtype, device="cuda")
            scale = None
            if self.info["mode"] == LOSSY and dtype in (torch.float8_e4m3fn, torch.int8):
                scale = torch.empty(self.shape[0], dtype=torch.float32, device="cuda")
            self.decompress_into(out, scale, s)
        return (out, scale) if scale is not None else out

    def decode_symbols(self, stream=None):
        """Decode the lattice symbols into a new int16 tensor, allocated on the stream the decode
        runs on."""
        torch = _torch()
        s = stream if stream is not None else torch.cuda.current_stream()
        with torch.cuda.stream(s):
            q = torch.empty(self.shape, dtype=torch.int16, device="cuda")
        _check(lib().ep_decode_symbols(self._h, C.c_void_p(q.data_ptr()), C.c_void_p(s.cuda_stream)),
               "ep_decode_symbols")
        return q

    def check(self, stream=None):
        _check(lib().ep_handle_check(self._h, _stream_ptr(stream)), "ep_handle_check")

    def release(self):
        if self._h:
            lib().ep_release(self._h)
            self._h = C.c_void_p()

    def __del__(self):
        try:
            self.release()
        except Exception:
            pass


def upload(stream: bytes, hip_stream=None) -> Handle:
    return Handle(stream, hip_stream)


def decompress(stream: bytes, dtype=None, device: str = "cuda"):
    """Decode a stream on the GPU ("decompress(stream) returns a tensor")."""
    h = Handle(stream)
    try:
        return h.decompress(dtype)
    finally:
        _torch().cuda.current_stream().synchronize()
        h.release()


def decompress_many(handles, outs, scales=None, stream=None):
    """One grouped call over several uploaded matrices."""
    torch = _torch()
    n = len(handles)
    if len(outs) != n or (scales is not None and len(scales) != n):
        raise ValueError("handles, outs and scales must have the same length")
    for i, (h, o) in enumerate(zip(handles, outs)):
        _need(o, f"outs[{i}]", o.dtype, shape=h.shape)
        if scales is not None and scales[i] is not None:
            _need(scales[i], f"scales[{i}]", torch.float32, min_numel=h.shape[0])
    hs = (C.c_void_p * n)(*[h.ptr.value for h in handles])
    cts = (C.c_int * n)(*[_dtype_code(o.dtype) for o in outs])
    os_ = (C.c_void_p * n)(*[o.data_ptr() for o in outs])
    sc = (C.c_void_p * n)(*[(s.data_ptr() if s is not None else None) for s in (scales or [None] * n)])
    _check(lib().ep_decompress_many(hs, cts, os_, sc, n, _stream_ptr(stream)), "ep_decompress_many")


def gemm_bf16(x, w, stream=None):
    """Y = X W^T in BF16 with fp32 accumulation (the library's own MFMA GEMM), on `stream`
    (default: the current stream; another stream first waits for the current one)."""
    torch = _torch()
    M, K = x.shape
    N = w.shape[0]
    _need(x, "x", torch.bfloat16)
    _need(w, "w", torch.bfloat16, shape=(N, K))
    s, other = _run_on(stream)
    with torch.cuda.stream(s):
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(lib().ep_gemm_bf16(C.c_void_p(x.data_ptr()), C.c_void_p(w.data_ptr()), M, N, K, C.c_void_p(y.data_ptr()),
                              C.c_void_p(s.cuda_stream)), "ep_gemm_bf16")
    _used_on(s, other, x, w)
    return y


def quantize_rows_fp8(x, stream=None):
    """Per-row FP8 E4M3 codes of BF16 rows and their fp32 scales (x = codes * scale[row]), on
    `stream` (default: the current stream; another stream first waits for the current one)."""
    torch = _torch()
    M, K = x.shape
    _need(x, "x", torch.bfloat16)
    s, other = _run_on(stream)
    with torch.cuda.stream(s):
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        sc = torch.empty(M, dtype=torch.float32, device=x.device)
    _check(lib().ep_quantize_rows_fp8(C.c_void_p(x.data_ptr()), M, K, C.c_void_p(q.data_ptr()),
                                      C.c_void_p(sc.data_ptr()), C.c_void_p(s.cuda_stream)), "ep_quantize_rows_fp8")
    _used_on(s, other, x)
    return q, sc


def gemm_fp8(xq, xs, wq, ws, bias=None, stream=None):
    """Y = diag(xs) Xq Wq^T diag(ws) (+ bias) from E4M3 codes (uint8 tensors), BF16 output, on
    `stream` (default: the current stream; another stream first waits for the current one)."""
    torch = _torch()
    M, K = xq.shape
    N = wq.shape[0]
    _need(xq, "xq", torch.uint8)
    _need(wq, "wq", torch.uint8, shape=(N, K))
    _need(xs, "xs", torch.float32, shape=(M,))
    _need(ws, "ws", torch.float32, shape=(N,))
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, shape=(N,))
    s, other = _run_on(stream)
    with torch.cuda.stream(s):
        y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    bp = C.c_void_p(bias.data_ptr()) if bias is not None else None
    _check(lib().ep_gemm_fp8(C.c_void_p(xq.data_ptr()), C.c_void_p(xs.data_ptr()), C.c_void_p(wq.data_ptr()),
                             C.c_void_p(ws.data_ptr()), M, N, K, bp, C.c_void_p(y.data_ptr()), C.c_void_p(s.cuda_stream)),
           "ep_gemm_fp8")
    _used_on(s, other, xq, xs, wq, ws, bias)
    return y


class CompressedLinear:
    """Linear layer that keeps only the compressed weight and decodes it on every forward
    ("EntroPack PyTorch Guide", section "Replace one linear layer before a whole model").

    compute="bf16" (default): for up to 64 activation rows of a row-layout stream (the layout
    from_linear codes) one kernel decodes every tile pair straight into the B operand of the BF16
    MFMA and the weight is never written; a layout-0 stream is fused that way through LDS for 5 to
    16 rows and by the decode kernel's own products for up to 4. For more rows the weight is decoded
    once per call into scratch slices that stay in the Infinity Cache, and a BF16 MFMA GEMM reads
    them from there (hipBLASLt's from 512 rows, above 64 when in_features <= 4096, from 256 when
    out_features <= 4096; else the library's own).
    compute="fp8": the weight is decoded to FP8 E4M3 with its row scales and the activations are
    quantized per row; the codes meet in the FP8 MFMA, fused in the same cases, else on slices.

    The forward takes BF16 activations. Other dtypes are refused unless cast=True is passed, so a
    precision change is never silent ("Diagnose compression failures in the correct order")."""

    def __init__(self, stream: bytes, bias=None, compute: str = "bf16"):
        if compute not in ("bf16", "fp8"):
            raise ValueError("compute must be 'bf16' or 'fp8'")
        self.stream = stream
        self.handle = Handle(stream)
        self.out_features, self.in_features = self.handle.shape
        self.bias = bias
        self.compute = compute

    @classmethod
    def from_linear(cls, linear, target_bpp: float = 4.0, compute: str = "bf16", **kw):
        """Compress an nn.Linear's weight (probability precision LAYER_PROB_BITS and tile layout
        LAYER_LAYOUT unless prob_bits= / layout= are given) and keep its bias in BF16 on the GPU."""
        kw.setdefault("prob_bits", LAYER_PROB_BITS)
        kw.setdefault("layout", LAYER_LAYOUT)
        s, _ = compress(linear.weight, target_bpp, **kw)
        bias = None
        if linear.bias is not None:
            bias = linear.bias.detach().to(device="cuda", dtype=_torch().bfloat16).contiguous()
        return cls(s, bias, compute)

    @property
    def actual_bpp(self) -> float:
        return self.handle.info["actual_bpp"]

    def save(self, path) -> None:
        """Write the compressed weight and the bias to a file (see save())."""
        save(path, self.stream, self.bias)

    @classmethod
    def load(cls, path, compute: str = "bf16"):
        """Rebuild a layer from a file written by save(); the bias goes to the current GPU. The
        compute mode is a choice of the forward, not part of the artifact."""
        stream, bias = load(path)
        b = None
        if bias is not None:
            torch = _torch()
            b = torch.from_numpy(bias.view("int16")).view(torch.bfloat16).cuda()
        return cls(stream, b, compute)

    def forward(self, x, stream=None, cast: bool = False):
        """Y = X W^T (+ bias) in BF16 on `stream` (default: the current stream). x must be BF16,
        or cast=True to convert it first. With an explicit stream other than the current one, that
        stream first waits for the work queued on the current stream (which produced x), and the
        conversion and the output allocation run on it."""
        torch = _torch()
        shp = x.shape
        if shp[-1] != self.in_features or not x.is_cuda:
            raise ValueError(f"input must be a GPU tensor with last dimension {self.in_features}, got {tuple(shp)}")
        if x.dtype != torch.bfloat16 and not cast:
            raise ValueError(f"the forward takes bfloat16 activations, got {x.dtype}; pass cast=True to convert")
        if x.device.index != torch.cuda.current_device():
            raise ValueError(f"x is on {x.device}, but the current device is cuda:{torch.cuda.current_device()}")
        if self.bias is not None:
            _need(self.bias, "bias", torch.bfloat16, shape=(self.out_features,))
        s, other = _run_on(stream)
        with torch.cuda.stream(s):
            rows = int(np.prod(shp[:-1], dtype=np.int64))
            x2 = x.reshape(rows, shp[-1]).to(torch.bfloat16).contiguous()
            y = torch.empty((x2.shape[0], self.out_features), dtype=torch.bfloat16, device=x.device)
            bp = C.c_void_p(self.bias.data_ptr()) if self.bias is not None else None
            fn = lib().ep_linear_forward_fp8 if self.compute == "fp8" else lib().ep_linear_forward
            _check(fn(self.handle.ptr, C.c_void_p(x2.data_ptr()), x2.shape[0], bp, C.c_void_p(y.data_ptr()),
                      C.c_void_p(s.cuda_stream)), "ep_linear_forward" + ("_fp8" if self.compute == "fp8" else ""))
        _used_on(s, other, x2, self.bias)   # x (or its converted copy) is read on s after this returns
        return y.reshape(*shp[:-1], self.out_features)

    __call__ = forward


def linear_forward_many(layers, x, stream=None):
    """[layer(x) for layer in layers] for CompressedLinear layers of one compute mode that take the
    same input x (BF16, [..., in_features] on the GPU), each output the same bits as the layer's own
    forward. Up to 64 activation rows of row-layout layers with one prob_bits decode in one fused
    launch (ep_linear_forward_many, ep_linear_forward_fp8_many), so that small layers share the
    GPU's rounds of tile pairs; above 64 rows BF16 layers can share one slice decode; other cases
    run the layers one by one."""
    torch = _torch()
    layers = list(layers)
    if not layers:
        return []
    fp8 = layers[0].compute == "fp8"
    if len(layers) > 32 or any(l.compute != layers[0].compute for l in layers):
        return [l(x, stream=stream) for l in layers]
    K = layers[0].in_features
    shp = x.shape
    if any(l.in_features != K for l in layers) or shp[-1] != K or not x.is_cuda:
        raise ValueError("the layers must share in_features, and x must be a GPU tensor of that last dimension")
    if x.dtype != torch.bfloat16:
        raise ValueError(f"the forward takes bfloat16 activations, got {x.dtype}")
    if x.device.index != torch.cuda.current_device():
        raise ValueError(f"x is on {x.device}, but the current device is cuda:{torch.cuda.current_device()}")
    for l in layers:
        if l.bias is not None:
            _need(l.bias, "bias", torch.bfloat16, shape=(l.out_features,))
    s, other = _run_on(stream)
    with torch.cuda.stream(s):
        rows = int(np.prod(shp[:-1], dtype=np.int64))
        x2 = x.reshape(rows, K).contiguous()
        ys = [torch.empty((rows, l.out_features), dtype=torch.bfloat16, device=x.device) for l in layers]
        n = len(layers)
        hs = (C.c_void_p * n)(*[l.handle.ptr.value for l in layers])
        bs = (C.c_void_p * n)(*[(l.bias.data_ptr() if l.bias is not None else None) for l in layers])
        os_ = (C.c_void_p * n)(*[y.data_ptr() for y in ys])
        fn = lib().ep_linear_forward_fp8_many if fp8 else lib().ep_linear_forward_many
        _check(fn(hs, n, C.c_void_p(x2.data_ptr()), rows, bs, os_, C.c_void_p(s.cuda_stream)),
               "ep_linear_forward_fp8_many" if fp8 else "ep_linear_forward_many")
    _used_on(s, other, x2, *[l.bias for l in layers])
    return [y.reshape(*shp[:-1], l.out_features) for y, l in zip(ys, layers)]
