"""ctypes binding of libqgemm.so with the C ABI's names (include/qgemm.h).

Argument marshalling only: tensors supply device pointers, torch's current HIP
stream supplies the stream, and every step of the product runs in the library's
kernels.  Output tensors are allocated with torch when the caller passes none.
The library must be built (gemm_q4_q5_amd.build); there is no other code path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqgemm.so")

Q4_K, Q5_K, Q6_K, NVFP4, FP8 = 12, 13, 14, 1001, 1002
LAYOUT_ROWS, LAYOUT_TILES = 0, 1
MAX_ROWS = 32
STATUS = {0: "QG_OK", -1: "QG_ERR_NULL", -2: "QG_ERR_SHAPE", -3: "QG_ERR_ROWS",
          -4: "QG_ERR_TYPE", -5: "QG_ERR_ALIGN", -6: "QG_ERR_LAUNCH"}


class QGError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class CWeight(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("data", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("m", ctypes.c_int64), ("k", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqgemm.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m gemm_q4_q5_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32, fp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        W = ctypes.POINTER(CWeight)
        sig = {
            "qg_row_bytes": ([i32, i64], i64),
            "qg_tiles_bytes": ([W], i64),
            "qg_pack_tiles": ([W, p, p], ctypes.c_int),
            "qg_status_str": ([ctypes.c_int], ctypes.c_char_p),
            "qg_last_error": ([], ctypes.c_char_p),
            "qgemv_q4k": ([p, p, fp, i64, i64, p], ctypes.c_int),
            "qgemv_q5k": ([p, p, fp, i64, i64, p], ctypes.c_int),
            "qgemv_q6k": ([p, p, fp, i64, i64, p], ctypes.c_int),
            "qgemv_nvfp4": ([p, p, p, fp, i64, i64, p], ctypes.c_int),
            "qgemv_fp8": ([p, p, p, fp, i64, i64, p], ctypes.c_int),
            "qgemm_rows": ([W, p, fp, i32, p], ctypes.c_int),
            "qgemv_add": ([W, p, fp, fp, i32, p], ctypes.c_int),
            "qgemv_pair": ([W, W, p, fp, fp, i32, p], ctypes.c_int),
            "qgemv_triple": ([W, W, W, p, fp, fp, fp, i32, p], ctypes.c_int),
            "qgemv_pair_swiglu": ([W, W, p, fp, i32, p], ctypes.c_int),
            "qgemm_prefill": ([W, p, fp, i64, p], ctypes.c_int),
            "qdequant": ([W, fp, p], ctypes.c_int),
            "qg_stream_read": ([ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_int64), i32, p, p],
                               ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != 0:
        raise QGError(rc, lib().qg_last_error().decode())


def row_bytes(wtype: int, k: int) -> int:
    return lib().qg_row_bytes(wtype, k)


@dataclass
class QWeight:
    """A quantized weight resident in device memory (raw bytes as stored)."""
    type: int
    data: "object"                 # torch.uint8 tensor [m, row_bytes]
    m: int
    k: int
    scales: Optional[object] = None  # NVFP4 e4m3 bytes [m, k/16]; FP8 bf16 [ceil(m/128), k/128]
    layout: int = 0                    # LAYOUT_ROWS, or LAYOUT_TILES (see pack_tiles)

    def c(self) -> CWeight:
        return CWeight(self.type, self.layout, self.data.data_ptr(),
                       self.scales.data_ptr() if self.scales is not None else None, self.m, self.k)

    @classmethod
    def from_host(cls, wtype: int, data, m: int, k: int, scales=None, device="cuda"):
        import torch
        d = torch.from_numpy(data).to(device)
        s = torch.from_numpy(scales).to(device) if scales is not None else None
        return cls(wtype, d, m, k, s)


def pack_tiles(w: QWeight) -> QWeight:
    """The 16-row tiled copy of a row-layout K-quant weight (same values, same bits of
    every product); a new device buffer of qg_tiles_bytes bytes."""
    import torch
    _check_weight(w)
    _devices(*_wt(w))
    cw = w.c()
    nbytes = lib().qg_tiles_bytes(ctypes.byref(cw))
    if nbytes < 0:
        _check(int(nbytes))
    dst = torch.empty((int(nbytes),), dtype=torch.uint8, device=w.data.device)
    _check(lib().qg_pack_tiles(ctypes.byref(cw), _ptr(dst), _stream()))
    return QWeight(w.type, dst, w.m, w.k, None, LAYOUT_TILES)


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# Argument checks.  The C ABI sees bare pointers and cannot know how large a buffer
# is, so a tensor of the wrong size, dtype, layout or device would become an
# out-of-bounds access inside a kernel; every wrapper checks its tensors against
# (m, k, n) here and raises QGError before anything reaches the library.
_ERR_SHAPE, _ERR_TYPE = -2, -4


def _fail(code, msg):
    raise QGError(code, msg)


def _dense(t, what, dtype, numel=None, shape=None):
    """t: a contiguous tensor of `dtype` with `numel` elements (or `shape`); where it
    lives is checked last, by _devices."""
    import torch
    if not isinstance(t, torch.Tensor):
        _fail(_ERR_TYPE, f"{what} must be a torch tensor")
    if t.dtype != dtype:
        _fail(_ERR_TYPE, f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        _fail(_ERR_SHAPE, f"{what} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        _fail(_ERR_SHAPE, f"{what} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        _fail(_ERR_SHAPE, f"{what} has {t.numel()} elements, expected {numel}")


def _weight_bytes(w: "QWeight"):
    """(data bytes, scales bytes) the library reads for weight w."""
    k, m = w.k, w.m
    if w.type == NVFP4:
        return m * (k // 2), m * (k // 16)
    if w.type == FP8:
        return m * k, 2 * ((m + 127) // 128) * (k // 128)
    rb = {Q4_K: 144, Q5_K: 176, Q6_K: 210}.get(w.type)
    if rb is None:
        _fail(_ERR_TYPE, f"unknown weight type {w.type}")
    rows = (m + 15) // 16 * 16 if w.layout == LAYOUT_TILES else m
    return rows * (k // 256) * rb, 0


def _check_weight(w: "QWeight", what="w"):
    import torch
    if w.m < 1 or w.k < 256 or w.k % 256:
        _fail(_ERR_SHAPE, f"{what}: m = {w.m}, k = {w.k} (k must be a positive multiple of 256)")
    nd, ns = _weight_bytes(w)
    _dense(w.data, f"{what}.data", torch.uint8)
    if w.data.numel() != nd:
        _fail(_ERR_SHAPE, f"{what}.data holds {w.data.numel()} bytes, type {w.type} {w.m}x{w.k} needs {nd}")
    if ns:
        if w.scales is None:
            _fail(_ERR_SHAPE, f"{what}: type {w.type} needs scales")
        _dense(w.scales, f"{what}.scales", torch.uint8)
        if w.scales.numel() != ns:
            _fail(_ERR_SHAPE, f"{what}.scales holds {w.scales.numel()} bytes, needs {ns}")


def _check_x(x, k, n_max=MAX_ROWS):
    """x: fp16 [k] or [n, k] on the GPU; returns n."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dim() not in (1, 2):
        _fail(_ERR_SHAPE, "x must be a 1-D [k] or 2-D [n, k] tensor")
    n = 1 if x.dim() == 1 else x.shape[0]
    if x.shape[-1] != k:
        _fail(_ERR_SHAPE, f"x has {x.shape[-1]} columns, the weight has k = {k}")
    if n < 1 or (n_max is not None and n > n_max):
        _fail(-3, f"x has {n} rows, need 1..{n_max}")
    _dense(x, "x", torch.float16)
    return n


def _devices(*ts):
    """Every tensor of the call on one GPU (checked after the shapes and dtypes)."""
    ts = [t for t in ts if t is not None]
    for t in ts:
        if not getattr(t, "is_cuda", False):
            _fail(_ERR_TYPE, "every tensor of a call must be a GPU tensor")
    if len({t.device for t in ts}) > 1:
        _fail(_ERR_TYPE, f"tensors on different devices: {sorted({str(t.device) for t in ts})}")


def _wt(w):
    return (w.data, w.scales)


def _out(shape, like, out, what="y"):
    import torch
    if out is not None:
        numel = 1
        for d in shape:
            numel *= d
        _dense(out, what, torch.float32, numel=numel)
        return out
    return torch.empty(shape, dtype=torch.float32, device=like.device)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _rows(x) -> int:
    return 1 if x.dim() == 1 else x.shape[0]


def _single(w: QWeight, x, y, wtype):
    """Checks of a single-token entry point; returns y."""
    if w.type != wtype:
        _fail(_ERR_TYPE, f"weight type {w.type}, this entry point takes {wtype}")
    _check_weight(w)
    if _check_x(x, w.k) != 1:
        _fail(-3, "the single-token entry points take one row of x")
    y = _out((w.m,), x, y)
    _devices(*_wt(w), x, y)
    return y


def qgemv_q4k(w: QWeight, x, y=None):
    _row_layout(w)
    y = _single(w, x, y, Q4_K)
    _check(lib().qgemv_q4k(_ptr(w.data), _ptr(x), _ptr(y), w.m, w.k, _stream()))
    return y


def qgemv_q5k(w: QWeight, x, y=None):
    _row_layout(w)
    y = _single(w, x, y, Q5_K)
    _check(lib().qgemv_q5k(_ptr(w.data), _ptr(x), _ptr(y), w.m, w.k, _stream()))
    return y


def qgemv_q6k(w: QWeight, x, y=None):
    _row_layout(w)
    y = _single(w, x, y, Q6_K)
    _check(lib().qgemv_q6k(_ptr(w.data), _ptr(x), _ptr(y), w.m, w.k, _stream()))
    return y


def qgemv_nvfp4(w: QWeight, x, y=None):
    y = _single(w, x, y, NVFP4)
    _check(lib().qgemv_nvfp4(_ptr(w.data), _ptr(w.scales), _ptr(x), _ptr(y), w.m, w.k, _stream()))
    return y


def qgemv_fp8(w: QWeight, x, y=None):
    y = _single(w, x, y, FP8)
    _check(lib().qgemv_fp8(_ptr(w.data), _ptr(w.scales), _ptr(x), _ptr(y), w.m, w.k, _stream()))
    return y


def _row_layout(w: QWeight) -> None:
    if w.layout != LAYOUT_ROWS:
        raise QGError(-4, "the single-token entry points take the row layout; use qgemm_rows")


def qgemv(w: QWeight, x, y=None):
    """The single-token GEMV entry point of w's type (qgemm_rows with one row for a
    tiled weight: the same kernel and bits)."""
    if w.layout != LAYOUT_ROWS:
        return qgemm_rows(w, x.reshape(1, -1), None if y is None else y.reshape(1, -1)).reshape(-1)
    f = {Q4_K: qgemv_q4k, Q5_K: qgemv_q5k, Q6_K: qgemv_q6k, NVFP4: qgemv_nvfp4, FP8: qgemv_fp8}[w.type]
    return f(w, x, y)


def qgemm_rows(w: QWeight, x, y=None):
    _check_weight(w)
    n = _check_x(x, w.k)
    y = _out((n, w.m), x, y)
    _devices(*_wt(w), x, y)
    cw = w.c()
    _check(lib().qgemm_rows(ctypes.byref(cw), _ptr(x), _ptr(y), n, _stream()))
    return y


def qgemv_add(w: QWeight, x, resid, y=None):
    import torch
    _check_weight(w)
    n = _check_x(x, w.k)
    _dense(resid, "resid", torch.float32, numel=n * w.m)
    y = _out((n, w.m), x, y)
    _devices(*_wt(w), x, resid, y)
    cw = w.c()
    _check(lib().qgemv_add(ctypes.byref(cw), _ptr(x), _ptr(resid), _ptr(y), n, _stream()))
    return y


def qgemv_pair(w0: QWeight, w1: QWeight, x, y0=None, y1=None):
    _check_weight(w0, "w0")
    _check_weight(w1, "w1")
    n = _check_x(x, w0.k)
    if w1.k != w0.k:
        _fail(_ERR_SHAPE, f"pair: k differs ({w0.k} vs {w1.k})")
    y0 = _out((n, w0.m), x, y0, "y0")
    y1 = _out((n, w1.m), x, y1, "y1")
    _devices(*_wt(w0), *_wt(w1), x, y0, y1)
    c0, c1 = w0.c(), w1.c()
    _check(lib().qgemv_pair(ctypes.byref(c0), ctypes.byref(c1), _ptr(x), _ptr(y0), _ptr(y1), n, _stream()))
    return y0, y1


def qgemv_triple(w0: QWeight, w1: QWeight, w2: QWeight, x, y0=None, y1=None, y2=None):
    for i, w in enumerate((w0, w1, w2)):
        _check_weight(w, f"w{i}")
    n = _check_x(x, w0.k)
    if not (w0.k == w1.k == w2.k):
        _fail(_ERR_SHAPE, "triple: k differs between the weights")
    y0 = _out((n, w0.m), x, y0, "y0")
    y1 = _out((n, w1.m), x, y1, "y1")
    y2 = _out((n, w2.m), x, y2, "y2")
    _devices(*_wt(w0), *_wt(w1), *_wt(w2), x, y0, y1, y2)
    c0, c1, c2 = w0.c(), w1.c(), w2.c()
    _check(lib().qgemv_triple(ctypes.byref(c0), ctypes.byref(c1), ctypes.byref(c2), _ptr(x),
                              _ptr(y0), _ptr(y1), _ptr(y2), n, _stream()))
    return y0, y1, y2


def qgemv_pair_swiglu(wg: QWeight, wu: QWeight, x, h=None):
    _check_weight(wg, "wg")
    _check_weight(wu, "wu")
    n = _check_x(x, wg.k)
    if (wu.m, wu.k) != (wg.m, wg.k):
        _fail(_ERR_SHAPE, "swiglu pair: gate and up must have the same m and k")
    h = _out((n, wg.m), x, h, "h")
    _devices(*_wt(wg), *_wt(wu), x, h)
    cg, cu = wg.c(), wu.c()
    _check(lib().qgemv_pair_swiglu(ctypes.byref(cg), ctypes.byref(cu), _ptr(x), _ptr(h), n, _stream()))
    return h


def qgemm_prefill(w: QWeight, x, y=None):
    """MFMA prefill GEMM: y[n, m] = x[n, k] . W^T for any n >= 1."""
    _check_weight(w)
    n = _check_x(x, w.k, n_max=None)
    y = _out((n, w.m), x, y)
    _devices(*_wt(w), x, y)
    cw = w.c()
    _check(lib().qgemm_prefill(ctypes.byref(cw), _ptr(x), _ptr(y), n, _stream()))
    return y


def qdequant(w: QWeight, out=None):
    _check_weight(w)
    out = _out((w.m, w.k), w.data, out, "out")
    _devices(*_wt(w), out)
    cw = w.c()
    _check(lib().qdequant(ctypes.byref(cw), _ptr(out), _stream()))
    return out


READ_PROBE_WORDS = 2048


def qg_stream_read(regions, out):
    """Read-stream probe: XOR every 32-bit word of the device tensors `regions`
    (one to three, each 16-byte aligned, a multiple of 16 bytes) into the int32
    device tensor `out` (READ_PROBE_WORDS elements, updated in place: the XOR of
    its words changes by the XOR of all words read)."""
    import torch
    _dense(out, "out", torch.int32, numel=READ_PROBE_WORDS)
    for i, t in enumerate(regions):
        if not t.is_contiguous():
            _fail(_ERR_SHAPE, f"region {i} must be contiguous")
    _devices(out, *regions)
    n = len(regions)
    ptrs = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in regions])
    nbytes = (ctypes.c_int64 * max(n, 1))(*[t.numel() * t.element_size() for t in regions])
    _check(lib().qg_stream_read(ptrs, nbytes, n, _ptr(out), _stream()))
    return out
