"""CPU checks of the C-ABI library: it loads, exports every declared symbol, and
rejects bad arguments on the host with the documented codes (no GPU involved:
validation runs before any HIP call)."""
import ctypes
import os
import re

import pytest

import gemm_q4_q5_amd as qg
from gemm_q4_q5_amd._lib import CWeight

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("qgemv_q4k", "qgemv_q5k", "qgemv_q6k", "qgemv_nvfp4", "qgemv_fp8", "qgemm_rows", "qgemv_add",
                 "qgemv_pair", "qgemv_triple", "qgemv_pair_swiglu", "qdequant", "qg_row_bytes",
                 "qg_tiles_bytes", "qg_pack_tiles",
                 "qg_status_str", "qg_last_error"):
        assert want in names


def test_library_exports_every_declared_symbol():
    L = qg.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_row_bytes():
    assert qg.row_bytes(qg.Q4_K, 2560) == 1440
    assert qg.row_bytes(qg.Q5_K, 9728) == 38 * 176
    assert qg.row_bytes(qg.Q6_K, 9728) == 38 * 210
    assert qg.row_bytes(qg.NVFP4, 8192) == 4096
    assert qg.row_bytes(qg.FP8, 2560) == 2560
    assert qg.row_bytes(qg.Q4_K, 100) == -1
    assert qg.row_bytes(99, 256) == -1


def test_status_strings():
    L = qg.lib()
    assert L.qg_status_str(0) == b"ok"
    assert L.qg_status_str(-5) == b"misaligned pointer"


FAKE = 0x10000  # 64 KiB: 16-byte aligned, never dereferenced (validation fails first)


def w(type_=12, data=FAKE, scales=None, m=8, k=512, layout=0):
    c = CWeight(type_, layout, data, scales, m, k)
    return ctypes.byref(c), c


@pytest.mark.parametrize("case,code", [
    (dict(data=None), -1),
    (dict(type_=7), -4),
    (dict(layout=2), -4),
    (dict(type_=1001, scales=FAKE, layout=1), -4),
    (dict(type_=1002, scales=FAKE, layout=1), -4),
    (dict(m=0), -2),
    (dict(k=300), -2),
    (dict(k=0), -2),
    (dict(data=FAKE + 4), -5),
    (dict(type_=1001, scales=None), -1),
    (dict(type_=1001, scales=FAKE + 8), -5),
    (dict(type_=1002, scales=None), -1),
    (dict(type_=1002, scales=FAKE + 8), -5),
    (dict(type_=1002, scales=FAKE, k=384), -2),
])
def test_rows_validation(case, code):
    L = qg.lib()
    ref, _keep = w(**case)
    assert L.qgemm_rows(ref, FAKE, FAKE, 1, None) == code
    assert L.qg_last_error() != b""


def test_rows_count_and_pointer_checks():
    L = qg.lib()
    ref, _k = w()
    assert L.qgemm_rows(ref, FAKE, FAKE, 0, None) == -3
    assert L.qgemm_rows(ref, FAKE, FAKE, 33, None) == -3
    assert L.qgemm_rows(ref, None, FAKE, 1, None) == -1
    assert L.qgemm_rows(ref, FAKE + 2, FAKE, 1, None) == -5
    assert L.qgemm_rows(ref, FAKE, FAKE + 2, 1, None) == -5
    assert L.qgemm_rows(None, FAKE, FAKE, 1, None) == -1


def test_gemv_single_validation():
    L = qg.lib()
    assert L.qgemv_q4k(None, FAKE, FAKE, 8, 512, None) == -1
    assert L.qgemv_q5k(FAKE, FAKE, FAKE, 8, 500, None) == -2
    assert L.qgemv_q6k(FAKE, FAKE, FAKE, 0, 512, None) == -2
    assert L.qgemv_nvfp4(FAKE, None, FAKE, FAKE, 8, 512, None) == -1
    # NVFP4 streams 256 weights per step: k a multiple of 16 but not of 256 is refused
    assert L.qgemv_nvfp4(FAKE, FAKE, FAKE, FAKE, 8, 272, None) == -2
    assert L.qgemv_nvfp4(FAKE, FAKE, FAKE, FAKE, 8, 16, None) == -2
    assert L.qgemv_fp8(FAKE, None, FAKE, FAKE, 8, 512, None) == -1
    assert L.qgemv_fp8(FAKE, FAKE, FAKE, FAKE, 8, 640, None) == -2
    assert L.qgemv_q4k(FAKE, FAKE + 8, FAKE, 8, 512, None) == -5


def test_fused_validation():
    L = qg.lib()
    a, _a = w(k=512)
    b, _b = w(k=768)
    c, _c = w(k=512)
    assert L.qgemv_pair(a, b, FAKE, FAKE, FAKE, 1, None) == -2
    assert L.qgemv_triple(a, c, b, FAKE, FAKE, FAKE, FAKE, 1, None) == -2
    assert L.qgemv_pair(a, c, FAKE, FAKE, None, 1, None) == -1
    assert L.qgemv_add(a, FAKE, None, FAKE, 1, None) == -1
    assert L.qgemv_add(a, FAKE, FAKE, FAKE, 40, None) == -3
    d, _d = w(m=16)
    assert L.qgemv_pair_swiglu(a, d, FAKE, FAKE, 1, None) == -2
    e, _e = w(type_=14)
    assert L.qgemv_pair_swiglu(a, e, FAKE, FAKE, 1, None) == -4
    assert L.qdequant(a, None, None) == -1


def _regions(ptrs, sizes):
    n = len(ptrs)
    return (ctypes.c_void_p * max(n, 1))(*ptrs), (ctypes.c_int64 * max(n, 1))(*sizes)


@pytest.mark.parametrize("ptrs,sizes,nreg,out,code", [
    ([FAKE], [64], 0, FAKE, -2),            # no region
    ([FAKE] * 4, [64] * 4, 4, FAKE, -2),    # more than three
    ([FAKE], [40], 1, FAKE, -2),            # not a multiple of 16 bytes
    ([FAKE], [0], 1, FAKE, -2),
    ([FAKE + 8], [64], 1, FAKE, -5),        # misaligned region
    ([FAKE], [64], 1, FAKE + 64, -5),       # out not 128-byte aligned
    ([0], [64], 1, FAKE, -1),
    ([FAKE], [64], 1, 0, -1),
])
def test_stream_read_validation(ptrs, sizes, nreg, out, code):
    L = qg.lib()
    p, b = _regions(ptrs, sizes)
    assert L.qg_stream_read(p, b, nreg, out, None) == code
    assert L.qg_last_error() != b""


def test_tiles_bytes_and_pack_validation():
    L = qg.lib()
    a, _a = w(type_=12, m=17, k=512)                  # 2 tiles of 16 rows, 288-byte rows
    assert L.qg_tiles_bytes(a) == 32 * 288
    b, _b = w(type_=14, m=2560, k=9728)
    assert L.qg_tiles_bytes(b) == 2560 * 38 * 210
    f, _f = w(type_=1001, scales=FAKE)
    assert L.qg_tiles_bytes(f) == -4
    assert L.qg_pack_tiles(a, None, None) == -1
    assert L.qg_pack_tiles(a, FAKE + 8, None) == -5
    t, _t = w(type_=12, m=17, k=512, layout=1)
    assert L.qg_pack_tiles(t, FAKE, None) == -4       # the source must be in the row layout
    assert L.qg_pack_tiles(f, FAKE, None) == -4
    g, _g = w(type_=12, m=8, k=512)
    u, _u = w(type_=12, m=8, k=512, layout=1)
    assert L.qgemv_pair_swiglu(g, u, FAKE, FAKE, 1, None) == -4   # gate and up in different layouts


def test_prefill_shape_limits():
    """n outside 1..2^30 and calls needing more than 2^31 - 1 blocks of Y are
    rejected before anything reaches the device."""
    L = qg.lib()
    ref, _k = w(m=8)
    assert L.qgemm_prefill(ref, FAKE, FAKE, 0, None) == -2
    assert L.qgemm_prefill(ref, FAKE, FAKE, (1 << 30) + 1, None) == -2
    big, _b = w(m=1 << 30)
    assert L.qgemm_prefill(big, FAKE, FAKE, 1 << 30, None) == -2
    assert b"blocks" in L.qg_last_error()
