"""The Python binding refuses mis-shaped, mistyped or misplaced tensors before any
pointer reaches the library (the C ABI cannot see buffer sizes, so a wrong size
would otherwise become an out-of-bounds access in a kernel).  CPU only: the library
entry is replaced by a trap, so a check that let a bad call through fails here."""
import numpy as np
import pytest
import torch

import gemm_q4_q5_amd as qg
from gemm_q4_q5_amd import _lib


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def trap():
        raise AssertionError("a bad call reached the library")
    monkeypatch.setattr(_lib, "lib", trap)


def _w(wtype=qg.Q4_K, m=32, k=512, layout=qg.LAYOUT_ROWS, extra=0, scales_extra=0):
    nd, ns = _lib._weight_bytes(qg.QWeight(wtype, None, m, k, None, layout))
    data = torch.zeros(nd + extra, dtype=torch.uint8)
    sc = torch.zeros(ns + scales_extra, dtype=torch.uint8) if ns else None
    return qg.QWeight(wtype, data, m, k, sc, layout)


def _x(n=1, k=512, dtype=torch.float16):
    return torch.zeros((n, k), dtype=dtype)


def _raises(code, fn, *a):
    with pytest.raises(qg.QGError) as e:
        fn(*a)
    assert e.value.code == code, str(e.value)
    return str(e.value)


def test_well_formed_cpu_call_is_refused_for_its_device():
    msg = _raises(-4, qg.qgemm_rows, _w(), _x(3))
    assert "GPU" in msg


def test_x_checks():
    _raises(-4, qg.qgemm_rows, _w(), _x(2, dtype=torch.float32))     # dtype
    _raises(-2, qg.qgemm_rows, _w(), _x(2, k=256))                   # k
    _raises(-2, qg.qgemm_rows, _w(), _x(2, k=1024)[:, ::2])          # not contiguous
    _raises(-3, qg.qgemm_rows, _w(), _x(33))                         # too many rows
    _raises(-3, qg.qgemv_q4k, _w(), _x(2))                           # GEMV takes one row
    _raises(-2, qg.qgemm_rows, _w(), torch.zeros((1, 1, 512), dtype=torch.float16))


def test_weight_size_checks():
    _raises(-2, qg.qgemm_rows, _w(extra=-1), _x())
    _raises(-2, qg.qgemm_rows, _w(extra=144), _x())
    # the tiled layout rounds m up to whole 16-row tiles
    w = _w(m=20, layout=qg.LAYOUT_TILES)
    assert w.data.numel() == 32 * 2 * 144
    _raises(-2, qg.qgemm_rows, qg.QWeight(qg.Q4_K, torch.zeros(20 * 2 * 144, dtype=torch.uint8), 20, 512,
                                          None, qg.LAYOUT_TILES), _x())
    _raises(-2, qg.qgemm_rows, _w(k=300), _x(k=300))
    _raises(-4, qg.qgemm_rows, qg.QWeight(qg.Q4_K, torch.zeros(32 * 288, dtype=torch.int8), 32, 512), _x())
    _raises(-4, qg.qgemm_rows, qg.QWeight(77, torch.zeros(10, dtype=torch.uint8), 32, 512), _x())


def test_scale_checks():
    _raises(-2, qg.qgemm_rows, _w(qg.NVFP4, scales_extra=-1), _x())
    _raises(-2, qg.qgemm_rows, _w(qg.FP8, m=130, scales_extra=2), _x())
    w = _w(qg.NVFP4)
    _raises(-2, qg.qgemm_rows, qg.QWeight(qg.NVFP4, w.data, w.m, w.k, None), _x())
    # FP8: two row blocks of scales for 130 rows, k/128 bf16 each
    assert _w(qg.FP8, m=130, k=512).scales.numel() == 2 * 2 * 4


def test_output_checks():
    w = _w()
    _raises(-2, qg.qgemm_rows, w, _x(2), torch.zeros((2, 31), dtype=torch.float32))
    _raises(-4, qg.qgemm_rows, w, _x(2), torch.zeros((2, 32), dtype=torch.float16))
    _raises(-2, qg.qgemm_rows, w, _x(2), torch.zeros((2, 64), dtype=torch.float32)[:, ::2])
    _raises(-2, qg.qgemv_add, w, _x(2), torch.zeros((2, 31), dtype=torch.float32))      # resid
    _raises(-2, qg.qgemv_pair, w, _w(k=1024), _x(2))                                     # k differs
    _raises(-2, qg.qgemv_pair_swiglu, w, _w(m=48), _x(1))                                # m differs
    _raises(-2, qg.qgemv_triple, w, w, w, _x(1), None, torch.zeros(5, dtype=torch.float32))
    _raises(-2, qg.qdequant, w, torch.zeros((32, 511), dtype=torch.float32))


def test_single_token_entry_points_check_the_type():
    _raises(-4, qg.qgemv_q5k, _w(qg.Q4_K), _x())
    _raises(-4, qg.qgemv_q4k, _w(qg.Q6_K), _x())


def test_prefill_takes_any_row_count():
    msg = _raises(-4, qg.qgemm_prefill, _w(), _x(100))   # only the device is wrong
    assert "GPU" in msg


def test_probe_checks():
    _raises(-2, qg.qg_stream_read, [torch.zeros(64, dtype=torch.uint8)], torch.zeros(10, dtype=torch.int32))
    _raises(-4, qg.qg_stream_read, [torch.zeros(64, dtype=torch.uint8)],
            torch.zeros(_lib.READ_PROBE_WORDS, dtype=torch.int32))
