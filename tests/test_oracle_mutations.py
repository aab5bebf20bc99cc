"""The oracle's pins are sharp: each plausible mistake, planted in a private copy of
oracle.c on the CPU, must make at least one pin fail.

Each mutant is compiled with gcc into a temporary directory and checked against the
same hand-derived golden blocks and the numpy fp64 matmul used by test_oracle.py.
"""
import ctypes
import importlib.util
import json
import os
import subprocess

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
GOLDEN = os.path.join(ROOT, "tests", "golden", "blocks.json")

MUTANTS = {
    "q45_nibble_order": ("(qs[32 * c + l] >> (4 * h))", "(qs[32 * c + l] >> (4 * (1 - h)))"),
    "q45_subblock_index": ("int j = 2 * c + h;", "int j = c + 4 * h;"),
    "q45_chunk_index": ("int c = p / 64;", "int c = (p / 32) % 4;"),
    "sixbit_high_scale_bits": ("((s[j - 4] >> 6) << 4)", "((s[j] >> 6) << 4)"),
    "sixbit_high_min_bits": ("((s[j] >> 6) << 4);\n    }", "((s[j - 4] >> 6) << 4);\n    }"),
    "sixbit_scale_min_swap": ("*sc = s[j] & 63;\n        *mn = s[j + 4] & 63;",
                              "*mn = s[j] & 63;\n        *sc = s[j + 4] & 63;"),
    "dmin_sign": ("d * sc * q - dmin * mn", "d * sc * q + dmin * mn"),
    "q5_high_bit_plane": ("16 * ((qh[l] >> j) & 1)", "16 * ((qh[l] >> c) & 1)"),
    "q5_qs_offset": ("b + (has_high ? 48 : 16)", "b + 16"),
    "q6_offset": ("sc[si] * (q - 32)", "sc[si] * (q - 31)"),
    "q6_scale_index": ("8 * s + 2 * g + l / 16", "8 * s + g + l / 16"),
    "q6_high_shift": ("(qh[32 * s + l] >> (2 * g)) & 3", "(qh[32 * s + l] >> g) & 3"),
    "q6_low_select": ("ql[64 * s + 32 * (g & 1) + l] >> (4 * (g >> 1))",
                      "ql[64 * s + 32 * (g >> 1) + l] >> (4 * (g & 1))"),
    "q6_unsigned_scales": ("const int8_t *sc = (const int8_t *)", "const uint8_t *sc = (const uint8_t *)"),
    "nvfp4_nibble_order": ("(4 * (i % 2))", "(4 * (1 - i % 2))"),
    "nvfp4_scale_group": ("scales[i / 16]", "scales[i / 32]"),
    "e4m3_bias": ("ldexp(1.0 + f / 8.0, e - 7)", "ldexp(1.0 + f / 8.0, e - 8)"),
    "e4m3_subnormal": ("ldexp(f / 8.0, -6)", "ldexp(f / 8.0, -7)"),
    "e2m1_bias": ("ldexp(1.0 + 0.5 * f, e - 1)", "ldexp(1.0 + 0.5 * f, e)"),
    "fp16_subnormal_flush": ("v = ldexp((double)f, -24);", "v = 0.0;"),
    "gemm_reversed_x": ("acc += w[kk] * xt[kk];", "acc += w[kk] * xt[k - 1 - kk];"),
    "fp8_scale_row_block": ("scales + (r / 128) * (k / 128) * 2", "scales + (r / 64) * (k / 128) * 2"),
    "fp8_scale_col_block": ("srow + (i / 128) * 2", "srow + (i / 256) * 2"),
    "bf16_bias": ("ldexp(1.0 + f / 128.0, e - 127)", "ldexp(1.0 + f / 128.0, e - 126)"),
    "gemm_unrounded_weights": ("for (int64_t kk = 0; kk < k; kk++) w[kk] = (float)w[kk];", ""),
    "q45_terms_in_fp32": ("w[p] = d * sc * q - dmin * mn;", "w[p] = (float)(d * sc * q) - (float)(dmin * mn);"),
    "gemm_transposed_out": ("y[t * nrows + i] = acc;", "y[i * n + t] = acc;"),
    "swiglu_exp_sign": ("g[i] / (1.0 + exp(-g[i])) * u[i]", "g[i] / (1.0 + exp(g[i])) * u[i]"),
    "swiglu_sigmoid_only": ("g[i] / (1.0 + exp(-g[i])) * u[i]", "1.0 / (1.0 + exp(-g[i])) * u[i]"),
    "swiglu_drops_up": ("g[i] / (1.0 + exp(-g[i])) * u[i]", "g[i] / (1.0 + exp(-g[i]))"),
}


def _load(path):
    L = ctypes.CDLL(path)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.oracle_dequant.argtypes = [i32, p, p, i64, i64, i64, i64, p]
    L.oracle_gemm.argtypes = [i32, p, p, i64, i64, p, i64, p, i64, p, p, i32]
    L.oracle_dequant64.argtypes = [i32, p, p, i64, i64, i64, i64, p]
    L.oracle_swiglu.argtypes = [p, p, i64, p]
    return L


def _test_oracle_module():
    spec = importlib.util.spec_from_file_location("t_oracle", os.path.join(ROOT, "tests", "test_oracle.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _swiglu_ok(L):
    """The SwiGLU pins of test_oracle."""
    def fn(g, u):
        g = np.ascontiguousarray(g, np.float64)
        u = np.ascontiguousarray(u, np.float64)
        out = np.empty_like(g)
        L.oracle_swiglu(g.ctypes.data, u.ctypes.data, g.size, out.ctypes.data)
        return out
    return _test_oracle_module()._swiglu_pins_hold(fn)


def _exact_block_ok(L):
    """The exact-weight pin of test_oracle (rationals from the stored fields)."""
    import struct
    from fractions import Fraction
    d16, dmin16 = np.float16(2.0e-2), np.float16(7.0e-5)
    blk = bytearray(144)
    blk[0:2] = struct.pack("<e", d16)
    blk[2:4] = struct.pack("<e", dmin16)
    blk[4], blk[8] = 63, 61
    for l in range(32):
        blk[16 + l] = l % 16
    data = np.frombuffer(bytes(blk), np.uint8).copy()
    out = np.empty(256, np.float64)
    L.oracle_dequant64(12, data.ctypes.data, None, 1, 256, 0, 1, out.ctypes.data)
    if not all(Fraction(float(out[l])) == Fraction(float(d16)) * 63 * (l % 16) - Fraction(float(dmin16)) * 61
               for l in range(32)):
        return False
    # one-hot x through the GEMM returns the fp32 weights exactly
    x = np.eye(256, dtype=np.float16)
    y = np.empty((256, 1)); a = np.empty((256, 1))
    L.oracle_gemm(12, data.ctypes.data, None, 1, 256, x.view(np.uint16).ctypes.data, 256, None, 1,
                  y.ctypes.data, a.ctypes.data, 1)
    return np.array_equal(y[:, 0], out.astype(np.float32).astype(np.float64))


def _fp8_grid_ok(L):
    """The hand-written FP8 grid of test_oracle."""
    codes, scales, want = _test_oracle_module()._fp8_grid()
    out = np.empty((130, 256), np.float32)
    L.oracle_dequant(1002, codes.ctypes.data, scales.ctypes.data, 130, 256, 0, 130, out.ctypes.data)
    return np.array_equal(out, want.astype(np.float32))


def _pins_pass(L):
    """True when every golden block, the exact-weight block, the FP8 grid and a
    numpy matmul check agree with library L."""
    if not _exact_block_ok(L) or not _fp8_grid_ok(L) or not _swiglu_ok(L):
        return False
    for fx in json.load(open(GOLDEN))["fixtures"]:
        data = np.frombuffer(bytes.fromhex(fx["data"]), np.uint8).copy()
        sc = np.frombuffer(bytes.fromhex(fx["scales"]), np.uint8).copy() if "scales" in fx else None
        out = np.empty(fx["k"], np.float32)
        L.oracle_dequant(fx["type"], data.ctypes.data, None if sc is None else sc.ctypes.data,
                         1, fx["k"], 0, 1, out.ctypes.data)
        for pos, val in fx["expect"].items():
            if out[int(pos)] != np.float32(val) or np.signbit(out[int(pos)]) != np.signbit(val):
                return False
    for wtype in (12, 13, 14, 1001, 1002):
        rng = synth.rng_for(5, wtype)
        m, k, n = 8, 512, 3
        data, scales = synth.weights(wtype, m, k, rng)
        x = synth.activations(n, k, rng)
        w = np.empty((m, k), np.float32)
        sp = None if scales is None else scales.ctypes.data
        L.oracle_dequant(wtype, data.ctypes.data, sp, m, k, 0, m, w.ctypes.data)
        y = np.empty((n, m)); a = np.empty((n, m))
        L.oracle_gemm(wtype, data.ctypes.data, sp, m, k, x.view(np.uint16).ctypes.data, n,
                      None, m, y.ctypes.data, a.ctypes.data, 1)
        ref = x.astype(np.float64) @ w.astype(np.float64).T
        if not np.allclose(y, ref, rtol=1e-12, atol=1e-9):
            return False
    return True


def _build(tmp_path, src_text, name):
    c = tmp_path / f"{name}.c"
    c.write_text(src_text)
    so = tmp_path / f"{name}.so"
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-fopenmp", "-fPIC", "-shared", "-I",
                           os.path.join(ROOT, "oracle"), "-o", str(so), str(c), "-lm"])
    return str(so)


def test_unmutated_copy_passes(tmp_path):
    assert _pins_pass(_load(_build(tmp_path, open(SRC).read(), "orig")))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique in oracle.c"
    so = _build(tmp_path, src.replace(old, new), name)
    assert not _pins_pass(_load(so)), f"planted mistake {name} went unnoticed"
