"""Pins for the CPU oracle: every check here compares it with something other than itself.

* exhaustive fp16 / e4m3 decode against numpy's and torch's own converters;
* the e2m1 value table of the OCP microscaling formats;
* hand-built superblocks whose expected weights were derived by hand from the
  closed forms (tests/golden/blocks.json, each entry citing its passage);
* the GEMM against numpy's fp64 matmul of the dequantized weights, and against
  one-hot inputs (which must return a weight column exactly).
"""
import json
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "blocks.json")


def test_fp16_decode_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.fp16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e4m3_decode_exhaustive(orc):
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.e4m3(i) for i in range(256)])
    nan = np.isnan(ref)
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert orc.e4m3(0x01) == 2.0 ** -9     # smallest subnormal
    assert orc.e4m3(0x7E) == 448.0         # largest finite


def test_bf16_decode_exhaustive(orc):
    import torch
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.bf16(i) for i in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert orc.bf16(0x3F80) == 1.0 and orc.bf16(0x0001) == 2.0 ** -133


def _fp8_grid():
    """A 130 x 256 block-scaled FP8 matrix whose weights are written out by hand
    (TandemLLM Kernels page, "FP8 matrix products": e4m3 codes, one bf16 scale per
    128 x 128 block).  Every code is 0x38 (e4m3 1.0) except four in row 0."""
    codes = np.full((130, 256), 0x38, dtype=np.uint8)
    codes[0, :4] = [0x01, 0xFE, 0x7E, 0x80]           # 2^-9, -448, 448, -0
    # bf16 scales: block (0,0) 0.25, (0,1) 2.0, (1,0) 0.5, (1,1) -4.0
    scales = np.array([[0x3E80, 0x4000], [0x3F00, 0xC080]], dtype=np.uint16).view(np.uint8).reshape(2, 4)
    want = np.empty((130, 256))
    want[:128, :128], want[:128, 128:], want[128:, :128], want[128:, 128:] = 0.25, 2.0, 0.5, -4.0
    want[0, :4] = [2.0 ** -11, -112.0, 112.0, -0.0]
    return codes, scales, want


def test_fp8_block_grid(orc):
    codes, scales, want = _fp8_grid()
    w = orc.dequant(synth.FP8, codes, scales, 130, 256)
    assert np.array_equal(w, want.astype(np.float32))
    assert np.signbit(w[0, 3])
    assert np.array_equal(orc.dequant64(synth.FP8, codes, scales, 130, 256), want)
    assert np.array_equal(orc.dequant(synth.FP8, codes, scales, 130, 256, r0=128, nr=2), want[128:].astype(np.float32))


def test_fp8_products_exact_in_fp32(orc):
    """e4m3 (4 significant bits) x bf16 (8): the fp32 weights are the exact ones."""
    codes, scales = synth.fp8_weights(300, 512, synth.rng_for(78))
    w64 = orc.dequant64(synth.FP8, codes, scales, 300, 512)
    assert np.array_equal(orc.dequant(synth.FP8, codes, scales, 300, 512).astype(np.float64), w64)


def test_e2m1_table(orc):
    # OCP MX e2m1 magnitudes for codes 0..7; bit 3 is the sign.
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        want = -table[c & 7] if c & 8 else table[c & 7]
        got = orc.e2m1(c)
        assert got == want and np.signbit(got) == bool(c & 8)


def test_nvfp4_products_exact_in_fp16(orc):
    """The NVFP4 page states e2m1 x e4m3 fits fp16 exactly (6 of 11 significant bits)."""
    for c in range(16):
        for s in range(256):
            sv = orc.e4m3(s)
            if np.isnan(sv):
                continue
            v = orc.e2m1(c) * sv
            assert float(np.float16(v)) == v
            assert float(np.float32(v)) == v


def test_row_bytes(orc):
    assert orc.row_bytes(12, 2560) == 10 * 144
    assert orc.row_bytes(13, 9728) == 38 * 176
    assert orc.row_bytes(14, 9728) == 38 * 210
    assert orc.row_bytes(1001, 2560) == 1280
    assert orc.row_bytes(12, 2561) == -1
    assert orc.row_bytes(1001, 24) == -1
    assert orc.row_bytes(7, 256) == -1


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["fixtures"]


@pytest.mark.parametrize("fx", _golden(), ids=lambda f: f["name"])
def test_golden_blocks(orc, fx):
    data = np.frombuffer(bytes.fromhex(fx["data"]), dtype=np.uint8)
    scales = np.frombuffer(bytes.fromhex(fx["scales"]), dtype=np.uint8) if "scales" in fx else None
    w = orc.dequant(fx["type"], data, scales, 1, fx["k"])[0]
    for pos, val in fx["expect"].items():
        assert w[int(pos)] == np.float32(val), (fx["name"], pos, w[int(pos)], val)
        assert np.signbit(w[int(pos)]) == np.signbit(val)


def test_golden_q6k_untouched_positions(orc):
    fx = next(f for f in _golden() if f["name"] == "q6k_A_bit_planes")
    w = orc.dequant(14, np.frombuffer(bytes.fromhex(fx["data"]), np.uint8), None, 1, 256)[0]
    rest = np.delete(w, [0, 32, 64, 96])
    assert np.all(rest == -32.0)


def test_block_and_row_stride(orc):
    """Blocks at their 144/176/210-byte strides, and rows after rows."""
    fx = {f["name"]: f for f in _golden()}
    for a, b, t in (("q4k_A_nibble_order", "q4k_B_6bit_high_bits", 12),
                    ("q5k_A_high_bit_plane", "q5k_B_scales_with_high_bits", 13),
                    ("q6k_B_signed_scales", "q6k_C_high_two_bits", 14)):
        A = bytes.fromhex(fx[a]["data"])
        B = bytes.fromhex(fx[b]["data"])
        single_a = orc.dequant(t, np.frombuffer(A, np.uint8), None, 1, 256)[0]
        single_b = orc.dequant(t, np.frombuffer(B, np.uint8), None, 1, 256)[0]
        mat = np.frombuffer(A + B + B + A + A + A, np.uint8)  # 2 rows x 3 blocks
        w = orc.dequant(t, mat, None, 2, 768)
        want = np.stack([np.concatenate([single_a, single_b, single_b]),
                         np.concatenate([single_a, single_a, single_a])])
        assert np.array_equal(w, want)
        assert np.array_equal(orc.dequant(t, mat, None, 2, 768, r0=1, nr=1)[0], want[1])


@pytest.mark.parametrize("wtype", [12, 13, 14, 1001, 1002])
def test_gemm_matches_numpy_fp64(orc, wtype):
    rng = synth.rng_for(123, wtype)
    m, k, n = 24, 768, 3
    data, scales = synth.weights(wtype, m, k, rng)
    x = synth.activations(n, k, rng)
    w = orc.dequant(wtype, data, scales, m, k).astype(np.float64)
    xd = x.astype(np.float64)
    y, a = orc.gemm(wtype, data, scales, m, k, x)
    np.testing.assert_allclose(y, xd @ w.T, rtol=1e-12, atol=1e-12 * (np.abs(xd) @ np.abs(w).T).max())
    np.testing.assert_allclose(a, np.abs(xd) @ np.abs(w).T, rtol=1e-12)
    rows = np.array([5, 0, 23, 5])
    y2, a2 = orc.gemm(wtype, data, scales, m, k, x, rows=rows)
    assert np.array_equal(y2, y[:, rows]) and np.array_equal(a2, a[:, rows])


@pytest.mark.parametrize("wtype", [12, 14, 1001, 1002])
def test_gemm_one_hot_returns_column(orc, wtype):
    rng = synth.rng_for(7, wtype)
    m, k = 16, 512
    data, scales = synth.weights(wtype, m, k, rng)
    w = orc.dequant(wtype, data, scales, m, k)
    cols = [0, 1, 255, 256, 300, 511]
    x = np.zeros((len(cols), k), dtype=np.float16)
    for t, c in enumerate(cols):
        x[t, c] = 1.0
    y, a = orc.gemm(wtype, data, scales, m, k, x)
    for t, c in enumerate(cols):
        assert np.array_equal(y[t], w[:, c].astype(np.float64))
        assert np.array_equal(a[t], np.abs(w[:, c]).astype(np.float64))


def test_gemm_thread_count_does_not_change_result(orc):
    rng = synth.rng_for(9)
    m, k = 64, 1024
    data, _ = synth.weights(12, m, k, rng)
    x = synth.activations(2, k, rng)
    y1, _ = orc.gemm(12, data, None, m, k, x, nthreads=1)
    assert orc.last_threads() == 1
    y4, _ = orc.gemm(12, data, None, m, k, x, nthreads=4)
    assert np.array_equal(y1, y4)


def test_bad_arguments_rejected(orc):
    data = np.zeros(144, np.uint8)
    with pytest.raises(ValueError):
        orc.dequant(12, data, None, 1, 100)
    with pytest.raises(ValueError):
        orc.dequant(1001, np.zeros(16, np.uint8), None, 1, 32)   # NVFP4 needs scales
    with pytest.raises(ValueError):
        orc.gemm(12, data, None, 1, 256, np.zeros((1, 128), np.float16))


def test_generator_is_deterministic_and_in_range():
    a, _ = synth.weights(12, 8, 512, synth.rng_for(0))
    b, _ = synth.weights(12, 8, 512, synth.rng_for(0))
    assert np.array_equal(a, b)
    blocks = a.reshape(8, 2, 144)
    d = blocks[..., 0:2].copy().view(np.float16).astype(np.float64)
    assert d.min() >= 1e-3 * (1 - 2 ** -10) and d.max() <= 2e-2 * (1 + 2 ** -10)
    c, s = synth.weights(1001, 4, 64, synth.rng_for(0))
    import torch
    sv = torch.from_numpy(s).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert sv.min() >= 0.0097 and sv.max() <= 1.0


@pytest.mark.parametrize("wtype", [12, 13, 14, 1001, 1002])
def test_dequant64_rounds_once_to_dequant(orc, wtype):
    """The fp32 weight is the exact weight rounded once (numpy's fp64 -> fp32
    conversion rounds to nearest even)."""
    m, k = 64, 512
    data, scales = synth.weights(wtype, m, k, synth.rng_for(77, wtype))
    exact = orc.dequant64(wtype, data, scales, m, k)
    assert np.array_equal(exact.astype(np.float32), orc.dequant(wtype, data, scales, m, k))
    assert np.array_equal(orc.dequant64(wtype, data, scales, m, k, r0=5, nr=3), exact[5:8])


def test_dequant64_keeps_bits_fp32_drops():
    """A Q4_K sub-block whose weights need more than 24 significant bits: d*sc*q
    and dmin*m are computed here with exact rationals from the stored fields."""
    import struct
    from fractions import Fraction
    orc_ = __import__("oracle")
    d16, dmin16 = np.float16(2.0e-2), np.float16(7.0e-5)   # exponents 2^-6 and 2^-14 apart
    sc, mn = 63, 61                                          # sub-block 0: s[0] = sc, s[4] = m
    blk = bytearray(144)
    blk[0:2] = struct.pack("<e", d16)
    blk[2:4] = struct.pack("<e", dmin16)
    blk[4 + 0] = sc
    blk[4 + 4] = mn
    for l in range(32):
        blk[16 + l] = l % 16   # low nibble: q of position l in sub-block 0
    w64 = orc_.dequant64(12, np.frombuffer(bytes(blk), np.uint8), None, 1, 256)[0]
    w32 = orc_.dequant(12, np.frombuffer(bytes(blk), np.uint8), None, 1, 256)[0]
    lost = 0
    for l in range(32):
        want = Fraction(float(d16)) * sc * (l % 16) - Fraction(float(dmin16)) * mn
        assert Fraction(float(w64[l])) == want, l
        lost += Fraction(float(w32[l])) != want
    assert lost > 0   # the fp32 weights are rounded, the fp64 ones are not


def _swiglu_pins_hold(fn):
    """Values the mathematics fixes for silu(g) * u, silu(g) = g / (1 + e^-g)
    (reflex-llm kernel notes, SwiGLU section):
      silu(0) = 0; silu(1) = 1 / (1 + e^-1) = 0.7310585786300049;
      silu(2) = 2 / (1 + e^-2) = 1.7615941559557646;
      silu(g) - silu(-g) = g for every g (g*s(g) - (-g)*(1 - s(g)), s the logistic);
      silu(g) -> g as g -> +inf and -> 0 as g -> -inf (40: within 1e-15 relative; -40:
      below 2e-16 in magnitude);
      linear in u (u = 0 gives 0, the sign and scale of u carry through)."""
    g = np.array([0.0, 1.0, 2.0, 40.0, -40.0, 1.0, 1.0, 2.0])
    u = np.array([3.0, 1.0, 1.0, 1.0, 1.0, 0.0, -2.5, 1.0])
    out = fn(g, u)
    ok = (out[0] == 0.0 and abs(out[1] - 0.7310585786300049) <= 1e-15
          and abs(out[2] - 1.7615941559557646) <= 1e-15
          and abs(out[3] - 40.0) <= 40.0 * 1e-15 and abs(out[4]) < 2e-16
          and out[5] == 0.0 and abs(out[6] + 2.5 * 0.7310585786300049) <= 3e-15)
    gs = synth.rng_for(17).standard_normal(64) * 8.0
    odd = fn(gs, np.ones_like(gs)) - fn(-gs, np.ones_like(gs))
    return bool(ok and np.allclose(odd, gs, rtol=1e-13, atol=1e-13))


def test_swiglu_pins(orc):
    assert _swiglu_pins_hold(orc.swiglu)
