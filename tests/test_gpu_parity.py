"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

* qdequant is bit-exact with the oracle's fp32 weights (every type, golden blocks,
  every e4m3 scale code, odd superblock counts that misalign Q6_K blocks);
* GEMV / rows / fused outputs are within 2e-3 * sum|w||x| of the oracle's fp64 sums,
  at sizes that span several workgroups and a ragged last one;
* weights that are exactly zero give exactly zero.
"""
import json
import os

import numpy as np
import pytest

import gemm_q4_q5_amd as qg
import oracle
import synth
from gpu_util import assert_within, bits, device, weight, x_dev

pytestmark = pytest.mark.gpu

TYPES = [qg.Q4_K, qg.Q5_K, qg.Q6_K, qg.NVFP4, qg.FP8]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "blocks.json")


def _dequant_bits_equal(wt, data, scales, m, k):
    import torch
    w = qg.QWeight.from_host(wt, data, m, k, scales, device=device())
    got = qg.qdequant(w)
    torch.cuda.synchronize()
    ref = oracle.dequant(wt, data, scales, m, k)
    g = got.cpu().numpy()
    assert np.array_equal(g.view(np.int32), ref.view(np.int32)), \
        f"type {wt}: {np.sum(g.view(np.int32) != ref.view(np.int32))} weights differ"


@pytest.mark.parametrize("wt", TYPES)
@pytest.mark.parametrize("m,k", [(1, 256), (37, 768), (130, 2560)])
def test_dequant_bit_exact(wt, m, k):
    print(f"dequant type={wt} m={m} k={k}", flush=True)
    data, scales = synth.weights(wt, m, k, synth.rng_for(11, wt, m, k))
    _dequant_bits_equal(wt, data, scales, m, k)


def test_dequant_golden_blocks():
    for fx in json.load(open(GOLDEN))["fixtures"]:
        print("golden", fx["name"], flush=True)
        data = np.frombuffer(bytes.fromhex(fx["data"]), np.uint8).copy()
        sc = np.frombuffer(bytes.fromhex(fx["scales"]), np.uint8).copy() if "scales" in fx else None
        k = fx["k"]
        if fx["type"] == qg.NVFP4 and k % 256:
            reps = 256 // k   # tile the 32-wide fixture to one 256-wide row
            data = np.tile(data, reps)
            sc = np.tile(sc, reps)
            k = 256
        _dequant_bits_equal(fx["type"], data.reshape(1, -1), None if sc is None else sc.reshape(1, -1), 1, k)


def test_dequant_every_e4m3_scale():
    # 16 rows x 256 weights = 256 scale slots: one per e4m3 code except the NaNs.
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F] + [0x38, 0x38], dtype=np.uint8)
    scales = codes.reshape(16, 16)
    data = synth.rng_for(3).integers(0, 256, size=(16, 128), dtype=np.uint8)
    _dequant_bits_equal(qg.NVFP4, data, scales, 16, 256)


@pytest.mark.parametrize("wt", TYPES)
@pytest.mark.parametrize("m,k", [(300, 2560), (77, 768), (1, 256), (1000, 4096)])
def test_gemv_vs_oracle(wt, m, k):
    import torch
    print(f"gemv type={wt} m={m} k={k}", flush=True)
    w, data, scales = weight(wt, m, k, 21)
    x = synth.activations(1, k, synth.rng_for(21, m, k))
    y = qg.qgemv(w, x_dev(x[0]))
    torch.cuda.synchronize()
    y_ref, a = oracle.gemm(wt, data, scales, m, k, x)
    assert_within(y.cpu().numpy(), y_ref[0], a[0], what=f"gemv type {wt}")


@pytest.mark.parametrize("wt", TYPES)
@pytest.mark.parametrize("n", [2, 5, 17, 32])
def test_rows_vs_oracle(wt, n):
    import torch
    m, k = 200, 1024
    print(f"rows type={wt} n={n}", flush=True)
    w, data, scales = weight(wt, m, k, 31)
    x = synth.activations(n, k, synth.rng_for(31, n))
    y = qg.qgemm_rows(w, x_dev(x))
    torch.cuda.synchronize()
    y_ref, a = oracle.gemm(wt, data, scales, m, k, x)
    assert_within(y.cpu().numpy(), y_ref, a, what=f"rows type {wt} n {n}")


@pytest.mark.parametrize("wt", TYPES)
def test_rows_match_single_gemv_bits(wt):
    import torch
    m, k = 333, 2560
    w, _, _ = weight(wt, m, k, 41)
    x = synth.duplicate_rows(synth.activations(32, k, synth.rng_for(41)))
    xd = x_dev(x)
    singles = [bits(qg.qgemv(w, xd[t])) for t in range(32)]
    for n in range(1, 33):
        y = qg.qgemm_rows(w, xd[:n])
        torch.cuda.synchronize()
        yb = bits(y)
        for t in range(n):
            assert np.array_equal(yb[t], singles[t]), f"type {wt}: n={n} row {t} differs from n=1"


def test_fused_equal_single_calls():
    import torch
    k = 2560
    wq, _, _ = weight(qg.Q4_K, 512, k, 51)
    wk, _, _ = weight(qg.Q4_K, 128, k, 52)
    wv, _, _ = weight(qg.Q6_K, 128, k, 53)
    x = x_dev(synth.activations(3, k, synth.rng_for(54)))
    for n in (1, 3):
        xs = x[:n]
        y0, y1, y2 = qg.qgemv_triple(wq, wk, wv, xs)
        p0, p1 = qg.qgemv_pair(wq, wk, xs)
        torch.cuda.synchronize()
        for w_, got in ((wq, y0), (wk, y1), (wv, y2), (wq, p0), (wk, p1)):
            assert np.array_equal(bits(got), bits(qg.qgemm_rows(w_, xs)))


def test_add_equals_resid_plus_product():
    import torch
    m, k = 640, 4096
    w, data, _ = weight(qg.Q4_K, m, k, 61)
    x = synth.activations(2, k, synth.rng_for(61))
    resid = torch.from_numpy(synth.rng_for(62).standard_normal((2, m)).astype(np.float32)).to(device())
    y = qg.qgemv_add(w, x_dev(x), resid)
    prod = qg.qgemm_rows(w, x_dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits(resid + prod))
    # in place
    r2 = resid.clone()
    qg.qgemv_add(w, x_dev(x), r2, r2)
    torch.cuda.synchronize()
    assert np.array_equal(bits(r2), bits(y))
    y_ref, a = oracle.gemm(qg.Q4_K, data, None, m, k, x)
    r = resid.cpu().numpy().astype(np.float64)
    assert_within(y.cpu().numpy(), y_ref + r, a, extra=2.0 ** -23 * np.abs(y_ref + r), what="add")


def test_zero_weights_give_exact_zero():
    import torch
    k, m = 512, 64
    data, _ = synth.weights(qg.Q4_K, m, k, synth.rng_for(71))
    blocks = data.reshape(m, 2, 144)
    blocks[0:16, :, 16:] = 0        # quants 0
    blocks[0:16, :, 4:16] = 0       # scales and mins 0
    blocks[16:32, :, 16:] = 0       # quants 0 ...
    blocks[16:32, :, 8:12] &= 0xC0  # ... and the mins of sub-blocks 0..3 zero (4..7 keep theirs)
    blocks[16:32, :, 12:16] &= 0x0F
    blocks[32:48, :, 0:4] = 0       # d = dmin = 0
    w = qg.QWeight.from_host(qg.Q4_K, data, m, k, device=device())
    x = synth.activations(1, k, synth.rng_for(72))
    y = qg.qgemv(w, x_dev(x[0]))
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert np.all(y[0:16] == 0.0) and np.all(y[32:48] == 0.0)
    y_ref, a = oracle.gemm(qg.Q4_K, data, None, m, k, x)
    assert_within(y, y_ref[0], a[0], what="zeros")


def test_repeat_calls_are_bit_identical():
    import torch
    w, _, _ = weight(qg.Q5_K, 2560, 9728, 81)
    x = x_dev(synth.activations(4, 9728, synth.rng_for(81)))
    a = bits(qg.qgemm_rows(w, x))
    b = bits(qg.qgemm_rows(w, x))
    torch.cuda.synchronize()
    assert np.array_equal(a, b)


# Gate and up tile groups in pairs, the gate sums handed over in LDS.  3 tokens: the
# decode path; 20 and 32: the general path (x staged per workgroup); 9728 rows at 32
# tokens: two K phases per wave; K = 9728 (16 K phases, so at least two per wave).
@pytest.mark.parametrize("m,n,k", [(384, 3, 2560), (384, 20, 2560), (3000, 32, 2560), (9728, 32, 2560),
                                   (640, 1, 9728), (640, 5, 9728)])
def test_swiglu_pair(m, n, k):
    import torch
    print(f"swiglu m={m} n={n} k={k}", flush=True)
    wg, dg, _ = weight(qg.Q4_K, m, k, 91)
    wu, du, _ = weight(qg.Q4_K, m, k, 92)
    x = synth.activations(n, k, synth.rng_for(93, n))
    h = qg.qgemv_pair_swiglu(wg, wu, x_dev(x))
    g, u = qg.qgemv_pair(wg, wu, x_dev(x))
    torch.cuda.synchronize()
    gr, ag = oracle.gemm(qg.Q4_K, dg, None, m, k, x)
    ur, au = oracle.gemm(qg.Q4_K, du, None, m, k, x)
    h_ref = oracle.swiglu(gr, ur)
    # |d silu/dg| <= 1.1 and |silu(g)| <= |g|: propagate the product bound, plus fp32 rounding.
    bound = 2e-3 * (1.1 * ag * np.abs(ur) + np.abs(gr) * au) + 1e-6 * np.abs(h_ref)
    err = np.abs(h.cpu().numpy() - h_ref)
    assert (err <= bound).all(), err.max()
    # row invariance: a row of the n-token call equals its one-token call bit for bit
    xd = x_dev(x)
    hb = bits(h)
    for t in sorted({0, n // 2, n - 1}):
        assert np.array_equal(hb[t], bits(qg.qgemv_pair_swiglu(wg, wu, xd[t:t + 1]))[0]), f"row {t}"


def test_q6k_full_int8_scale_range():
    """Q6_K scales over every int8 code (the workload draws 0..63; the format allows -128..127)."""
    import torch
    for m, k in ((64, 768), (300, 2560)):
        data, _ = synth.weights(qg.Q6_K, m, k, synth.rng_for(101, m), q6_scale_range=(-128, 128))
        _dequant_bits_equal(qg.Q6_K, data, None, m, k)
        w = qg.QWeight.from_host(qg.Q6_K, data, m, k, device=device())
        x = synth.activations(3, k, synth.rng_for(102, m))
        y = qg.qgemm_rows(w, x_dev(x))
        torch.cuda.synchronize()
        y_ref, a = oracle.gemm(qg.Q6_K, data, None, m, k, x)
        assert_within(y.cpu().numpy(), y_ref, a, what="q6k full scales")


# Several K phases per wave.  8190 x 7936 has 512 row tiles (the last ragged) and 31
# superblocks in 16 phases (the last period 15 long): below 4 tokens a wave computes
# two phases, from 4 tokens on four; every row must keep the bits of its one-token
# call, and the sums stay within the tolerance of the oracle's.
@pytest.mark.parametrize("wt", [qg.Q4_K, qg.Q6_K, qg.FP8])
def test_phases_per_wave_keep_rows_bit_identical(wt):
    import torch
    m, k = 8190, 7936
    print(f"phases type={wt} {m}x{k} N=1..32", flush=True)
    w, data, scales = weight(wt, m, k, 301)
    x = synth.duplicate_rows(synth.activations(32, k, synth.rng_for(302)))
    xd = x_dev(x)
    singles = [bits(qg.qgemv(w, xd[t])) for t in range(32)]
    for n in (2, 3, 4, 5, 16, 17, 32):
        yb = bits(qg.qgemm_rows(w, xd[:n]))
        for t in range(n):
            assert np.array_equal(yb[t], singles[t]), f"type {wt}: n={n} row {t} differs from n=1"
    y = qg.qgemm_rows(w, xd)
    torch.cuda.synchronize()
    rng = synth.rng_for(303, wt)
    rows = np.unique(np.concatenate([[0, 1, m - 2, m - 1], rng.choice(m, size=96, replace=False)]))
    y_ref, a = oracle.gemm(wt, data, scales, m, k, x, rows=rows)
    assert_within(y.cpu().numpy()[:, rows], y_ref, a, what=f"phases type {wt}")


# The layer's Q6_K down projection (160 row tiles, 16 phases): one token on the decode
# path, 3..7 tokens two phases per wave in 8-wave workgroups, from 8 tokens the general
# path's grid search; every row keeps the bits of its one-token call.
def test_down_shape_bits_across_launch_shapes():
    import torch
    m, k = 2560, 9728
    w, data, scales = weight(qg.Q6_K, m, k, 305)
    x = synth.duplicate_rows(synth.activations(32, k, synth.rng_for(306)))
    xd = x_dev(x)
    singles = [bits(qg.qgemv(w, xd[t])) for t in range(32)]
    for n in (2, 3, 4, 5, 6, 7, 8, 9, 17, 32):
        print(f"down {m}x{k} n={n}", flush=True)
        yb = bits(qg.qgemm_rows(w, xd[:n]))
        for t in range(n):
            assert np.array_equal(yb[t], singles[t]), f"n={n} row {t} differs from n=1"
    y = qg.qgemm_rows(w, xd[:7])
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, m - 1], synth.rng_for(307).choice(m, size=64, replace=False)]))
    y_ref, a = oracle.gemm(qg.Q6_K, data, scales, m, k, x[:7], rows=rows)
    assert_within(y.cpu().numpy()[:, rows], y_ref, a, what="down 7 tokens")


# The gate/up pair at the layer's shape: the launch shape changes with n (decode path
# below 8 tokens, two phases per wave in 16-wave workgroups from 8 on); each output
# must equal the plain call on its matrix, and every row its one-token call, bit for bit.
def test_pair_layer_shape_bits_across_launch_shapes():
    import torch
    m, k = 9728, 2560
    wg, _, _ = weight(qg.Q4_K, m, k, 311)
    wu, _, _ = weight(qg.Q4_K, m, k, 312)
    x = x_dev(synth.activations(32, k, synth.rng_for(313)))
    single_g = [bits(qg.qgemv(wg, x[t])) for t in range(32)]
    single_u = [bits(qg.qgemv(wu, x[t])) for t in range(32)]
    for n in (1, 4, 7, 8, 9, 16, 17, 32):
        print(f"pair {m}x{k} n={n}", flush=True)
        g, u = qg.qgemv_pair(wg, wu, x[:n])
        torch.cuda.synchronize()
        gb, ub = bits(g), bits(u)
        assert np.array_equal(gb, bits(qg.qgemm_rows(wg, x[:n])))
        assert np.array_equal(ub, bits(qg.qgemm_rows(wu, x[:n])))
        for t in range(n):
            assert np.array_equal(gb[t], single_g[t]) and np.array_equal(ub[t], single_u[t]), f"n={n} row {t}"


# The largest K the boundary accepts (2^20 = 4096 superblocks): 16 phases of 256
# superblocks, x staged in many chunks; 17 rows (a ragged second tile).
@pytest.mark.parametrize("wt", [qg.Q4_K, qg.Q6_K, qg.FP8])
def test_maximum_k(wt):
    import torch
    m, k = 17, 1 << 20
    print(f"max k type={wt}", flush=True)
    w, data, scales = weight(wt, m, k, 321)
    x = synth.activations(32, k, synth.rng_for(322))
    xd = x_dev(x)
    single = [bits(qg.qgemv(w, xd[t])) for t in (0, 4, 31)]
    for n in (5, 32):
        y = qg.qgemm_rows(w, xd[:n])
        torch.cuda.synchronize()
        yb = bits(y)
        for i, t in enumerate((0, 4, 31)):
            if t < n:
                assert np.array_equal(yb[t], single[i]), f"n={n} row {t}"
    y_ref, a = oracle.gemm(wt, data, scales, m, k, x)
    assert_within(y.cpu().numpy(), y_ref, a, what=f"max k type {wt}")
    yp = qg.qgemm_prefill(w, xd[:3])
    torch.cuda.synchronize()
    assert_within(yp.cpu().numpy(), y_ref[:3], a[:3], what=f"max k prefill type {wt}")


# Q6_K with 16 phases and more than 8192 rows at 17..32 tokens: the host's grid search
# would pick 16-wave workgroups of four phases, an instance that is not built (it does
# not fit 128 registers); the fallback (8-wave workgroups, four phases) must keep every
# row's one-token bits and the oracle's tolerance.
def test_q6k_many_rows_two_token_groups():
    import torch
    m, k = 12288, 9728
    print(f"q6k {m}x{k} n=17,32", flush=True)
    w, data, scales = weight(qg.Q6_K, m, k, 331)
    x = synth.duplicate_rows(synth.activations(32, k, synth.rng_for(332)))
    xd = x_dev(x)
    toks = (0, 5, 16, 31)
    singles = {t: bits(qg.qgemv(w, xd[t])) for t in toks}
    for n in (17, 32):
        y = qg.qgemm_rows(w, xd[:n])
        torch.cuda.synchronize()
        yb = bits(y)
        for t in toks:
            if t < n:
                assert np.array_equal(yb[t], singles[t]), f"n={n} row {t} differs from n=1"
    rng = synth.rng_for(333)
    rows = np.unique(np.concatenate([[0, 8191, 8192, m - 1], rng.choice(m, size=64, replace=False)]))
    y_ref, a = oracle.gemm(qg.Q6_K, data, scales, m, k, x, rows=rows)
    assert_within(y.cpu().numpy()[:, rows], y_ref, a, what="q6k many rows")
