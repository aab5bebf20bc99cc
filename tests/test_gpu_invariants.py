"""Invariants of the products that hold bit for bit at any size, on the GPU.

* Scaling x by a power of two scales every output by the same power exactly: every
  rounding in the path (fp16 x, the fp32 MFMA sums, the sub-block sums of x, the
  scale multiplies) is scale-free while nothing overflows or goes subnormal.  The
  residual add, scaled with it, keeps the property.
* Permuting the weight rows permutes the output columns: a row's arithmetic depends
  on the matrix shape (its K split) and on its own bytes only.  FP8 rows keep their
  128-row scale block (rows move within a block, and blocks move whole).
* Permuting the tokens permutes the output rows (1..32-token calls and the prefill).

These follow from the definition of the product (a sum per output over k of w * x)
and from the row-invariance contract of the 1..32-token calls (TandemLLM Kernels
page, "Decode kernels"), not from the oracle.  Rows layout and the 16-row tiled
layout; token counts that take the decode path and the general path."""
import numpy as np
import pytest

import gemm_q4_q5_amd as qg
import synth
from gpu_util import bits, device, x_dev

pytestmark = pytest.mark.gpu

TYPES = [qg.Q4_K, qg.Q5_K, qg.Q6_K, qg.NVFP4, qg.FP8]
NAMES = {qg.Q4_K: "q4k", qg.Q5_K: "q5k", qg.Q6_K: "q6k", qg.NVFP4: "nvfp4", qg.FP8: "fp8"}


def _weight(wt, m, k, seed):
    data, scales = synth.weights(wt, m, k, synth.rng_for(seed, wt, m, k))
    return data, scales


def _dev(wt, data, scales, m, k):
    return qg.QWeight.from_host(wt, np.ascontiguousarray(data), m, k,
                                None if scales is None else np.ascontiguousarray(scales), device=device())


def _scaled(x, s):
    """x * 2^s in fp16, asserting that it is exact (no overflow, no subnormal loss)."""
    xs = (x.astype(np.float32) * np.float32(2.0 ** s)).astype(np.float16)
    assert np.array_equal(xs.astype(np.float32), x.astype(np.float32) * np.float32(2.0 ** s))
    return xs


def _row_perm(wt, m, rng):
    if wt != qg.FP8:
        return rng.permutation(m)
    nblk = m // 128
    order = rng.permutation(nblk)
    return np.concatenate([128 * b + rng.permutation(128) for b in order])


def _permute_rows(wt, data, scales, perm):
    d = data[perm]
    if scales is None:
        return d, None
    if wt == qg.NVFP4:
        return d, scales[perm]
    return d, scales[perm[::128] // 128]   # FP8: one scale row per 128-row block


@pytest.mark.parametrize("wt", TYPES, ids=[NAMES[t] for t in TYPES])
def test_power_of_two_scaling(wt):
    import torch
    m, k = (384, 2560) if wt == qg.FP8 else (333, 2560)
    print(f"scaling {NAMES[wt]} {m}x{k}", flush=True)
    data, scales = _weight(wt, m, k, 601)
    w = _dev(wt, data, scales, m, k)
    ws = [w] + ([qg.pack_tiles(w)] if wt in (qg.Q4_K, qg.Q5_K, qg.Q6_K) else [])
    x = synth.activations(70, k, synth.rng_for(602, wt))
    x[np.abs(x) < 2.0 ** -12] = 0   # keep x * 2^-1 out of the fp16 subnormals
    r = synth.rng_for(603, wt).standard_normal((5, m)).astype(np.float32)
    for s in (3, -1):
        xs = _scaled(x, s)
        f = np.float32(2.0 ** s)
        for wv in ws:
            for n in (1, 5, 32):
                a = qg.qgemm_rows(wv, x_dev(x[:n]))
                b = qg.qgemm_rows(wv, x_dev(xs[:n]))
                torch.cuda.synchronize()
                assert np.array_equal(bits(a * f), bits(b)), f"rows n={n} s={s} layout={wv.layout}"
            a = qg.qgemv_add(wv, x_dev(x[:5]), torch.from_numpy(r).to(device()))
            b = qg.qgemv_add(wv, x_dev(xs[:5]), torch.from_numpy(r * f).to(device()))
            assert np.array_equal(bits(a * f), bits(b)), f"add s={s}"
            a = qg.qgemm_prefill(wv, x_dev(x))
            b = qg.qgemm_prefill(wv, x_dev(xs))
            torch.cuda.synchronize()
            assert np.array_equal(bits(a * f), bits(b)), f"prefill s={s} layout={wv.layout}"


@pytest.mark.parametrize("wt", TYPES, ids=[NAMES[t] for t in TYPES])
def test_row_permutation(wt):
    import torch
    m, k = (384, 1536) if wt == qg.FP8 else (333, 1536)
    print(f"row permutation {NAMES[wt]} {m}x{k}", flush=True)
    data, scales = _weight(wt, m, k, 611)
    perm = _row_perm(wt, m, synth.rng_for(612, wt))
    dp, sp = _permute_rows(wt, data, scales, perm)
    w, wp = _dev(wt, data, scales, m, k), _dev(wt, dp, sp, m, k)
    pairs = [(w, wp)]
    if wt in (qg.Q4_K, qg.Q5_K, qg.Q6_K):
        pairs.append((qg.pack_tiles(w), qg.pack_tiles(wp)))
    x = x_dev(synth.activations(70, k, synth.rng_for(613, wt)))
    for a_w, b_w in pairs:
        for n in (1, 9, 32):
            a = bits(qg.qgemm_rows(a_w, x[:n]))
            b = bits(qg.qgemm_rows(b_w, x[:n]))
            assert np.array_equal(a[:, perm], b), f"rows n={n} layout={a_w.layout}"
        a = bits(qg.qgemm_prefill(a_w, x))
        b = bits(qg.qgemm_prefill(b_w, x))
        torch.cuda.synchronize()
        assert np.array_equal(a[:, perm], b), f"prefill layout={a_w.layout}"


@pytest.mark.parametrize("wt", TYPES, ids=[NAMES[t] for t in TYPES])
def test_token_permutation(wt):
    import torch
    m, k = (256, 2560) if wt == qg.FP8 else (200, 2560)
    print(f"token permutation {NAMES[wt]} {m}x{k}", flush=True)
    data, scales = _weight(wt, m, k, 621)
    w = _dev(wt, data, scales, m, k)
    x = synth.activations(130, k, synth.rng_for(622, wt))
    rng = synth.rng_for(623, wt)
    for n in (3, 32):
        p = rng.permutation(n)
        a = bits(qg.qgemm_rows(w, x_dev(x[:n])))
        b = bits(qg.qgemm_rows(w, x_dev(x[:n][p])))
        assert np.array_equal(a[p], b), f"rows n={n}"
    p = rng.permutation(130)
    a = bits(qg.qgemm_prefill(w, x_dev(x)))
    b = bits(qg.qgemm_prefill(w, x_dev(x[p])))
    torch.cuda.synchronize()
    assert np.array_equal(a[p], b), "prefill"
