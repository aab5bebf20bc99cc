"""GPU parity on cancelling Q4_K / Q5_K rows (synth.kquant_cancelling): weights
d*sc*q - dmin*m whose two terms cancel exactly (every weight 0) or to one part in a
million.  Every call is held to |y - y_ref| <= 2e-3 * sum|w||x| against the oracle,
and an output whose sum|w||x| is 0 must be exactly 0 (exactly the residual for the
residual-add call): the error has to scale with the weights themselves, not with the
terms that cancel in them (reflex-llm Performance page, Path E, "What worked", the
value formula)."""
import numpy as np
import pytest

import gemm_q4_q5_amd as qg
import oracle
import synth
from gpu_util import assert_within, bits, device, x_dev

pytestmark = pytest.mark.gpu

MODES = ["exact", "near", "mixed"]


def _weight(wt, m, k, mode, seed):
    data, _ = synth.kquant_cancelling(wt, m, k, synth.rng_for(seed, wt, m, k), mode)
    return qg.QWeight.from_host(wt, data, m, k, device=device()), data


@pytest.mark.parametrize("wt", [qg.Q4_K, qg.Q5_K])
@pytest.mark.parametrize("mode", MODES)
def test_gemv_and_rows(wt, mode):
    import torch
    m, k = 300, 2560
    print(f"cancel gemv/rows type={wt} mode={mode}", flush=True)
    w, data = _weight(wt, m, k, mode, 401)
    x = synth.activations(32, k, synth.rng_for(402, wt))
    y_ref, a = oracle.gemm(wt, data, None, m, k, x)
    y1 = qg.qgemv(w, x_dev(x[0]))
    torch.cuda.synchronize()
    assert_within(y1.cpu().numpy(), y_ref[0], a[0], what=f"gemv {mode}")
    for n in (1, 17, 32):
        y = qg.qgemm_rows(w, x_dev(x[:n]))
        torch.cuda.synchronize()
        assert_within(y.cpu().numpy(), y_ref[:n], a[:n], what=f"rows n={n} {mode}")
        assert np.array_equal(bits(y)[0], bits(y1))
    wt_tiles = qg.pack_tiles(w)
    yt = qg.qgemm_rows(wt_tiles, x_dev(x[:17]))
    torch.cuda.synchronize()
    assert np.array_equal(bits(yt), bits(qg.qgemm_rows(w, x_dev(x[:17]))))


@pytest.mark.parametrize("mode", MODES)
def test_fused_calls(mode):
    import torch
    k = 2560
    print(f"cancel fused mode={mode}", flush=True)
    wq, dq = _weight(qg.Q4_K, 512, k, mode, 411)
    wk, dk = _weight(qg.Q5_K, 128, k, mode, 412)
    dv, _ = synth.weights(qg.Q6_K, 128, k, synth.rng_for(413))
    wv = qg.QWeight.from_host(qg.Q6_K, dv, 128, k, device=device())
    x = synth.activations(5, k, synth.rng_for(414, MODES.index(mode)))
    for n in (1, 5):
        xs = x_dev(x[:n])
        y0, y1, y2 = qg.qgemv_triple(wq, wk, wv, xs)
        p0, p1 = qg.qgemv_pair(wq, wk, xs)
        torch.cuda.synchronize()
        for wt, data, m, got in ((qg.Q4_K, dq, 512, y0), (qg.Q5_K, dk, 128, y1), (qg.Q4_K, dq, 512, p0),
                                 (qg.Q5_K, dk, 128, p1)):
            y_ref, a = oracle.gemm(wt, data, None, m, k, x[:n])
            assert_within(got.cpu().numpy(), y_ref, a, what=f"fused n={n} {mode}")
        y_ref, a = oracle.gemm(qg.Q6_K, dv, None, 128, k, x[:n])
        assert_within(y2.cpu().numpy(), y_ref, a, what=f"triple Q6_K n={n}")


@pytest.mark.parametrize("mode", MODES)
def test_residual_add(mode):
    import torch
    m, k = 640, 4096
    print(f"cancel add mode={mode}", flush=True)
    w, data = _weight(qg.Q4_K, m, k, mode, 421)
    x = synth.activations(3, k, synth.rng_for(422))
    resid = torch.from_numpy(synth.rng_for(423).standard_normal((3, m)).astype(np.float32)).to(device())
    y = qg.qgemv_add(w, x_dev(x), resid)
    torch.cuda.synchronize()
    y_ref, a = oracle.gemm(qg.Q4_K, data, None, m, k, x)
    r = resid.cpu().numpy()
    got = y.cpu().numpy()
    assert_within(got, y_ref + r, a, extra=2.0 ** -23 * np.abs(y_ref + r), what=f"add {mode}")
    zero = a == 0
    assert np.array_equal(got[zero], r[zero])   # exactly the residual where the product is exactly 0


@pytest.mark.parametrize("mode", MODES)
def test_swiglu(mode):
    import torch
    m, k, n = 384, 2560, 3
    print(f"cancel swiglu mode={mode}", flush=True)
    wg, dg = _weight(qg.Q4_K, m, k, mode, 431)
    du, _ = synth.weights(qg.Q4_K, m, k, synth.rng_for(432))
    wu = qg.QWeight.from_host(qg.Q4_K, du, m, k, device=device())
    x = synth.activations(n, k, synth.rng_for(433))
    h = qg.qgemv_pair_swiglu(wg, wu, x_dev(x))
    torch.cuda.synchronize()
    gr, ag = oracle.gemm(qg.Q4_K, dg, None, m, k, x)
    ur, au = oracle.gemm(qg.Q4_K, du, None, m, k, x)
    h_ref = oracle.swiglu(gr, ur)
    bound = 2e-3 * (1.1 * ag * np.abs(ur) + np.abs(gr) * au) + 1e-6 * np.abs(h_ref)
    got = h.cpu().numpy()
    assert (np.abs(got - h_ref) <= bound).all()
    assert np.all(got[ag == 0] == 0.0)   # silu(0) * u = 0 where the gate is exactly 0


@pytest.mark.parametrize("wt", [qg.Q4_K, qg.Q5_K])
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("m,n", [(300, 1), (300, 40), (1000, 300)])
def test_prefill(wt, mode, m, n):
    import torch
    k = 1024
    print(f"cancel prefill type={wt} mode={mode} m={m} n={n}", flush=True)
    w, data = _weight(wt, m, k, mode, 441)
    x = synth.activations(n, k, synth.rng_for(442, n))
    y = qg.qgemm_prefill(w, x_dev(x))
    torch.cuda.synchronize()
    y_ref, a = oracle.gemm(wt, data, None, m, k, x)
    assert_within(y.cpu().numpy(), y_ref, a, what=f"prefill {mode}")
