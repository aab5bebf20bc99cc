"""GPU parity at the full sizes of the five workloads, through the same entry points
(and so the same launch configurations) the benchmark times.

Outputs are checked against the CPU oracle on a seeded sample of weight rows (the
oracle computes any row on its own), always including the first and last rows so
the ragged last workgroup is covered; row invariance is checked bit for bit on
every row.

Workloads (seed i for workload i, tensor j of a workload drawn from rng_for(i, j)):
  0  one Q4_K GEMV 1024 x 1024, N = 1 (all rows checked)
  1  a Qwen3-4B-shaped decode layer: QKV triple, Wo + residual, gate/up pair, down,
     at N = 1 and N = 32
  2  row invariance: Q4_K 9728 x 2560 and Q5_K 2560 x 9728, N = 1..32 with
     duplicated rows
  3  prefill chunk N = 512 on the MFMA path: Q4_K 9728 x 2560, Q6_K 2560 x 9728,
     Q5_K 4096 x 2560
  4  NVFP4 16384 x 8192 and 151936 x 2560 at N = 1, 16, 32
"""
import numpy as np
import pytest

import gemm_q4_q5_amd as qg
import oracle
import synth
from gpu_util import assert_within, bits, device, x_dev

pytestmark = pytest.mark.gpu

SAMPLE = 192


def sample_rows(m, seed):
    """Sorted sample of rows: first, last, and a seeded draw of the rest."""
    rng = synth.rng_for(seed, m)
    pick = rng.choice(m, size=min(m, SAMPLE), replace=False)
    return np.unique(np.concatenate([[0, m - 1], pick])).astype(np.int64)


def check_rows(wt, data, scales, m, k, x, y, seed, what, resid=None):
    rows = sample_rows(m, seed)
    y_ref, a = oracle.gemm(wt, data, scales, m, k, x, rows=rows)
    got = np.asarray(y, dtype=np.float64).reshape(x.shape[0], m)[:, rows]
    extra = None
    if resid is not None:
        y_ref = y_ref + resid[:, rows].astype(np.float64)
        extra = 2.0 ** -23 * np.abs(y_ref)
    assert_within(got, y_ref, a, extra=extra, what=what)


def host_weight(seed, j, wt, m, k):
    data, scales = synth.weights(wt, m, k, synth.rng_for(seed, j))
    return data, scales, qg.QWeight.from_host(wt, data, m, k, scales, device=device())


def test_workload0_q4k_1024():
    import torch
    print("workload 0: Q4_K 1024x1024 N=1", flush=True)
    data, _, w = host_weight(0, 0, qg.Q4_K, 1024, 1024)
    x = synth.activations(1, 1024, synth.rng_for(0, 1))
    y = qg.qgemv_q4k(w, x_dev(x[0]))
    torch.cuda.synchronize()
    y_ref, a = oracle.gemm(qg.Q4_K, data, None, 1024, 1024, x)
    assert_within(y.cpu().numpy()[None, :], y_ref, a, what="workload 0")


@pytest.fixture(scope="module")
def layer():
    W = {}
    for j, (name, wt, m, k) in enumerate(synth.QWEN3_4B_LAYER):
        W[name] = host_weight(1, j, wt, m, k) + (wt, m, k)
    return W


@pytest.mark.parametrize("n", [1, 32])
def test_workload1_decode_layer(layer, n):
    import torch
    print(f"workload 1: decode layer N={n}", flush=True)
    rng = synth.rng_for(1, 99, n)
    xh = synth.activations(n, 2560, rng)
    xo = synth.activations(n, 4096, rng)
    xf = synth.activations(n, 9728, rng)
    resid = rng.standard_normal((n, 2560)).astype(np.float32)
    L = {name: v[2] for name, v in layer.items()}
    q, kk, v = qg.qgemv_triple(L["wq"], L["wk"], L["wv"], x_dev(xh))
    o = qg.qgemv_add(L["wo"], x_dev(xo), torch.from_numpy(resid).to(device()))
    g, u = qg.qgemv_pair(L["gate"], L["up"], x_dev(xh))
    if n == 1:
        d = qg.qgemv_q6k(L["down"], x_dev(xf[0]))[None, :]
    else:
        d = qg.qgemm_rows(L["down"], x_dev(xf))
    torch.cuda.synchronize()
    outs = {"wq": (q, xh), "wk": (kk, xh), "wv": (v, xh), "gate": (g, xh), "up": (u, xh), "down": (d, xf)}
    for j, (name, (y, x)) in enumerate(outs.items()):
        data, scales, w, wt, m, k = layer[name]
        check_rows(wt, data, scales, m, k, x, y.cpu().numpy(), 100 + j, f"{name} N={n}")
        # fused outputs equal the plain row-invariant call bit for bit
        assert np.array_equal(bits(y.reshape(n, m)), bits(qg.qgemm_rows(w, x_dev(x)))), name
    data, scales, w, wt, m, k = layer["wo"]
    check_rows(wt, data, scales, m, k, xo, o.cpu().numpy(), 110, f"wo+resid N={n}", resid=resid)


@pytest.mark.parametrize("wt,m,k", [(qg.Q4_K, 9728, 2560), (qg.Q5_K, 2560, 9728)])
def test_workload2_row_invariance(wt, m, k):
    import torch
    print(f"workload 2: type {wt} {m}x{k} N=1..32", flush=True)
    j = 0 if wt == qg.Q4_K else 1
    data, scales, w = host_weight(2, j, wt, m, k)
    x = synth.duplicate_rows(synth.activations(32, k, synth.rng_for(2, 10 + j)))
    xd = x_dev(x)
    single = [bits(qg.qgemv(w, xd[t])) for t in range(32)]
    for n in range(1, 33):
        yb = bits(qg.qgemm_rows(w, xd[:n]))
        for t in range(n):
            assert np.array_equal(yb[t], single[t]), f"N={n}: row {t} differs from its N=1 call"
    # duplicated inputs give duplicated outputs
    for src, dst in ((0, 16), (0, 31), (1, 10)):
        assert np.array_equal(single[src], single[dst])
    y = qg.qgemm_rows(w, xd)
    torch.cuda.synchronize()
    check_rows(wt, data, scales, m, k, x, y.cpu().numpy(), 200 + j, f"workload 2 type {wt}")


@pytest.mark.parametrize("j,wt,m,k", [(0, qg.Q4_K, 9728, 2560), (1, qg.Q6_K, 2560, 9728), (2, qg.Q5_K, 4096, 2560)])
def test_workload3_prefill_512(j, wt, m, k):
    import torch
    print(f"workload 3: prefill type {wt} {m}x{k} N=512", flush=True)
    data, scales, w = host_weight(3, j, wt, m, k)
    x = synth.activations(512, k, synth.rng_for(3, 10 + j))
    y = qg.qgemm_prefill(w, x_dev(x))
    torch.cuda.synchronize()
    rows = sample_rows(m, 300 + j)[:64]
    rows = np.unique(np.concatenate([rows, [m - 1]]))
    y_ref, a = oracle.gemm(wt, data, scales, m, k, x, rows=rows)
    assert_within(y.cpu().numpy()[:, rows], y_ref, a, what=f"prefill type {wt}")
    # The timed copy: the same weights repacked into 16-row tiles give the same bits.
    yt = qg.qgemm_prefill(qg.pack_tiles(w), x_dev(x))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), yt.view(torch.int32)), "tiled prefill differs from the row layout"


@pytest.fixture(scope="module", params=[(16384, 8192), (151936, 2560)], ids=["16384x8192", "head151936x2560"])
def nvfp4_weight(request):
    m, k = request.param
    j = 0 if m == 16384 else 1
    data, scales, w = host_weight(4, j, qg.NVFP4, m, k)
    return data, scales, w, m, k, j


@pytest.mark.parametrize("n", [1, 16, 32])
def test_workload4_nvfp4(nvfp4_weight, n):
    import torch
    data, scales, w, m, k, j = nvfp4_weight
    print(f"workload 4: NVFP4 {m}x{k} N={n}", flush=True)
    x = synth.activations(n, k, synth.rng_for(4, 10 + j, n))
    xd = x_dev(x)
    y = qg.qgemv_nvfp4(w, xd[0])[None, :] if n == 1 else qg.qgemm_rows(w, xd)
    torch.cuda.synchronize()
    check_rows(qg.NVFP4, data, scales, m, k, x, y.cpu().numpy(), 400 + j, f"nvfp4 {m}x{k} N={n}")
    if n > 1:
        y1 = bits(qg.qgemv_nvfp4(w, xd[n - 1]))
        assert np.array_equal(bits(y)[n - 1], y1), "last row differs from its N=1 call"
