"""GPU parity of the MFMA prefill GEMM against the CPU oracle.

The weight tile is rounded once to fp16 before the matrix cores see it, so the
output is held to |y - y_ref| <= 2e-3 * sum|w||x| against the oracle's exact fp64
product, and -- much tighter -- to fp32-accumulation error against the fp64
product of the fp16-rounded oracle weights (which pins the MFMA operand layout).
"""
import numpy as np
import pytest

import gemm_q4_q5_amd as qg
import oracle
import synth
from gpu_util import assert_within, bits, device, weight, x_dev

pytestmark = pytest.mark.gpu

TYPES = [qg.Q4_K, qg.Q5_K, qg.Q6_K, qg.NVFP4]


@pytest.mark.parametrize("wt", TYPES)
@pytest.mark.parametrize("m,k,n", [(300, 1024, 130), (64, 256, 1), (130, 768, 17), (1000, 512, 256)])
def test_prefill_vs_oracle(wt, m, k, n):
    import torch
    print(f"prefill type={wt} m={m} k={k} n={n}", flush=True)
    w, data, scales = weight(wt, m, k, 201)
    x = synth.activations(n, k, synth.rng_for(202, n, k))
    y = qg.qgemm_prefill(w, x_dev(x))
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    y_ref, a = oracle.gemm(wt, data, scales, m, k, x)
    assert_within(got, y_ref, a, what=f"prefill type {wt}")
    # fp64 product of the fp16-rounded weights: only fp32 accumulation error remains
    w16 = oracle.dequant(wt, data, scales, m, k).astype(np.float16).astype(np.float64)
    y16 = x.astype(np.float64) @ w16.T
    a16 = np.abs(x.astype(np.float64)) @ np.abs(w16).T
    assert_within(got, y16, a16, tol=2e-6, what=f"prefill type {wt} vs fp16 weights")


def test_prefill_deterministic():
    import torch
    w, _, _ = weight(qg.Q4_K, 512, 2560, 211)
    x = x_dev(synth.activations(200, 2560, synth.rng_for(212)))
    a = bits(qg.qgemm_prefill(w, x))
    b = bits(qg.qgemm_prefill(w, x))
    torch.cuda.synchronize()
    assert np.array_equal(a, b)
