"""GPU parity of the MFMA prefill GEMM against the CPU oracle.

The prefill's operands are the 1..32-token product's: NVFP4 and FP8 codes exact in
fp16 with their scales applied per block, Q6_K (q - 32)*sc*2^-16 in fp16 (exact for
|sc| <= 64) with d applied per superblock, Q4_K / Q5_K through the exact split (no
rounding).  The output is held to |y - y_ref| <= 2e-3 * sum|w||x|
against the oracle's fp64 product, and -- much tighter -- to fp32-accumulation error
against the fp64 product of what the operands stand for (which pins the MFMA operand
layout).  An identity input returns what each weight becomes (Q6_K / FP8 / NVFP4: bit
for bit; Q4_K / Q5_K: the exact weight to within two fp32 roundings).
"""
import numpy as np
import pytest

import gemm_q4_q5_amd as qg
import oracle
import synth
from gpu_util import assert_within, bits, device, prefill_operand, weight, x_dev

pytestmark = pytest.mark.gpu

TYPES = [qg.Q4_K, qg.Q5_K, qg.Q6_K, qg.NVFP4, qg.FP8]


@pytest.mark.parametrize("wt", TYPES)
# 64-token x 128-row blocks: one superblock (k = 256) up to 9 (k = 2304); ragged in
# tokens and rows (a last block with 1..63 of each); one block, and grids of thousands.
# Q6_K grids of fewer than 256 such blocks run as 80-row blocks of two K halves (an odd
# superblock count leaves the second half one short): (300, 1024), (130, 768),
# (1000, 512, 256) and (2500, 2304, 500).
@pytest.mark.parametrize("m,k,n", [(300, 1024, 130), (64, 256, 1), (130, 768, 17), (1000, 512, 256),
                                   (2000, 256, 2050), (1000, 512, 2000), (1000, 256, 2100), (2500, 2304, 500)])
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
    w16 = prefill_operand(wt, data, scales, m, k)
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


# (m, k) with k tokens of an identity input: square and ragged blocks, up to 8
# superblocks per row.
@pytest.mark.parametrize("wt", TYPES)
@pytest.mark.parametrize("m,k", [(300, 512), (1500, 2048), (1250, 1280), (2048, 2048)])
def test_prefill_weight_operand_is_exact_weight_rounded_once(wt, m, k):
    """x = I (k tokens): y[t][r] is what the kernel makes of w[r][t] alone.  NVFP4,
    FP8, Q6_K: one nonzero product of exact fp16 values scaled by an exact factor, so y
    equals prefill_operand bit for bit (the exact weight; for Q6_K with |sc| > 64 its
    fp16-rounded operand times d).  Q4_K / Q5_K (exact split): d*sc*(q - c) exact in
    fp32 plus the fp32 remainder r = d*sc*c - dmin*m, two roundings of quantities no
    larger than the weight, so |y - w| <= 2^-22 |w| and zero weights give exactly
    zero."""
    import torch
    print(f"prefill operand type={wt} m={m} k={k}", flush=True)
    w, data, scales = weight(wt, m, k, 231)
    y = qg.qgemm_prefill(w, x_dev(np.eye(k, dtype=np.float16)))
    torch.cuda.synchronize()
    want = prefill_operand(wt, data, scales, m, k)
    if wt in (qg.Q4_K, qg.Q5_K):
        got = y.T.contiguous().cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - want) <= 2.0 ** -22 * np.abs(want))
        return
    want = want.astype(np.float32) + np.float32(0.0)   # the sum with the zero products turns -0 into +0
    assert np.array_equal(bits(y.T.contiguous()), bits(torch.from_numpy(want)))


def test_prefill_more_token_tiles_than_a_grid_dimension():
    """8.4 M tokens in 64-token blocks: 131,074 token blocks, more than a second grid
    dimension holds; the grid is one-dimensional.  x is generated on the GPU and
    sampled tokens (first, last, both sides of the 65,535 x 128 mark) are checked
    against the oracle."""
    import torch
    m, k = 100, 256
    n = 65536 * 128 + 77
    print(f"prefill type=Q4_K m={m} k={k} n={n}", flush=True)
    w, data, scales = weight(qg.Q4_K, m, k, 241)
    g = torch.Generator(device=device()).manual_seed(242)
    x = (torch.rand((n, k), generator=g, device=device(), dtype=torch.float32) * 2 - 1).to(torch.float16)
    y = qg.qgemm_prefill(w, x)
    torch.cuda.synchronize()
    toks = [0, 1, 65535 * 128 - 1, 65535 * 128, 65535 * 128 + 5, n - 78, n - 1]
    xs = x[toks].cpu().numpy()
    got = y[toks].cpu().numpy().astype(np.float64)
    del x, y
    torch.cuda.empty_cache()
    y_ref, a = oracle.gemm(qg.Q4_K, data, scales, m, k, xs)
    assert_within(got, y_ref, a, what="prefill, 65,537 token tiles")
