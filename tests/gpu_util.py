"""Helpers shared by the GPU parity tests (inputs from synth, references from oracle)."""
import numpy as np

import oracle
import synth

TOL = 2e-3   # |y - y_ref| <= TOL * sum_k |w||x|  (per output)


def device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    return torch.device("cuda:0")


def weight(wtype, m, k, seed, *path):
    """(QWeight on the GPU, host data, host scales)."""
    import gemm_q4_q5_amd as qg
    data, scales = synth.weights(wtype, m, k, synth.rng_for(seed, wtype, m, k, *path))
    return qg.QWeight.from_host(wtype, data, m, k, scales, device=device()), data, scales


def x_dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(device())


def assert_within(y, y_ref, a, extra=None, tol=TOL, what=""):
    """Element-wise |y - y_ref| <= tol * a (+ extra); outputs with a == 0 must be exact."""
    y = np.asarray(y, dtype=np.float64)
    bound = tol * a + (0.0 if extra is None else extra)
    err = np.abs(y - y_ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} outputs out of bound; worst err {err.max():.3e}, "
                           f"at bound {bound.flat[np.argmax(err - bound)]:.3e}")
    return float((err / np.maximum(a, 1e-30)).max())


def bits(t):
    import torch
    return t.detach().contiguous().view(torch.int32).cpu().numpy()


def prefill_operand(wtype, data, scales, m, k):
    """What the prefill's weight operands stand for, in weight units (fp64): the
    oracle's exact weight, except Q6_K, whose operand is the fp16 rounding of
    sc*(q - 32)*2^-16 (exact for |sc| <= 64) scaled by d*2^16 (the integer sc*(q - 32)
    is the exact weight over its superblock's d)."""
    w = oracle.dequant64(wtype, data, scales, m, k)
    if wtype != synth.Q6_K:
        return w
    blk = np.ascontiguousarray(data).reshape(m, k // 256, 210)
    d = blk[..., 208:210].copy().view(np.float16)[..., 0].astype(np.float64)   # [m, nb]
    d = np.repeat(d, 256, axis=1)
    ki = np.divide(w, d, out=np.zeros_like(w), where=d != 0)
    return d * (ki * 2.0 ** -16).astype(np.float16).astype(np.float64) * 2.0 ** 16
