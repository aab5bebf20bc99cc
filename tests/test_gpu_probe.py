"""GPU check of the read-stream probe: the XOR it folds into *out equals the XOR of
every 32-bit word of the regions, computed on the host (so every byte was read
exactly once, or an even number of times -- the counts are checked separately by
the HBM counters of the profiles)."""
import numpy as np
import pytest

import gemm_q4_q5_amd as qg
from gpu_util import device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("sizes", [[16], [48, 16], [1 << 20], [123456 * 16, 16 * 5, 7 * 4096 * 16 + 48]])
def test_stream_read_xor(sizes):
    import torch
    print(f"stream_read sizes={sizes}", flush=True)
    rng = np.random.default_rng(sum(sizes))
    host = [rng.integers(0, 2**32, size=s // 4, dtype=np.uint32) for s in sizes]
    regions = [torch.from_numpy(h.view(np.int32)).to(device()) for h in host]
    out = torch.zeros(2048, dtype=torch.int32, device=device())
    qg.qg_stream_read(regions, out)
    torch.cuda.synchronize()
    want = np.uint32(0)
    for h in host:
        want ^= np.bitwise_xor.reduce(h)
    assert np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)) == want
    # a second call folds the same value in again: back to zero
    qg.qg_stream_read(regions, out)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)) == 0
