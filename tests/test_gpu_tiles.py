"""The 16-row tiled layout (qg_pack_tiles): the same weights in another order, so every
call gives the same bits on the tiled copy as on the row layout -- rows at several
token counts (decode and general paths, one to four phases per wave), the residual
add, the pair and the triple (also mixing layouts), SwiGLU, the prefill GEMM and the
dequant probe -- at ragged shapes (a last tile of fewer than 16 rows)."""
import numpy as np
import pytest

import gemm_q4_q5_amd as qg
import synth
from gpu_util import bits, weight, x_dev

pytestmark = pytest.mark.gpu


def _tiled(w):
    t = qg.pack_tiles(w)
    assert t.layout == qg.LAYOUT_TILES and t.data.numel() == -(-w.m // 16) * 16 * qg.row_bytes(w.type, w.k)
    return t


@pytest.mark.parametrize("wt,m,k", [(qg.Q4_K, 333, 2560), (qg.Q5_K, 2560, 9728), (qg.Q6_K, 2500, 9728),
                                    (qg.Q6_K, 77, 768), (qg.Q4_K, 9728, 2560)])
def test_tiled_calls_equal_row_layout(wt, m, k):
    import torch
    print(f"tiles type={wt} {m}x{k}", flush=True)
    w, _, _ = weight(wt, m, k, 341)
    t = _tiled(w)
    x = x_dev(synth.activations(32, k, synth.rng_for(342)))
    for n in (1, 5, 8, 17, 32):
        a, b = qg.qgemm_rows(w, x[:n]), qg.qgemm_rows(t, x[:n])
        torch.cuda.synchronize()
        assert np.array_equal(bits(a), bits(b)), f"rows n={n}"
    r = torch.from_numpy(synth.rng_for(343).standard_normal((4, m)).astype(np.float32)).to(x.device)
    assert np.array_equal(bits(qg.qgemv_add(w, x[:4], r)), bits(qg.qgemv_add(t, x[:4], r)))
    assert np.array_equal(bits(qg.qgemv(w, x[0])), bits(qg.qgemv(t, x[0])))
    assert np.array_equal(bits(qg.qgemm_prefill(w, x[:20])), bits(qg.qgemm_prefill(t, x[:20])))
    assert np.array_equal(bits(qg.qdequant(w)), bits(qg.qdequant(t)))


def test_tiled_fused_calls():
    import torch
    k = 2560
    wq, _, _ = weight(qg.Q4_K, 1000, k, 351)
    wk, _, _ = weight(qg.Q4_K, 250, k, 352)
    wv, _, _ = weight(qg.Q6_K, 250, k, 353)
    tq, tk, tv = _tiled(wq), _tiled(wk), _tiled(wv)
    x = x_dev(synth.activations(32, k, synth.rng_for(354)))
    for n in (1, 9, 32):
        xs = x[:n]
        ref = [bits(y) for y in qg.qgemv_triple(wq, wk, wv, xs)]
        for ws in ((tq, tk, tv), (tq, wk, tv)):   # all tiled, and the two layouts mixed
            got = [bits(y) for y in qg.qgemv_triple(*ws, xs)]
            assert all(np.array_equal(a, b) for a, b in zip(ref, got)), f"triple n={n}"
        p0 = [bits(y) for y in qg.qgemv_pair(wq, wq, xs)]
        p1 = [bits(y) for y in qg.qgemv_pair(tq, wq, xs)]
        assert all(np.array_equal(a, b) for a, b in zip(p0, p1)), f"pair n={n}"
        h0 = bits(qg.qgemv_pair_swiglu(wk, wk, xs))
        h1 = bits(qg.qgemv_pair_swiglu(tk, tk, xs))
        torch.cuda.synchronize()
        assert np.array_equal(h0, h1), f"swiglu n={n}"
