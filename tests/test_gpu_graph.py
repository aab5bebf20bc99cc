"""HIP graph capture: the calls record plain kernel launches (no memset nodes), so a
captured sequence replayed several times -- with the program's own eager work and
synchronisations between replays, and new inputs each time -- gives exactly the
outputs of the same calls run eagerly."""
import numpy as np
import pytest

import gemm_q4_q5_amd as qg
import synth
from gpu_util import bits, weight, x_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_eager_calls():
    import torch
    k = 2560
    wq, _, _ = weight(qg.Q4_K, 2000, k, 401)
    wk, _, _ = weight(qg.Q4_K, 512, k, 402)
    wv, _, _ = weight(qg.Q6_K, 512, k, 403)
    w8, _, _ = weight(qg.FP8, 640, k, 404)
    n, npf = 8, 300
    x = x_dev(synth.activations(n, k, synth.rng_for(405)))
    xp = x_dev(synth.activations(npf, k, synth.rng_for(406)))
    resid = torch.zeros((n, 2000), dtype=torch.float32, device=x.device)

    def calls(out):
        out["rows"] = qg.qgemm_rows(w8, x, out.get("rows"))
        out["q"], out["k"], out["v"] = qg.qgemv_triple(wq, wk, wv, x, out.get("q"), out.get("k"), out.get("v"))
        out["add"] = qg.qgemv_add(wq, x, resid, out.get("add"))
        out["sw"] = qg.qgemv_pair_swiglu(wk, wk, x, out.get("sw"))
        out["pf"] = qg.qgemm_prefill(wq, xp, out.get("pf"))
        out["pf6"] = qg.qgemm_prefill(wv, xp, out.get("pf6"))   # Q6_K: the two K halves
        return out

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph_out = {}
    with torch.cuda.stream(side):
        calls(graph_out)   # allocate the outputs the graph writes
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(graph_out)
    for rep in range(3):
        print(f"graph replay {rep}", flush=True)
        x.copy_(x_dev(synth.activations(n, k, synth.rng_for(407, rep))))
        xp.copy_(x_dev(synth.activations(npf, k, synth.rng_for(408, rep))))
        resid.normal_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {name: bits(t) for name, t in graph_out.items()}
        eager = calls({})
        torch.cuda.synchronize()
        for name, t in eager.items():
            assert np.array_equal(got[name], bits(t)), f"replay {rep}: {name} differs from the eager call"
