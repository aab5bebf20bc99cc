"""The adversarial cancelling Q4_K / Q5_K rows (synth.kquant_cancelling), checked
through the oracle: the weights the oracle decodes from the packed bytes must be
the closed form d*sc*q - dmin*m of the fields the rows were built from (reflex-llm
Performance page, Path E, "What worked": the K-quant weight value), and the rows
must really cancel -- exactly (every weight 0, so sum|w||x| = 0) or nearly
(0 < |w| <= 1e-6 * d*sc*q)."""
import numpy as np
import pytest

import oracle
import synth


def _closed_form(f):
    """[m, nb*256] exact weights from the fields, in fp64 (every product is exact there)."""
    d = f["d"].view(np.float16).astype(np.float64)[..., None, None]
    dmin = f["dmin"].view(np.float16).astype(np.float64)[..., None, None]
    sc = f["sc"][..., None].astype(np.float64)
    mn = f["mn"][..., None].astype(np.float64)
    w = d * sc * f["q"] - dmin * mn
    return w.reshape(w.shape[0], -1), (d * sc * f["q"]).reshape(w.shape[0], -1)


@pytest.mark.parametrize("wt", [synth.Q4_K, synth.Q5_K])
@pytest.mark.parametrize("mode", ["exact", "near", "mixed"])
def test_oracle_decodes_the_fields(orc, wt, mode):
    m, k = 40, 1024
    data, f = synth.kquant_cancelling(wt, m, k, synth.rng_for(7, wt), mode)
    w = orc.dequant64(wt, data, None, m, k)
    want, _ = _closed_form(f)
    assert np.array_equal(w, want)


@pytest.mark.parametrize("wt", [synth.Q4_K, synth.Q5_K])
def test_exact_rows_are_all_zero(orc, wt):
    m, k = 40, 2560
    data, _ = synth.kquant_cancelling(wt, m, k, synth.rng_for(8, wt), "exact")
    x = synth.activations(3, k, synth.rng_for(9))
    y, a = orc.gemm(wt, data, None, m, k, x)
    assert np.all(orc.dequant64(wt, data, None, m, k) == 0.0)
    assert np.all(a == 0.0) and np.all(y == 0.0)
    # ... while the two terms of each weight are large
    _, f = synth.kquant_cancelling(wt, m, k, synth.rng_for(8, wt), "exact")
    _, big = _closed_form(f)
    assert np.all(big > 1e-3)


@pytest.mark.parametrize("wt", [synth.Q4_K, synth.Q5_K])
def test_near_rows_cancel_to_one_part_in_a_million(orc, wt):
    m, k = 40, 1024
    data, f = synth.kquant_cancelling(wt, m, k, synth.rng_for(10, wt), "near")
    w = orc.dequant64(wt, data, None, m, k)
    _, big = _closed_form(f)
    assert np.all(w != 0.0)
    assert np.all(np.abs(w) <= 1e-6 * big)


def test_mixed_rows_hold_all_three_kinds(orc):
    m, k = 64, 1024
    data, f = synth.kquant_cancelling(synth.Q4_K, m, k, synth.rng_for(11), "mixed")
    w = orc.dequant64(synth.Q4_K, data, None, m, k)
    _, big = _closed_form(f)
    ordinary = np.repeat((f["mn"] == 0) & (f["sc"] == 1), 32, axis=-1).reshape(m, -1)
    assert (w[~ordinary] == 0).any()                                              # exact cancellation
    assert ((w[~ordinary] != 0) & (np.abs(w[~ordinary]) <= 1e-6 * big[~ordinary])).any()   # near
    assert ordinary.any()
