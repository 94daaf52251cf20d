"""The stored oracle values behind the bf16 GPU bars reproduce on the CPU.

One branch of the 2k-prefix workload (the branch whose bar is widest) is
recomputed from scratch by the oracle twice: with float32 contractions (the
stored probabilities) and with float64 contractions (one of the stored
alternatives).  The float64 result must equal its stored value, and the
branch's stored spread must cover the distance between the two, since the
spread is the largest such distance over all alternatives.  Calls only
`oracle` and `synth`.
"""
import gc
import json
import os

import numpy as np
import pytest

from oracle import model as om
from synth import make_instance, make_weights, workload
from tests.golden.make_golden import bars, fingerprint

pytestmark = pytest.mark.slow


def test_stored_probabilities_and_spread_of_a_2k_prefix_branch_reproduce():
    with open(os.path.join(os.path.dirname(__file__), "golden", "probs_w2.json")) as f:
        g = json.load(f)
    wl = workload(2)
    inst = make_instance(wl)
    w = make_weights(wl)
    assert g["fingerprint"] == fingerprint(wl, inst, w)
    ps = g["passes"][0]
    b = int(np.argmax(ps["spread"]))
    seq, lab = inst.full_sequences(0)[ps["branches"][b]]
    m = om.from_weights(w)
    p32 = om.score_from_scratch(m, [seq], [lab])[0]
    del m
    gc.collect()
    # the BLAS splits no dot product across threads, so the float32 sums are
    # in the same order on any thread count
    assert np.max(np.abs(p32 - np.asarray(ps["probs"][b]))) <= 1e-7
    m = om.from_weights(w, gemm="fp64")
    p64 = om.score_from_scratch(m, [seq], [lab])[0]
    del m
    gc.collect()
    assert np.max(np.abs(p64 - np.asarray(ps["by_order"]["fp64"][b]))) <= 1e-9
    assert ps["spread"][b] >= float(np.max(np.abs(p64 - p32))) - 1e-12
    assert ps["spread"][b] > 1e-3  # this branch's bar is the derived one, not the floor
    assert bars(ps["spread"])[b] == pytest.approx(3 * ps["spread"][b])
