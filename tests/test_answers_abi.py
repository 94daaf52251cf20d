"""jev_answers through the C ABI, on the CPU: the pages' worked values, the
oracle's answer functions on random distributions, and error paths.

The pinned values are the jdon.com openjev-sglang article's ("confidence"
section: 0.641 for (0.9, 0.05, 0.05), 0 for the uniform and 1 for a one-hot
distribution; "three question types" section: the score example 1.0), stored
in tests/golden/answer_examples.json.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import answers as oa

jev = pytest.importorskip("shared_prefix_kv_amd.jev")

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "answer_examples.json")
NOUL, CHOICE, SCORE = jev.JEV_ANSWER_NOUL, jev.JEV_ANSWER_CHOICE, jev.JEV_ANSWER_SCORE


def run(dists, kinds):
    off = np.zeros(len(dists) + 1, dtype=np.int64)
    off[1:] = np.cumsum([len(d) for d in dists])
    flat = np.concatenate([np.asarray(d, dtype=np.float32) for d in dists])
    return jev.answers(flat, off, kinds)


def test_confidence_and_score_match_the_printed_examples():
    g = json.load(open(GOLDEN))
    cases = g["confidence"]["cases"]
    _, _, conf = run([c["p"] for c in cases], [CHOICE] * len(cases))
    for c, v in zip(cases, conf):
        assert round(v, c["printed_decimals"]) == pytest.approx(c["printed_confidence"], abs=1e-12)
    sc = g["score"]["cases"]
    val, choice, _ = run([c["p"] for c in sc], [SCORE] * len(sc))
    for c, v in zip(sc, val):
        assert v == pytest.approx(c["printed_value"], abs=1e-6)  # float32 inputs
    assert list(choice) == [1]


def test_kinds_ties_and_special_cases():
    val, choice, conf = run([[0.77, 0.23], [0.2, 0.5, 0.5], [0.0, 0.0, 1.0], [0.25] * 4, [0.1, 0.2, 0.3, 0.4]],
                            [NOUL, CHOICE, SCORE, CHOICE, SCORE])
    assert val[0] == pytest.approx(0.77, abs=1e-7)          # P(yes): the first label
    assert val[1] == 1.0 and choice[1] == 1                 # tie -> lowest index
    assert val[2] == 2.0 and conf[2] == pytest.approx(1.0, abs=1e-15)  # one-hot; 0 ln 0 = 0
    assert conf[3] == pytest.approx(0.0, abs=1e-15)         # uniform over 4
    assert val[4] == pytest.approx(0.2 + 0.6 + 1.2, abs=1e-6)


def test_random_distributions_match_the_oracle():
    rng = np.random.default_rng(7)
    dists, kinds = [], []
    for _ in range(300):
        k = int(rng.integers(2, 65))
        p = rng.dirichlet(np.full(k, float(rng.choice([0.05, 0.5, 5.0])))).astype(np.float32)
        if rng.random() < 0.2:
            p[rng.integers(0, k, size=max(1, k // 3))] = 0.0   # exact zeros
        dists.append(p)
        kinds.append(int(rng.integers(0, 3)))
    val, choice, conf = run(dists, kinds)
    for p, kd, v, c, cf in zip(dists, kinds, val, choice, conf):
        q = [float(x) for x in p]
        ref = {NOUL: oa.noul(q), CHOICE: float(oa.choice(q)[0]), SCORE: oa.score(q)}[kd]
        assert v == pytest.approx(ref, rel=1e-12, abs=1e-12)
        assert c == oa.choice(q)[0]
        assert cf == pytest.approx(oa.confidence(q), rel=1e-10, abs=1e-12)


@pytest.mark.parametrize("dists,kinds", [
    ([[1.0]], [NOUL]),                       # K = 1
    ([[1.0 / 65] * 65], [NOUL]),             # K = 65
    ([[0.5, float("nan")]], [NOUL]),         # not finite
    ([[0.5, float("inf")]], [NOUL]),
    ([[1.2, -0.2]], [SCORE]),                # negative
    ([[0.5, 0.5]], [3]),                     # unknown kind
])
def test_bad_inputs_are_rejected_without_output(dists, kinds):
    off = np.zeros(len(dists) + 1, dtype=np.int64)
    off[1:] = np.cumsum([len(d) for d in dists])
    flat = np.concatenate([np.asarray(d, dtype=np.float32) for d in dists])
    with pytest.raises(jev.JevError) as e:
        jev.answers(flat, off, kinds)
    assert e.value.code == jev.JEV_EINVAL


def test_null_pointers_and_offsets_through_the_raw_abi():
    import ctypes
    L = jev.lib()
    value = (ctypes.c_double * 2)(-7.0, -7.0)
    p = (ctypes.c_float * 4)(0.5, 0.5, 0.5, 0.5)
    off = (ctypes.c_int64 * 3)(0, 2, 4)
    bad_off = (ctypes.c_int64 * 3)(1, 2, 4)
    kinds = (ctypes.c_int32 * 2)(0, 0)
    assert L.jev_answers(0, None, None, None, None, None, None) == jev.JEV_OK
    assert L.jev_answers(-1, p, off, kinds, value, None, None) == jev.JEV_EINVAL
    assert L.jev_answers(2, None, off, kinds, value, None, None) == jev.JEV_EINVAL
    assert L.jev_answers(2, p, bad_off, kinds, value, None, None) == jev.JEV_EINVAL
    assert L.jev_answers(2, p, off, kinds, None, None, None) == jev.JEV_EINVAL
    assert list(value) == [-7.0, -7.0]
    assert L.jev_answers(2, p, off, kinds, value, None, None) == jev.JEV_OK   # choice/confidence optional
    assert list(value) == [0.5, 0.5]
    assert math.isfinite(value[0])
