"""Pins of the label softmax and the answer layer against the values the
pages print (CPU only)."""
import json
import math
import os

import numpy as np

from oracle import answers
from oracle.model import label_softmax

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_worked_yes_no_example():
    g = load("worked_example_yes_no.json")
    p = label_softmax(g["logprobs"])
    assert [round(x, g["printed_decimals"]) for x in p] == g["printed_probs"]
    # closed form for two labels: P(yes) = 1 / (1 + exp(l_no - l_yes))
    assert abs(p[0] - 1.0 / (1.0 + math.exp(-1.5 + 0.3))) < 1e-15
    assert abs(p.sum() - 1.0) < 1e-15


def test_label_softmax_shift_invariance_and_stability():
    l = np.array([-0.3, -1.5, -7.0, 0.2])
    assert np.allclose(label_softmax(l), label_softmax(l + 1234.5), atol=1e-15)
    big = label_softmax([1000.0, 999.0])  # a naive exp would overflow
    assert np.isfinite(big).all() and abs(big[0] - 1 / (1 + math.exp(-1))) < 1e-15


def test_confidence_examples():
    g = load("answer_examples.json")["confidence"]
    for case in g["cases"]:
        c = answers.confidence(case["p"])
        assert round(c, case["printed_decimals"]) == case["printed_confidence"]
        if "printed_entropy" in case:
            assert round(answers.entropy(case["p"]), case["printed_decimals"]) == case["printed_entropy"]


def test_score_and_choice_examples():
    g = load("answer_examples.json")["score"]
    for case in g["cases"]:
        assert abs(answers.score(case["p"]) - case["printed_value"]) < 1e-12
    assert answers.choice([0.2, 0.5, 0.5])[0] == 1          # tie -> lowest index
    assert answers.noul([0.77, 0.23]) == 0.77
