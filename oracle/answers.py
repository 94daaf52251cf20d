"""Answer post-processing of label distributions (test infrastructure only).

jdon.com openjev-sglang article:
* "three question types" section: a yes/no ("noul") question reports P(yes);
  a choice question reports the most likely option and the whole
  distribution; a score question reports the expectation sum_i i * P_i with
  options numbered from 0;
* "confidence" section: confidence = 1 - H(P) / ln K with the Shannon entropy
  in natural log; it measures how concentrated P is, not how often it is
  right.
Reading: argmax ties go to the lowest option index; 0 * ln 0 = 0.
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple


def noul(p: Sequence[float]) -> float:
    """P(yes), with the yes label first."""
    return float(p[0])


def choice(p: Sequence[float]) -> Tuple[int, Sequence[float]]:
    best = 0
    for i in range(1, len(p)):
        if p[i] > p[best]:
            best = i
    return best, list(p)


def score(p: Sequence[float]) -> float:
    return float(sum(i * float(pi) for i, pi in enumerate(p)))


def entropy(p: Sequence[float]) -> float:
    return -sum(float(pi) * math.log(float(pi)) for pi in p if pi > 0.0)


def confidence(p: Sequence[float]) -> float:
    k = len(p)
    return 1.0 - entropy(p) / math.log(k)
