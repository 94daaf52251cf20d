"""Pure-Python float64 brute force of the attention-only model, for tiny shapes.

Written with plain lists and the math module, independent of the numpy
oracle, so that a transposed operand, a wrong head mapping or a dropped term
in either shows up as a mismatch.  Weights are the [out, in] row-major
matrices of ``synth.Weights`` converted to nested lists of floats.
"""
from __future__ import annotations

import math
from typing import List, Sequence

Vec = List[float]
Mat = List[List[float]]


def matvec(w: Mat, x: Vec) -> Vec:
    """y[o] = sum_i w[o][i] * x[i]."""
    return [sum(w[o][i] * x[i] for i in range(len(x))) for o in range(len(w))]


def rms(x: Vec, g: Vec, eps: float) -> Vec:
    ms = sum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [x[i] * r * g[i] for i in range(len(x))]


def rope_vec(x: Vec, pos: int, theta: float) -> Vec:
    dh = len(x)
    half = dh // 2
    out = [0.0] * dh
    for i in range(half):
        ang = pos * theta ** (-(2.0 * i) / dh)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = x[i] * c - x[i + half] * s
        out[i + half] = x[i + half] * c + x[i] * s
    return out


def forward_last(tokens: Sequence[int], E: Mat, U: Mat, layers, g_final: Vec,
                 hq: int, hkv: int, dh: int, theta: float, eps: float) -> Vec:
    """Returns log-probabilities over the vocabulary at the last position.

    layers: list of dicts with keys g, wq, wk, wv, wo (nested lists)."""
    n = len(tokens)
    x = [list(E[t]) for t in tokens]
    group = hq // hkv
    for L in layers:
        qs, ks, vs = [], [], []
        for t in range(n):
            h = rms(x[t], L["g"], eps)
            q = matvec(L["wq"], h)
            k = matvec(L["wk"], h)
            v = matvec(L["wv"], h)
            qs.append([rope_vec(q[j * dh:(j + 1) * dh], t, theta) for j in range(hq)])
            ks.append([rope_vec(k[j * dh:(j + 1) * dh], t, theta) for j in range(hkv)])
            vs.append([v[j * dh:(j + 1) * dh] for j in range(hkv)])
        newx = []
        for t in range(n):
            att = []
            for j in range(hq):
                kv = j // group
                sc = [sum(qs[t][j][e] * ks[u][kv][e] for e in range(dh)) / math.sqrt(dh)
                      for u in range(t + 1)]
                mx = max(sc)
                w = [math.exp(s - mx) for s in sc]
                z = sum(w)
                att += [sum(w[u] * vs[u][kv][e] for u in range(t + 1)) / z for e in range(dh)]
            y = matvec(L["wo"], att)
            newx.append([x[t][i] + y[i] for i in range(len(y))])
        x = newx
    hfin = rms(x[-1], g_final, eps)
    z = matvec(U, hfin)
    mx = max(z)
    lse = mx + math.log(sum(math.exp(v - mx) for v in z))
    return [v - lse for v in z]
