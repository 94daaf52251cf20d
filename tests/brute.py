"""Pure-Python float64 brute force of the attention-only model, for tiny shapes.

Written with plain lists and the math module, independent of the numpy
oracle, so that a transposed operand, a wrong head mapping or a dropped term
in either shows up as a mismatch.  Weights are the [out, in] row-major
matrices of ``synth.Weights`` converted to nested lists of floats.

bf16 storage: ``forward_last(..., round_at=...)`` rounds values to bfloat16
(8 significant bits, round to nearest, ties to even, straight from the float64
value) at the named points, so that the oracle's bf16 mode can be pinned point
by point:

  "norm"   RMSNorm output of each block
  "qk"     q and k after RoPE
  "v"      v
  "attn"   attention output (all heads of a token)
  "resid"  residual stream after each add
  "final"  final RMSNorm output

"qk_before_rope" rounds q and k before RoPE instead: a plausible misreading,
used to show that the pin tells the two apart.
"""
from __future__ import annotations

import math
from typing import List, Sequence

Vec = List[float]
Mat = List[List[float]]


STORE_POINTS = ("norm", "qk", "v", "attn", "resid", "final")


def bf16(x: float) -> float:
    """Nearest bfloat16 value of x: frexp gives x = m * 2**e with
    0.5 <= |m| < 1, so m * 256 carries the 8 significant bits; Python's round()
    takes the nearest integer with ties to even."""
    if x == 0.0 or not math.isfinite(x):
        return x
    m, e = math.frexp(x)
    return math.ldexp(round(m * 256.0), e - 8)


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
                 hq: int, hkv: int, dh: int, theta: float, eps: float,
                 round_at: Sequence[str] = ()) -> Vec:
    """Returns log-probabilities over the vocabulary at the last position.

    layers: list of dicts with keys g, wq, wk, wv, wo (nested lists).
    round_at: storage points rounded to bf16 (module docstring)."""
    def r(point: str, vec: Vec) -> Vec:
        return [bf16(a) for a in vec] if point in round_at else vec

    n = len(tokens)
    x = [list(E[t]) for t in tokens]
    group = hq // hkv
    for L in layers:
        qs, ks, vs = [], [], []
        for t in range(n):
            h = r("norm", rms(x[t], L["g"], eps))
            q = matvec(L["wq"], h)
            k = matvec(L["wk"], h)
            v = matvec(L["wv"], h)
            qs.append([r("qk", rope_vec(r("qk_before_rope", q[j * dh:(j + 1) * dh]), t, theta))
                       for j in range(hq)])
            ks.append([r("qk", rope_vec(r("qk_before_rope", k[j * dh:(j + 1) * dh]), t, theta))
                       for j in range(hkv)])
            vs.append([r("v", v[j * dh:(j + 1) * dh]) for j in range(hkv)])
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
            y = matvec(L["wo"], r("attn", att))
            newx.append(r("resid", [x[t][i] + y[i] for i in range(len(y))]))
        x = newx
    hfin = r("final", rms(x[-1], g_final, eps))
    z = matvec(U, hfin)
    mx = max(z)
    lse = mx + math.log(sum(math.exp(v - mx) for v in z))
    return [v - lse for v in z]
