"""From-scratch forward of the synthetic attention-only model, and label scoring.

Test infrastructure only (see the package docstring).

Model (the synthetic configurations; the pages use a trained Qwen model whose
weights are not available here): embedding -> L x [RMSNorm -> causal
self-attention with RoPE and grouped KV heads -> residual add] -> RMSNorm ->
unembedding.  Readings taken where the pages say nothing:

* RMSNorm: y = x / sqrt(mean(x^2) + eps) * g, eps = 1e-6, g = ones.
* RoPE: rotate-half pairing (i, i + dh/2), inverse frequency theta^(-2i/dh),
  angle = logical position * inverse frequency, computed in float64.
* Attention: scale 1/sqrt(dh); key u visible to query t iff u <= t; query
  head j reads KV head floor(j / (Hq/Hkv)).
* bf16 storage rounding (bf16 models only) at: RMSNorm outputs; q and k after
  RoPE; v; the attention output; the residual stream after each add; the final
  RMSNorm output.  Logits, log-probabilities and label probabilities are not
  rounded.

Contractions (the projections, q.k, p.v and the unembedding) accumulate in
float32 by default, as the method's "fp32 accumulate" asks.  The ``gemm``
field selects another accumulation, used only to measure how far a change of
summation order alone moves the result (the reproducibility floor that the
bf16 parity bars are derived from): "fp64" (float64 products and sums, then
the same storage rounding), "fp32_krev" (float32, contraction index run in
reverse) and "fp32_khalves" (float32, the two halves of the contraction
summed separately, then added).  The ``elementwise`` field does the same for
the steps between contractions (RMSNorm, RoPE, the attention softmax, the
residual add): float64 by default, or "fp32" (RoPE angles still taken in
float64 and rounded to float32, as a table would hold them).  All of these are
faithful implementations of the same definition.

Scoring (jdon.com openjev-sglang article, "prefill-only" section and
"inference flow" steps 4-5): run the whole prompt once, take the
log-probabilities over the full vocabulary at the last position, read them at
the candidate label ids, and renormalise with a max-subtracted softmax.  No
token is decoded.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

from .bf16 import bits_to_f32, round_bf16


@dataclass
class OracleModel:
    """Weights as float32 (bf16-exact for bf16 models) plus the precision mode.

    mode: "bf16" (emulate bf16 storage, fp32 GEMMs), "f32" (fp32 storage and
    GEMMs) or "f64" (everything float64, no rounding; invariant tests).
    gemm: accumulation of the contractions ("fp32", "fp64", "fp32_krev",
    "fp32_khalves"; see the module docstring).  Ignored in "f64" mode.
    """
    n_layers: int
    d: int
    hq: int
    hkv: int
    dh: int
    vocab: int
    theta: float
    eps: float
    mode: str
    embed: np.ndarray
    unembed: np.ndarray
    wq: List[np.ndarray]
    wk: List[np.ndarray]
    wv: List[np.ndarray]
    wo: List[np.ndarray]
    attn_norm: List[np.ndarray]
    final_norm: np.ndarray
    gemm: str = "fp32"
    elementwise: str = "fp64"

    @property
    def gemm_dtype(self):
        return np.float64 if (self.mode == "f64" or self.gemm == "fp64") else np.float32

    @property
    def ew_dtype(self):
        return np.float32 if (self.elementwise == "fp32" and self.mode != "f64") else np.float64


GEMM_ORDERS = ("fp32", "fp64", "fp32_krev", "fp32_khalves")


def from_weights(w, mode: Optional[str] = None, gemm: str = "fp32", elementwise: str = "fp64") -> OracleModel:
    """Builds the oracle's float view of ``synth.Weights``."""
    s = w.shape
    mode = mode or ("bf16" if s.dtype == "bf16" else "f32")
    if gemm not in GEMM_ORDERS:
        raise ValueError(f"unknown accumulation {gemm!r}")
    if elementwise not in ("fp64", "fp32"):
        raise ValueError(f"unknown elementwise precision {elementwise!r}")
    conv = (lambda a: bits_to_f32(a)) if a_is_bits(w) else (lambda a: np.asarray(a, np.float32))
    wide = mode == "f64" or gemm == "fp64"
    cast = (lambda a: conv(a).astype(np.float64)) if wide else conv
    return OracleModel(
        s.n_layers, s.d, s.hq, s.hkv, s.dh, s.vocab, s.rope_theta, s.eps, mode,
        cast(w.embed), cast(w.unembed),
        [cast(a) for a in w.wq], [cast(a) for a in w.wk], [cast(a) for a in w.wv],
        [cast(a) for a in w.wo], [cast(a) for a in w.attn_norm], cast(w.final_norm), gemm, elementwise)


def contract(m: OracleModel, a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """a [..., k] times b [k, n]: products and sums in the model's accumulation
    (float32 by default; see the module docstring for the alternatives)."""
    gd = m.gemm_dtype
    a = np.asarray(a, gd)
    b = np.asarray(b, gd)
    if gd == np.float64 or m.gemm == "fp32":
        return a @ b
    if m.gemm == "fp32_krev":
        return np.ascontiguousarray(a[..., ::-1]) @ np.ascontiguousarray(b[::-1])
    half = a.shape[-1] // 2
    return a[..., :half] @ b[:half] + a[..., half:] @ b[half:]


def a_is_bits(w) -> bool:
    return w.embed is not None and w.embed.dtype == np.uint16


def store(m: OracleModel, x: np.ndarray) -> np.ndarray:
    """Rounds a value to the model's storage type (no-op in f64 mode)."""
    if m.mode == "bf16":
        return round_bf16(x)
    if m.mode == "f32":
        return np.asarray(x, dtype=np.float32)
    return np.asarray(x, dtype=np.float64)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float, dtype=np.float64) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis (float64 by default)."""
    xd = np.asarray(x, dtype)
    ms = np.mean(xd * xd, axis=-1, keepdims=True)
    return xd / np.sqrt(ms + dtype(eps)) * np.asarray(g, dtype)


def rope(x: np.ndarray, positions: np.ndarray, theta: float, dtype=np.float64) -> np.ndarray:
    """Rotate-half RoPE of x [n, heads, dh] at the given logical positions.
    Angles in float64; the rotation in ``dtype`` (float64 by default)."""
    n, _, dh = x.shape
    half = dh // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / dh)
    ang = np.asarray(positions, np.float64)[:, None] * inv_freq[None, :]
    c = np.cos(ang).astype(dtype)[:, None, :]
    s = np.sin(ang).astype(dtype)[:, None, :]
    xd = np.asarray(x, dtype)
    x1, x2 = xd[..., :half], xd[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def attention(m: OracleModel, q: np.ndarray, k: np.ndarray, v: np.ndarray,
              q_pos: np.ndarray, k_pos: np.ndarray, q_chunk: int = 1024) -> np.ndarray:
    """Causal GQA attention.

    q [nq, Hq, dh], k/v [nk, Hkv, dh]; key u is visible to query t iff
    k_pos[u] <= q_pos[t].  Scores q.k (GEMM precision), scaled by 1/sqrt(dh),
    softmax in float64, then P.v (GEMM precision).  Returns float64 [nq, Hq, dh].
    """
    nq, hq, dh = q.shape
    group = hq // k.shape[1]
    scale = 1.0 / math.sqrt(dh)
    out = np.zeros((nq, hq, dh), dtype=np.float64)
    q_pos = np.asarray(q_pos, np.int64)
    k_pos = np.asarray(k_pos, np.int64)

    def head(j: int) -> None:
        kh = j // group
        kj = np.ascontiguousarray(k[:, kh, :], dtype=m.gemm_dtype)
        vj = np.ascontiguousarray(v[:, kh, :], dtype=m.gemm_dtype)
        for t0 in range(0, nq, q_chunk):
            t1 = min(nq, t0 + q_chunk)
            qj = np.ascontiguousarray(q[t0:t1, j, :], dtype=m.gemm_dtype)
            # keys no query of this chunk can see contribute nothing; skip them
            ks = np.nonzero(k_pos <= q_pos[t0:t1].max())[0]
            ew = m.ew_dtype
            s = contract(m, qj, kj[ks].T).astype(ew) * ew(scale)
            visible = k_pos[None, ks] <= q_pos[t0:t1, None]
            s = np.where(visible, s, ew(-np.inf))
            mx = s.max(axis=1, keepdims=True)
            p = np.exp(s - mx)
            p /= p.sum(axis=1, keepdims=True)
            out[t0:t1, j, :] = contract(m, p, vj[ks]).astype(np.float64)

    if hq == 1 or nq * k.shape[0] < (1 << 16):
        for j in range(hq):
            head(j)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(head, range(hq)))
    return out


def _gemm(m: OracleModel, a: np.ndarray, w: np.ndarray) -> np.ndarray:
    """a [n, in] times w[out, in]^T in the model's accumulation."""
    return contract(m, a, w.T)


def layer_qkv(m: OracleModel, l: int, x: np.ndarray, positions: np.ndarray):
    """RMSNorm -> q, k, v projections -> RoPE on q and k; all stored-rounded."""
    n = x.shape[0]
    h = store(m, rmsnorm(x, m.attn_norm[l], m.eps, m.ew_dtype))
    q = _gemm(m, h, m.wq[l]).reshape(n, m.hq, m.dh)
    k = _gemm(m, h, m.wk[l]).reshape(n, m.hkv, m.dh)
    v = _gemm(m, h, m.wv[l]).reshape(n, m.hkv, m.dh)
    q = store(m, rope(q, positions, m.theta, m.ew_dtype))
    k = store(m, rope(k, positions, m.theta, m.ew_dtype))
    v = store(m, v)
    return q, k, v


def layer_out(m: OracleModel, l: int, x: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Attention output (stored-rounded) -> output projection -> residual add."""
    n = x.shape[0]
    a = store(m, a).reshape(n, m.hq * m.dh)
    y = _gemm(m, a, m.wo[l])
    return store(m, np.asarray(x, m.ew_dtype) + np.asarray(y, m.ew_dtype))


def final_hidden(m: OracleModel, tokens: Sequence[int]) -> np.ndarray:
    """Runs the full sequence from scratch; returns the last position's
    final-RMSNorm output (stored-rounded), shape [d]."""
    tokens = np.asarray(tokens, np.int64)
    n = tokens.shape[0]
    pos = np.arange(n, dtype=np.int64)
    x = store(m, m.embed[tokens])
    for l in range(m.n_layers):
        q, k, v = layer_qkv(m, l, x, pos)
        a = attention(m, q, k, v, pos, pos)
        x = layer_out(m, l, x, a)
    return store(m, rmsnorm(x[-1:], m.final_norm, m.eps, m.ew_dtype))[0]


def full_logprobs(m: OracleModel, hidden: np.ndarray) -> np.ndarray:
    """log_softmax over the whole vocabulary of hidden . U^T (float64 out).

    hidden: [d] or [B, d].  Logits in GEMM precision, log-softmax in float64.
    """
    z = _gemm(m, np.atleast_2d(hidden), m.unembed).astype(np.float64)
    mx = z.max(axis=1, keepdims=True)
    lse = mx + np.log(np.exp(z - mx).sum(axis=1, keepdims=True))
    lp = z - lse
    return lp[0] if np.ndim(hidden) == 1 else lp


def label_softmax(label_logprobs: Sequence[float]) -> np.ndarray:
    """Stable (max-subtracted) softmax over the label log-probabilities, float64.

    jdon.com openjev-sglang article, "inference flow" step 5 and the yes/no
    example of the "prefill-only" section.
    """
    l = np.asarray(label_logprobs, np.float64)
    e = np.exp(l - l.max())
    return e / e.sum()


def score_from_scratch(m: OracleModel, seqs: Sequence[Sequence[int]],
                       labels: Sequence[Sequence[int]]) -> List[np.ndarray]:
    """Label probabilities of every sequence, each recomputed from scratch."""
    hid = np.stack([final_hidden(m, s) for s in seqs])
    lp = full_logprobs(m, hid)
    return [label_softmax(lp[i, np.asarray(lab, np.int64)]) for i, lab in enumerate(labels)]


# ---------------------------------------------------------------------------
# Shared-prefix variant.  Used only by the invariant test that checks, inside
# the oracle, that reusing a prefix's cached K/V gives the same result as the
# from-scratch run (the causality argument behind prefix caching: LLM2Jev
# shared-prefix page, Radix Cache section; jdon.com article, Radix Cache
# paragraph of the SGLang front-end section).
# ---------------------------------------------------------------------------

def prefill_cache(m: OracleModel, tokens: Sequence[int]):
    """Per-layer (k, v) of a prefix computed once."""
    tokens = np.asarray(tokens, np.int64)
    pos = np.arange(tokens.shape[0], dtype=np.int64)
    x = store(m, m.embed[tokens])
    cache = []
    for l in range(m.n_layers):
        q, k, v = layer_qkv(m, l, x, pos)
        cache.append((k, v))
        a = attention(m, q, k, v, pos, pos)
        x = layer_out(m, l, x, a)
    return cache


def final_hidden_with_cache(m: OracleModel, cache, prefix_len: int,
                            suffix: Sequence[int]) -> np.ndarray:
    """Final hidden state of prefix+suffix computing only the suffix rows."""
    suffix = np.asarray(suffix, np.int64)
    pos = prefix_len + np.arange(suffix.shape[0], dtype=np.int64)
    kpos = np.arange(prefix_len + suffix.shape[0], dtype=np.int64)
    x = store(m, m.embed[suffix])
    for l in range(m.n_layers):
        q, k, v = layer_qkv(m, l, x, pos)
        kc, vc = cache[l]
        a = attention(m, q, np.concatenate([kc, k]), np.concatenate([vc, v]), pos, kpos)
        x = layer_out(m, l, x, a)
    return store(m, rmsnorm(x[-1:], m.final_norm, m.eps, m.ew_dtype))[0]
