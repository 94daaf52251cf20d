"""Seeded synthetic inputs: weights, token ids and label ids.

This module only draws numbers.  It holds none of the scoring arithmetic, and
both the oracle and the GPU path take their inputs from it.

Recipe:

* Weights.  Every weight tensor is filled in row-major order, in chunks of
  ``CHUNK`` elements.  Chunk ``c`` of tensor ``t`` of workload ``w`` (its seed
  root: the workload's index unless it names another) is
  ``np.random.default_rng([w, 0, t, c]).standard_normal(n, float32)`` times
  ``float32(init_std)``.  bf16 workloads round each value once to bf16
  (round-to-nearest-even) and store the 16-bit patterns (``uint16``); the f32
  workload stores ``float32``.  Tensor ids: 0 embedding E [V, d];
  1 unembedding U [V, d]; for layer l: 16+8l Wq [Hq*dh, d], 17+8l Wk [Hkv*dh, d],
  18+8l Wv [Hkv*dh, d], 19+8l Wo [d, Hq*dh] (all [out, in]).  RMSNorm gains are
  ones (parameter-free norm), but they are still materialised as tensors.
* Tokens.  ``default_rng([w, 1])``: for each request in order, the prefix, then
  each branch suffix, uniform in [0, V).  Extra passes draw fresh suffixes
  after all earlier draws.  Trees: root, then for each child its segment
  followed by its leaves' segments.
* Labels.  ``default_rng([w, 2])``: per branch in order,
  ``choice(V, K, replace=False)``, unless the request fixes the label ids.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from .configs import ModelShape, Workload

CHUNK = 1 << 22

TID_E = 0
TID_U = 1


def tid_layer(layer: int, which: str) -> int:
    return 16 + 8 * layer + {"wq": 0, "wk": 1, "wv": 2, "wo": 3}[which]


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _round_bits_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even (inputs are finite)."""
    u = x.view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def _fill(shape, wl_index: int, tid: int, std: float, bf16: bool) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    n_chunks = (n + CHUNK - 1) // CHUNK
    std32 = np.float32(std)

    def work(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        rng = np.random.default_rng([wl_index, 0, tid, c])
        v = rng.standard_normal(hi - lo, dtype=np.float32)
        v *= std32
        out[lo:hi] = _round_bits_bf16(v) if bf16 else v

    if n_chunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(work, range(n_chunks)))
    return out.reshape(shape)


@dataclass
class Weights:
    """Storage: ``uint16`` bf16 bit patterns (bf16 models) or ``float32``."""
    shape: ModelShape
    embed: np.ndarray
    unembed: np.ndarray
    wq: List[np.ndarray]
    wk: List[np.ndarray]
    wv: List[np.ndarray]
    wo: List[np.ndarray]
    attn_norm: List[np.ndarray]
    final_norm: np.ndarray

    @property
    def is_bf16(self) -> bool:
        return self.shape.dtype == "bf16"


def make_weights(wl: Workload, with_embed: bool = True) -> Weights:
    m = wl.model
    bf = m.dtype == "bf16"
    std = m.init_std
    ones = (np.full(m.d, 0x3F80, dtype=np.uint16) if bf else np.ones(m.d, dtype=np.float32))
    emb = _fill((m.vocab, m.d), wl.seed_index, TID_E, std, bf) if with_embed else None
    unemb = _fill((m.vocab, m.d), wl.seed_index, TID_U, std, bf) if with_embed else None
    wq, wk, wv, wo = [], [], [], []
    for l in range(m.n_layers):
        wq.append(_fill((m.hq * m.dh, m.d), wl.seed_index, tid_layer(l, "wq"), std, bf))
        wk.append(_fill((m.hkv * m.dh, m.d), wl.seed_index, tid_layer(l, "wk"), std, bf))
        wv.append(_fill((m.hkv * m.dh, m.d), wl.seed_index, tid_layer(l, "wv"), std, bf))
        wo.append(_fill((m.d, m.hq * m.dh), wl.seed_index, tid_layer(l, "wo"), std, bf))
    return Weights(m, emb, unemb, wq, wk, wv, wo,
                   [ones.copy() for _ in range(m.n_layers)], ones.copy())


@dataclass
class Branch:
    request: int            # index of the prefix it continues
    tokens: np.ndarray      # int32 suffix tokens
    labels: np.ndarray      # int32 candidate label ids (distinct)


@dataclass
class Instance:
    workload: Workload
    prefixes: List[np.ndarray] = field(default_factory=list)   # prefix_branches kind
    passes: List[List[Branch]] = field(default_factory=list)   # per pass, branches in order
    # tree kind: full candidate sequences and their labels, plus the segments
    candidates: List[np.ndarray] = field(default_factory=list)
    cand_labels: List[np.ndarray] = field(default_factory=list)
    tree_root: Optional[np.ndarray] = None
    tree_children: List[np.ndarray] = field(default_factory=list)
    tree_leaves: List[List[np.ndarray]] = field(default_factory=list)

    def full_sequences(self, pass_index: int = 0):
        """(tokens, labels) of every scored sequence, prefix included, in order."""
        if self.workload.kind == "tree":
            return list(zip(self.candidates, self.cand_labels))
        return [(np.concatenate([self.prefixes[b.request], b.tokens]), b.labels)
                for b in self.passes[pass_index]]


def make_instance(wl: Workload) -> Instance:
    V = wl.model.vocab
    tok_rng = np.random.default_rng([wl.seed_index, 1])
    lab_rng = np.random.default_rng([wl.seed_index, 2])

    def draw_tokens(n: int) -> np.ndarray:
        return tok_rng.integers(0, V, size=n, dtype=np.int64).astype(np.int32)

    def draw_labels(k: int, fixed) -> np.ndarray:
        if fixed is not None:
            return np.asarray(fixed, dtype=np.int32)
        return lab_rng.choice(V, size=k, replace=False).astype(np.int32)

    inst = Instance(wl)
    if wl.kind == "tree":
        t = wl.tree
        inst.tree_root = draw_tokens(t.root_len)
        for ci, clen in enumerate(t.child_lens):
            child = draw_tokens(clen)
            inst.tree_children.append(child)
            leaves = []
            for _ in range(t.leaves_per_child[ci]):
                leaf = draw_tokens(t.leaf_len)
                leaves.append(leaf)
                inst.candidates.append(np.concatenate([inst.tree_root, child, leaf]))
                inst.cand_labels.append(draw_labels(t.k_labels, None))
            inst.tree_leaves.append(leaves)
        return inst

    for r in wl.requests:
        inst.prefixes.append(draw_tokens(r.prefix_len))
    first = []
    for ri, r in enumerate(wl.requests):
        for _ in range(r.n_branches):
            first.append(Branch(ri, draw_tokens(r.suffix_len), None))
    inst.passes.append(first)
    for _ in range(1, wl.passes):
        more = []
        for ri, r in enumerate(wl.requests):
            for _ in range(r.n_branches):
                more.append(Branch(ri, draw_tokens(r.suffix_len), None))
        inst.passes.append(more)
    for p in inst.passes:
        for b in p:
            r = wl.requests[b.request]
            b.labels = draw_labels(r.k_labels, r.fixed_labels)
    return inst
