"""Shapes and structure of the five synthetic scoring workloads.

Every workload is prefill-only scoring: token prefixes are prefilled once into
16-token KV pages, then branches (suffixes) are scored by reading the last
position's logits at K candidate label ids and renormalising them over the
labels.  The structures mirror what the pages describe:

* a 2000-token conversation with 5 short questions (jdon.com openjev-sglang
  article, section on SGLang's Rust front end and Radix Cache);
* a state -> instructions -> criteria tree submitted in staged rounds
  (LLM2Jev "shared prefix" page, staged-submission section);
* 1.2k-token documents with several questions and 64-way choices
  (openjev-multimodal performance page, four-questions table; jdon.com
  article, 64-way letter-label section);
* a long resident state re-used by a second batch of questions
  (openjev-multimodal performance page, repeated-state section).

The models are synthetic: an attention-only pre-norm stack
(embedding -> [RMSNorm -> causal GQA self-attention with RoPE -> residual] x L
-> RMSNorm -> unembedding) with N(0, 0.02) weights.  No tokenizer, text or
trained weights are involved; uniform random token ids stand in for text.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

PAGE_TOKENS = 16


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d: int
    hq: int
    hkv: int
    dh: int
    vocab: int
    dtype: str  # "f32" or "bf16": storage type of weights and activations
    rope_theta: float = 1.0e4
    eps: float = 1.0e-6
    init_std: float = 0.02

    @property
    def group(self) -> int:
        return self.hq // self.hkv


@dataclass(frozen=True)
class Request:
    """One shared prefix with several scored branches below it."""
    prefix_len: int
    n_branches: int
    suffix_len: int
    k_labels: int
    fixed_labels: Optional[Tuple[int, ...]] = None  # same label ids for every branch


@dataclass(frozen=True)
class TreeSpec:
    """Two-level candidate tree: root state -> instruction nodes -> leaves."""
    root_len: int
    child_lens: Tuple[int, ...]            # one entry per instruction node
    leaves_per_child: Tuple[int, ...]      # number of leaves under each child
    leaf_len: int
    k_labels: int


@dataclass(frozen=True)
class Workload:
    index: int        # 1-based position in the lists below
    name: str
    model: ModelShape
    requests: Tuple[Request, ...] = ()
    tree: Optional[TreeSpec] = None
    passes: int = 1   # >1: later passes draw fresh suffixes over the resident prefix
    seed: Optional[int] = None  # seed root (default: the index)

    @property
    def kind(self) -> str:
        return "tree" if self.tree is not None else "prefix_branches"

    @property
    def seed_index(self) -> int:
        return self.index if self.seed is None else self.seed


TINY_F32 = ModelShape(n_layers=1, d=256, hq=4, hkv=4, dh=64, vocab=1024, dtype="f32")
TINY_F32_GQA2 = ModelShape(n_layers=2, d=256, hq=2, hkv=1, dh=64, vocab=1024, dtype="f32")
QWEN_LIKE_4L = ModelShape(n_layers=4, d=4096, hq=32, hkv=4, dh=128, vocab=151936, dtype="bf16")
LONG_8L = ModelShape(n_layers=8, d=4096, hq=32, hkv=8, dh=128, vocab=151936, dtype="bf16")
QWEN_LIKE_1L = ModelShape(n_layers=1, d=4096, hq=32, hkv=4, dh=128, vocab=151936, dtype="bf16")

# Yes/no label ids of the worked example in the jdon.com article
# (prefill-only section): "yes" = 9891, "no" = 2201.
YES_NO_IDS = (9891, 2201)

WORKLOADS: List[Workload] = [
    Workload(1, "tiny_f32_128x4x16", TINY_F32,
             requests=(Request(prefix_len=128, n_branches=4, suffix_len=16, k_labels=2),)),
    Workload(2, "prefix2000_x5x48_yesno", QWEN_LIKE_4L,
             requests=(Request(prefix_len=2000, n_branches=5, suffix_len=48, k_labels=2,
                               fixed_labels=YES_NO_IDS),)),
    Workload(3, "tree800_2x60_3x40", QWEN_LIKE_4L,
             tree=TreeSpec(root_len=800, child_lens=(60, 60), leaves_per_child=(3, 3),
                           leaf_len=40, k_labels=2)),
    Workload(4, "batch16_prefix1200_x8x64_k64", QWEN_LIKE_4L,
             requests=tuple(Request(prefix_len=1200, n_branches=8, suffix_len=64, k_labels=64)
                            for _ in range(16))),
    Workload(5, "prefix32768_x64x128_k4_2pass", LONG_8L,
             requests=(Request(prefix_len=32768, n_branches=64, suffix_len=128, k_labels=4),),
             passes=2),
]


# Parity-only cases (never timed):
# 6  workload 2 cut to its first block: the same seed, so the same tokens,
#    labels, embedding, unembedding and block-0 weights, run by the same
#    kernel instances; its accumulation-order floor lies below 1e-3;
# 7  workload 3's tree and 8 workload 4's batch on the tiny float32 model
#    (the other reading of "same model shapes as config 1");
# 9  a 2,100-token prefix on the tiny float32 model: a round whose longest
#    attention tile has more than 48 pages (two wave groups per workgroup) and
#    whose long causal tiles are split in two;
# 10 a tiny float32 model with two query heads on one KV head (three rotated
#    heads, so one 128-column projection tile holds both rotated and V
#    columns), two blocks, a prefix long enough for full-K projections.
PARITY_WORKLOADS: List[Workload] = [
    Workload(6, "prefix2000_x5x48_yesno_1block", QWEN_LIKE_1L,
             requests=(Request(prefix_len=2000, n_branches=5, suffix_len=48, k_labels=2,
                               fixed_labels=YES_NO_IDS),), seed=2),
    Workload(7, "tree800_2x60_3x40_tiny_f32", TINY_F32,
             tree=TreeSpec(root_len=800, child_lens=(60, 60), leaves_per_child=(3, 3),
                           leaf_len=40, k_labels=2)),
    Workload(8, "batch16_prefix1200_x8x64_k64_tiny_f32", TINY_F32,
             requests=tuple(Request(prefix_len=1200, n_branches=8, suffix_len=64, k_labels=64)
                            for _ in range(16))),
    Workload(9, "prefix2100_x4x20_tiny_f32", TINY_F32,
             requests=(Request(prefix_len=2100, n_branches=4, suffix_len=20, k_labels=3),)),
    Workload(10, "prefix300_x6x24_tiny_f32_gqa2", TINY_F32_GQA2,
             requests=(Request(prefix_len=300, n_branches=6, suffix_len=24, k_labels=3),)),
]


def workload(index_or_name) -> Workload:
    for w in WORKLOADS + PARITY_WORKLOADS:
        if w.index == index_or_name or w.name == index_or_name:
            return w
    raise KeyError(index_or_name)
