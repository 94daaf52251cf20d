"""CPU oracle for shared-prefix, prefill-only branch scoring.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything in this package; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path: the only common module is ``synth`` (seeded inputs, no scoring
arithmetic).

What it computes is the plain definition of the method: every branch is run
from scratch over its full token sequence (prefix + suffix, no prefix
sharing), the last position's log-probabilities over the whole vocabulary are
formed, and the ones at the candidate label ids are renormalised with a
max-subtracted softmax (jdon.com openjev-sglang article: "inference flow"
steps 4-5 and the "prefill-only" section with its yes/no example).  The
planner (``plan.py``) is an independent implementation of the token-prefix
tree, depth-ordered submission rounds and page assignment (LLM2Jev
shared-prefix page: staged-submission and Radix Cache sections).

Precision: GEMMs in float32 (BLAS sgemm), softmax / RMS / RoPE angles in
float64, bf16 storage rounding emulated (round-to-nearest-even) at the points
listed in ``model.py``.  A pure float64 mode (no rounding) serves the
invariant tests.

Pins (see ``tests/test_oracle_*.py``): the worked example of the jdon.com
article, the confidence and expected-score examples, closed forms and
invariants of RMSNorm / RoPE / attention, brute-force pure-Python forwards on
tiny models, the shared-equals-from-scratch invariant and brute-force trie
construction.  "Parity unpinned": the whole-model numbers of the synthetic
configurations have no value printed on the pages; they rest on the pins
above.
"""
