"""Long resident prefix (workload 5) vs stored oracle values, through the C ABI.

A 32,768-token prefix over 8 blocks (8 KV heads) is prefilled once; two passes
of 64 fresh 128-token branches are scored against it while it stays resident
(openjev-multimodal performance page, repeated-state section).  The oracle
recomputed a seeded subset of branches of each pass from scratch
(tests/golden/probs_w5.json); each is held to its own bar, max(1e-3, 3 x the
spread of the oracle's probabilities under other accumulation orders).
"""
import numpy as np
import pytest
import torch

from synth import make_instance, workload
from tests.gpu_common import check_branches, device_context, golden, split_probs, stored_bars

pytestmark = pytest.mark.gpu


def test_w5_resident_prefix_two_passes_match_oracle():
    g = golden(5)
    if not all(ps.get("spread") for ps in g["passes"]):
        pytest.skip("the stored workload-5 oracle values carry no accumulation-order spread yet, so there is "
                    "no per-branch bar (tests/golden/make_golden.py writes it)")
    wl = workload(5)
    inst = make_instance(wl)
    P = len(inst.prefixes[0])
    ctx, _ = device_context(5, n_pages=3072, max_pos=P + 256, max_tok=P + 256)
    (h,) = ctx.prefill_prefix([0], [inst.prefixes[0]])
    torch.cuda.synchronize()
    assert ctx.page_table(h)[0] == list(range(P // 16))
    for p in range(2):
        br = inst.passes[p]
        probs, loff = ctx.score_branches([h] * len(br), [b.tokens for b in br], [b.labels for b in br])
        torch.cuda.synchronize()
        got = split_probs(probs, loff)
        sel = g["passes"][p]["branches"]
        check_branches(f"w5 pass {p} branches {sel} vs oracle", [got[b] for b in sel], g["passes"][p]["probs"],
                       stored_bars(g, p))
        st = ctx.stats()
        assert st["computed_tokens"] == 64 * 128 and st["cached_tokens"] == 64 * P
        assert st["pages_in_use"] == P // 16
        for p_ in got:
            assert abs(float(np.sum(p_)) - 1.0) < 1e-4
    ctx.free_pages([h])
    assert ctx.stats()["pages_in_use"] == 0
