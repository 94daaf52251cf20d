"""jev_score_branches_noalloc (the entry point for callers that cannot
allocate) against jev_score_branches, through the C ABI: the same kernels with
their scratch in the library's static device array instead of the workspace,
so the probabilities are bitwise equal.  Two calls in a row, the second with
fewer, shorter branches; then a round needing more partial-state rows than the
array holds is refused with JEV_ENOMEM and changes nothing."""
import numpy as np
import pytest
import torch

from synth import make_instance, workload
from tests.gpu_common import device_context, record

pytestmark = pytest.mark.gpu


def test_noalloc_scoring_equals_workspace_scoring():
    from shared_prefix_kv_amd import jev
    inst = make_instance(workload(2))
    ctx, _ = device_context(2, n_pages=1024, max_pos=4096, max_tok=10240)
    (h,) = ctx.prefill_prefix([0], [inst.prefixes[0]])
    br = inst.passes[0]
    rng = np.random.default_rng(31)
    calls = [([b.tokens for b in br], [b.labels for b in br]),
             ([b.tokens[:17] for b in br[:3]], [b.labels for b in br[:3]])]
    for i, (sufs, labs) in enumerate(calls):
        ref, loff = ctx.score_branches([h] * len(sufs), sufs, labs)
        torch.cuda.synchronize()
        out = torch.full_like(ref, float("nan"))
        got, loff2 = ctx.score_branches([h] * len(sufs), sufs, labs, probs=out, noalloc=True)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr() and np.array_equal(loff, loff2)
        diff = float((got - ref).abs().max())
        record(f"noalloc call {i} ({len(sufs)} branches) vs workspace call", diff, 0.0)
        assert torch.equal(got, ref)
    before = ctx.stats()
    many = [list(rng.integers(0, 151936, 48)) for _ in range(64)]
    with pytest.raises(jev.JevError) as e:
        ctx.score_branches([h] * 64, many, [[9891, 2201]] * 64, noalloc=True)
    assert e.value.code == jev.JEV_ENOMEM and "static scratch" in str(e.value)
    assert ctx.stats() == before
    ctx.free_pages([h])
    assert ctx.stats()["pages_in_use"] == 0
    ctx.close()
