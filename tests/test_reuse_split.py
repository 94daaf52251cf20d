"""Reuse inside a resident node at page boundaries, on the CPU.

A candidate that leaves the resident tree partway through a node reuses the
whole pages it shares with that node: the node is split at the page boundary
and the candidate continues the first part.  Pinned on small hand-made trees
(page size 16) and compared with the oracle's statement of the rule.
"""
import pytest

from oracle import plan as op
from synth import workload

jev = pytest.importorskip("shared_prefix_kv_amd.jev")


def dry(n_pages):
    m = workload(1).model
    desc = jev.make_desc(m.n_layers, m.d, m.hq, m.hkv, m.dh, m.vocab, m.dtype, m.rope_theta, m.eps, 40000, 4096)
    return jev.Context(desc, n_pages)


def anchors(plan, n):
    """(anchor handle, matched tokens) per candidate: the serialisation ends
    with the candidate count and one (anchor, matched, read-out node) triple
    per candidate."""
    tail = plan[len(plan) - 3 * n - 1:]
    assert tail[0] == n
    return [(tail[1 + 3 * c], tail[2 + 3 * c]) for c in range(n)]


R = list(range(1, 51))          # 50 tokens: pages of 16, 16, 16, 2


def setup(n_pages=40):
    ctx = dry(n_pages)
    tree = op.ResidentTree(op.PagePool(n_pages))
    (h,) = ctx.prefill_prefix([0], [R])
    assert tree.prefill([(0, R)]) == [h]
    return ctx, tree, h


@pytest.mark.parametrize("seq,anchor_len", [
    (R[:37] + [900, 901], 32),      # diverges at 37: two whole pages reused
    (R[:15] + [900], 0),            # less than a page shared: nothing reused
    (R + [900], 50),                # the whole node, one token left: full-node match
    (list(R), 48),                  # the whole node but no token left: three pages reused
    (R[:16] + [900], 16),           # exactly one page
])
def test_reuse_length(seq, anchor_len):
    ctx, tree, h = setup()
    want = op.plan_with_reuse(tree, [seq])
    got = ctx.plan([seq])
    assert got == want.serialize()
    assert anchors(got, 1)[0][1] == anchor_len
    split = anchor_len not in (0, 50)
    # a split anchors at a new handle (h + 1) holding the first anchor_len / 16 pages
    assert anchors(got, 1)[0][0] == (h + 1 if split else (h if anchor_len else 0))
    # jev_plan changes nothing
    assert ctx.page_table(h) == ([0, 1, 2, 3], [16, 16, 16, 2])
    assert ctx.stats()["resident_prefixes"] == 1


def test_ties_go_to_the_earliest_child_and_candidates_resolve_in_order():
    ctx = dry(40)
    tree = op.ResidentTree(op.PagePool(40))
    a = R[:40]
    b = R[:34] + [700] * 10
    ha, hb = ctx.prefill_prefix([0, 0], [a, b])
    assert tree.prefill([(0, a), (0, b)]) == [ha, hb]
    seqs = [R[:33] + [900], R[:48] + [901], R[:20] + [902]]
    got = ctx.plan(seqs)
    assert got == op.plan_with_reuse(tree, seqs).serialize()
    # first candidate: both children share 32 -> the earlier one (a) is split at 32;
    # second: continues that head, then matches a's 8-token tail in full (40);
    # third: shares 20 with the head (32 long) -> the head is split again at 16
    assert [x[1] for x in anchors(got, 3)] == [32, 40, 16]
