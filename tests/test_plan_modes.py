"""Candidate-first staged rounds (jev_set_plan_mode), on the CPU.

LLM2Jev shared-prefix page, staged-submission section: one real candidate is
scored first and builds the shared prefix (state + its question's
instructions), then the candidates that reuse it are submitted, with the next
question's first candidate in the same round building that question's
instructions, and the rest in a third round; every candidate is scored once
and no warmup question is added.  The page's example order is
{department.shipping} -> {department.billing, department.returns,
severity[0]} -> {severity[1], severity[2]}.
"""
import numpy as np
import pytest

from oracle import plan as op
from synth import make_instance, workload

jev = pytest.importorskip("shared_prefix_kv_amd.jev")


def dry(wl, n_pages, mode):
    m = wl.model
    desc = jev.make_desc(m.n_layers, m.d, m.hq, m.hkv, m.dh, m.vocab, m.dtype, m.rope_theta, m.eps, 40000, 4096)
    ctx = jev.Context(desc, n_pages)
    ctx.set_plan_mode(mode)
    return ctx


def page_example():
    """State, two questions' instructions, three criteria each (lengths are
    arbitrary; the tokens of different parts are disjoint)."""
    state = list(range(100, 180))
    dept, sev = list(range(200, 230)), list(range(300, 321))
    crit = [[1, 2, 3], [4, 5, 6, 7], [8, 9], [11, 12], [13, 14, 15], [16]]
    return [state + dept + crit[0], state + dept + crit[1], state + dept + crit[2],
            state + sev + crit[3], state + sev + crit[4], state + sev + crit[5]]


def readouts_by_round(plan):
    return [sorted(c for x in rnd for c in x.readout) for rnd in plan.rounds]


def test_page_example_order():
    seqs = page_example()
    p = op.plan_candidates(op.ResidentTree(op.PagePool(64)), seqs, "candidate_first")
    assert readouts_by_round(p) == [[0], [1, 2, 3], [4, 5]]
    # round 1 builds state and department instructions with its candidate
    assert [(x.depth, x.b - x.a) for x in p.rounds[0]] == [(1, 80), (2, 30), (3, 3)]
    # round 2 builds the severity instructions with severity[0]
    assert [(x.depth, x.cand_min) for x in p.rounds[1]] == [(2, 3), (3, 1), (3, 2), (3, 3)]
    d = op.plan_candidates(op.ResidentTree(op.PagePool(64)), seqs, "depth")
    assert readouts_by_round(d) == [[], [], [0, 1, 2, 3, 4, 5]]
    ctx = dry(workload(1), 64, jev.JEV_PLAN_CANDIDATE_FIRST)
    assert ctx.plan(seqs) == p.serialize()


def check_invariants(plan, n):
    seen_nodes, round_of = set(), {}
    for r, rnd in enumerate(plan.rounds):
        for x in rnd:
            assert id(x) not in seen_nodes          # every node computed once
            seen_nodes.add(id(x))
            round_of[id(x)] = r
    for r, rnd in enumerate(plan.rounds):
        for x in rnd:
            if x.parent is not None:                # parent computed no later
                assert round_of[id(x.parent)] <= r
    reads = sorted(c for rnd in plan.rounds for x in rnd for c in x.readout)
    assert reads == list(range(n))                  # every candidate read out once


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_plan_of_each_config_matches_oracle(idx):
    wl = workload(idx)
    seqs = [s for s, _ in make_instance(wl).full_sequences(0)]
    p = op.plan_candidates(op.ResidentTree(op.PagePool(4096)), seqs, "candidate_first")
    check_invariants(p, len(seqs))
    assert dry(wl, 4096, jev.JEV_PLAN_CANDIDATE_FIRST).plan(seqs) == p.serialize()
    # same nodes (and tokens computed) as the depth order
    d = op.plan_candidates(op.ResidentTree(op.PagePool(4096)), seqs, "depth")
    key = lambda plan: sorted((x.anchor, x.cand_min, x.a, x.b) for r in plan.rounds for x in r)
    assert key(p) == key(d)


def test_config3_rounds_follow_the_page():
    wl = workload(3)
    seqs = [s for s, _ in make_instance(wl).full_sequences(0)]
    p = op.plan_candidates(op.ResidentTree(op.PagePool(4096)), seqs, "candidate_first")
    assert readouts_by_round(p) == [[0], [1, 2, 3], [4, 5]]


@pytest.mark.parametrize("seed", range(60))
def test_plan_random_tries_bit_exact(seed):
    rng = np.random.default_rng(900 + seed)
    n = int(rng.integers(1, 12))
    base = list(rng.integers(0, 3, 90))
    seqs = []
    for _ in range(n):
        cut = int(rng.integers(0, 90))
        seqs.append(base[:cut] + list(rng.integers(0, 3, int(rng.integers(1, 45)))))
    if rng.integers(0, 3) == 0:
        seqs.append(list(seqs[0]))
    if rng.integers(0, 3) == 0:
        seqs.append(list(seqs[-1][: max(1, len(seqs[-1]) // 2)]))   # a candidate ending inside another
    n_pages = int(rng.integers(20, 200))
    ctx = dry(workload(1), n_pages, jev.JEV_PLAN_CANDIDATE_FIRST)
    tree = op.ResidentTree(op.PagePool(n_pages))
    if rng.integers(0, 2):
        k = int(rng.integers(1, 40))
        (h,) = ctx.prefill_prefix([0], [base[:k]])
        assert tree.prefill([(0, base[:k])]) == [h]
    try:
        want = op.plan_with_reuse(tree, seqs, "candidate_first")
    except op.PoolExhausted:
        with pytest.raises(jev.JevError) as e:
            ctx.plan(seqs)
        assert e.value.code == jev.JEV_ENOMEM
        return
    check_invariants(want, len(seqs))
    assert ctx.plan(seqs) == want.serialize()


def test_mode_errors_and_switching():
    wl = workload(1)
    ctx = dry(wl, 64, jev.JEV_PLAN_DEPTH)
    with pytest.raises(jev.JevError) as e:
        ctx.set_plan_mode(2)
    assert e.value.code == jev.JEV_EINVAL
    seqs = page_example()
    depth = ctx.plan(seqs)
    ctx.set_plan_mode(jev.JEV_PLAN_CANDIDATE_FIRST)
    first = ctx.plan(seqs)
    ctx.set_plan_mode(jev.JEV_PLAN_DEPTH)
    assert ctx.plan(seqs) == depth and first != depth
