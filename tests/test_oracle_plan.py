"""Pins of the oracle planner: brute-force trie from pairwise common prefixes,
plan invariants, and the page ids the configurations must get (CPU only)."""
import numpy as np
import pytest

from oracle import plan as op
from synth import make_instance, workload


def lcp(a, b):
    n = 0
    while n < len(a) and n < len(b) and a[n] == b[n]:
        n += 1
    return n


def brute_nodes(seqs):
    """Undissolved compressed trie as a set of (candidate set, a, b).

    For candidate c the positions where the set {c' : lcp(c, c') >= p} changes
    (plus its own end) cut its path into runs (a, b]; each run is a node
    shared by exactly the candidates whose common prefix with c reaches b."""
    out = set()
    n = len(seqs)
    L = [[lcp(seqs[i], seqs[j]) for j in range(n)] for i in range(n)]
    for c in range(n):
        cuts = sorted({L[c][j] for j in range(n)} | {len(seqs[c])} | {0})
        cuts = [x for x in cuts if x <= len(seqs[c])]
        for a, b in zip(cuts, cuts[1:]):
            members = tuple(sorted(j for j in range(n) if L[c][j] >= b))
            out.add((members, a, b))
    return out


def collect(nodes):
    acc = []
    for x in nodes:
        acc.append(x)
        acc += collect(x.children)
    return acc


@pytest.mark.parametrize("seed", range(40))
def test_trie_matches_pairwise_lcp_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 8))
    base = list(rng.integers(0, 3, 30))
    seqs = []
    for _ in range(n):
        cut = int(rng.integers(0, 30))
        seqs.append(base[:cut] + list(rng.integers(0, 3, int(rng.integers(1, 12)))))
    rel = {c: list(map(int, s)) for c, s in enumerate(seqs)}
    nodes = collect(op._build(list(range(n)), 0, rel, 0))
    got = {(tuple(x.cands), x.a, x.b) for x in nodes}
    assert got == brute_nodes(rel)


def _check_plan_invariants(seqs, plan, n_pages):
    nodes = {x.node_id: x for rnd in plan.rounds for x in rnd}
    read = []
    for r, rnd in enumerate(plan.rounds):
        for x in rnd:
            assert x.depth == r + 1
            if x.parent is not None:
                assert x.parent.depth == x.depth - 1
                assert x.a == x.parent.b
            else:
                assert x.a == 0
            if x.children and not x.readout:
                assert x.b - x.a >= op.PAGE          # dissolved otherwise
            assert len(x.pages) == op.n_pages_for(x.b - x.a)
            read += x.readout
        keys = [(x.depth, x.cand_min) for x in rnd]
        assert keys == sorted(keys)
    assert sorted(read) == list(range(len(seqs)))        # each candidate once
    # every token position of every candidate maps to one (page, slot) along
    # its path; identical prefixes map to identical pages
    for c, s in enumerate(seqs):
        x = nodes[plan.readout_node[c]]
        assert x.b + plan.anchor_len[c] == len(s)
        path = []
        while x is not None:
            path.append(x)
            x = x.parent
        slots = []
        for x in reversed(path):
            for i in range(x.b - x.a):
                slots.append((x.pages[i // op.PAGE], i % op.PAGE))
        assert len(slots) == len(s) - plan.anchor_len[c]
        assert len(set(slots)) == len(slots)
    # a node (hence its pages) is shared only by candidates whose tokens agree
    # on the node's whole path
    for x in nodes.values():
        heads = {tuple(seqs[c][: plan.anchor_len[c] + x.b]) for c in x.cands}
        assert len(heads) == 1
    # no page held by two live nodes at once
    live = set()
    for r, rnd in enumerate(plan.rounds):
        for x in rnd:
            for p in x.pages:
                assert p not in live and 0 <= p < n_pages
                live.add(p)
        for x in rnd:
            if not x.children:
                live -= set(x.pages)


@pytest.mark.parametrize("seed", range(40))
def test_plan_invariants_random(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(1, 9))
    base = list(rng.integers(0, 4, 80))
    seqs = []
    for _ in range(n):
        cut = int(rng.integers(0, 80))
        seqs.append(base[:cut] + list(rng.integers(0, 4, int(rng.integers(1, 40)))))
    pool = op.PagePool(4096)
    tree = op.ResidentTree(pool)
    before = sorted(pool.free)
    plan = op.plan_candidates(tree, seqs)
    _check_plan_invariants(seqs, plan, 4096)
    assert sorted(pool.free) == before


def test_short_shared_run_is_dissolved():
    # two candidates share only 3 tokens below a 20-token common prefix
    common = list(range(100, 120))
    seqs = [common + [1, 2, 3] + [7] * 10, common + [1, 2, 3] + [8] * 10, common + [9] * 10]
    plan = op.plan_candidates(op.ResidentTree(op.PagePool(64)), seqs)
    assert len(plan.rounds) == 2
    leaves = plan.rounds[1]
    assert [(x.a, x.b) for x in leaves] == [(20, 33), (20, 33), (20, 30)]


def test_candidate_ending_inside_tree_is_read_out_there():
    seqs = [list(range(40)), list(range(40)) + list(range(500, 520)), list(range(40))]
    plan = op.plan_candidates(op.ResidentTree(op.PagePool(64)), seqs)
    top = plan.rounds[0][0]
    assert top.readout == [0, 2] and plan.readout_node == [0, 1, 0]


def test_config3_plan_matches_staged_rounds_and_expected_pages():
    """LLM2Jev staged-submission example: state -> 2 questions -> 3 criteria
    each, scored in 3 rounds, every candidate exactly once, in input order."""
    inst = make_instance(workload(3))
    pool = op.PagePool(1024)
    plan = op.plan_candidates(op.ResidentTree(pool), inst.candidates)
    assert len(plan.rounds) == 3
    r1, r2, r3 = plan.rounds
    assert [(x.a, x.b) for x in r1] == [(0, 800)] and r1[0].pages == list(range(50))
    assert [(x.a, x.b) for x in r2] == [(800, 860), (800, 860)]
    assert r2[0].pages == [50, 51, 52, 53] and r2[1].pages == [54, 55, 56, 57]
    assert len(r3) == 6
    for i, x in enumerate(r3):
        assert (x.a, x.b) == (860, 900)
        assert x.pages == [58 + 3 * i, 59 + 3 * i, 60 + 3 * i]
        assert x.readout == [i]
    assert plan.readout_node == [3, 4, 5, 6, 7, 8]
    assert pool.n_free() == 1024


def test_explicit_prefix_and_branch_pages_for_configs():
    # config 2: prefix 0..124, leaves 125..139 three pages each
    inst = make_instance(workload(2))
    pool = op.PagePool(200)
    tree = op.ResidentTree(pool)
    (h,) = tree.prefill([(0, inst.prefixes[0])])
    assert tree.nodes[h].pages == list(range(125))
    pages = op.branch_pages(tree, [h] * 5, [b.tokens for b in inst.passes[0]])
    assert pages == [list(range(125 + 3 * i, 128 + 3 * i)) for i in range(5)]
    # config 4: request r -> 75r..75r+74; leaves from 1200, 4 pages each
    inst = make_instance(workload(4))
    pool = op.PagePool(2000)
    tree = op.ResidentTree(pool)
    hs = tree.prefill([(0, p) for p in inst.prefixes])
    for r, hh in enumerate(hs):
        assert tree.nodes[hh].pages == list(range(75 * r, 75 * r + 75))
    pages = op.branch_pages(tree, [hs[b.request] for b in inst.passes[0]],
                            [b.tokens for b in inst.passes[0]])
    assert pages[0] == [1200, 1201, 1202, 1203] and pages[-1] == [1708, 1709, 1710, 1711]
    # config 5: prefix 0..2047; both passes use leaves 2048..2559
    inst = make_instance(workload(5))
    pool = op.PagePool(3000)
    tree = op.ResidentTree(pool)
    (h,) = tree.prefill([(0, inst.prefixes[0])])
    assert tree.nodes[h].pages == list(range(2048))
    for p in range(2):
        pages = op.branch_pages(tree, [h] * 64, [b.tokens for b in inst.passes[p]])
        assert pages[0][0] == 2048 and pages[-1][-1] == 2559


def test_resident_match_dedupe_refcount_and_free():
    pool = op.PagePool(32)
    tree = op.ResidentTree(pool)
    (a,) = tree.prefill([(0, list(range(20)))])
    (b,) = tree.prefill([(a, list(range(20, 25)))])
    assert tree.prefill([(0, list(range(20)))]) == [a] and tree.nodes[a].refs == 2
    assert tree.match(list(range(30))) == (b, 25)
    assert tree.match(list(range(25))) == (a, 20)          # one token must stay
    assert tree.match(list(range(20))) == (0, 0)
    assert tree.match([5, 6]) == (0, 0)
    assert tree.path_pages(b) == [(0, 16), (1, 4), (2, 5)]
    tree.release(a)
    tree.release(a)                  # refs 0 but child b keeps it
    assert a in tree.nodes
    tree.release(b)                  # frees b, then a
    assert tree.nodes == {} and pool.n_free() == 32


def test_pool_exhaustion_is_all_or_nothing():
    pool = op.PagePool(10)
    tree = op.ResidentTree(pool)
    with pytest.raises(op.PoolExhausted):
        tree.prefill([(0, list(range(100))), (0, list(range(100, 200)))])
    assert pool.n_free() == 10 and tree.nodes == {}
    (h,) = tree.prefill([(0, list(range(100)))])         # 7 pages
    with pytest.raises(op.PoolExhausted):
        op.plan_candidates(tree, [list(range(100)) + [1] * 40, list(range(100)) + [2] * 40])
    assert pool.n_free() == 3
    plan = op.plan_candidates(tree, [list(range(100)) + [1] * 16, list(range(100)) + [2] * 16])
    assert [x.pages for x in plan.rounds[0]] == [[7], [8]]
