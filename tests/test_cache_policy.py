"""Resident-prefix cache policy (jev_set_cache_policy), on the CPU.

openjev-multimodal performance page, repeated-state section: the KV at the
end of a repeated state is kept for the next request, and several states can
be kept and used in turn (four 800-token states in rotation).  With
JEV_CACHE_LRU a prefix whose last reference is dropped stays resident; a call
short of pages evicts cached prefixes without children, least recently used
first.  Every handle, page table, stat and plan is compared bit for bit with
the oracle's call-level model (oracle/plan.py, Session).
"""
import numpy as np
import pytest

from oracle import plan as op
from synth import workload

jev = pytest.importorskip("shared_prefix_kv_amd.jev")


def dry(n_pages, mode=None, keep=True):
    m = workload(1).model
    desc = jev.make_desc(m.n_layers, m.d, m.hq, m.hkv, m.dh, m.vocab, m.dtype, m.rope_theta, m.eps, 40000, 4096)
    ctx = jev.Context(desc, n_pages)
    if keep:
        ctx.set_cache_policy(jev.JEV_CACHE_LRU)
    if mode is not None:
        ctx.set_plan_mode(mode)
    return ctx


def same_state(ctx, ses, live):
    st = ctx.stats()
    for k, v in ses.stats().items():
        assert st[k] == v, k
    for h in live:
        pages, valid = ctx.page_table(h)
        assert list(zip(pages, valid)) == ses.tree.path_pages(h)


def test_rotating_states_hit_and_evict_least_recently_used():
    states = [list(range(60 * i, 60 * i + 50)) for i in range(4)]   # 4 pages each
    ctx, ses = dry(13), op.Session(13, keep=True)
    for rnd in range(3):
        for s in states:
            (h,) = ctx.prefill_prefix([0], [s])
            assert [h] == ses.prefill([(0, s)])
            same_state(ctx, ses, [h])
            ctx.free_pages([h])
            ses.release([h])
            same_state(ctx, ses, [])
    st = ctx.stats()
    # 13 pages hold three 4-page states: every new state evicts the oldest
    assert st["cached_prefixes"] == 3 and st["cached_pages"] == 12 and st["evictions"] == 9
    # the most recent state is a hit: same handle, no pages taken
    before = ctx.stats()["pages_in_use"]
    (h,) = ctx.prefill_prefix([0], [states[3]])
    assert [h] == ses.prefill([(0, states[3])])
    assert ctx.stats()["pages_in_use"] == before and ctx.stats()["cached_prefixes"] == 2
    same_state(ctx, ses, [h])


def test_referenced_paths_are_never_evicted():
    ctx, ses = dry(6), op.Session(6, keep=True)
    (a,) = ctx.prefill_prefix([0], [list(range(32))])          # 2 pages, kept referenced
    assert [a] == ses.prefill([(0, list(range(32)))])
    (b,) = ctx.prefill_prefix([a], [list(range(32, 64))])      # 2 pages under a, then cached
    assert [b] == ses.prefill([(a, list(range(32, 64)))])
    ctx.free_pages([b]); ses.release([b])
    # 3 pages needed, 2 free: only b can go
    (c,) = ctx.prefill_prefix([0], [list(range(200, 240))])
    assert [c] == ses.prefill([(0, list(range(200, 240)))])
    same_state(ctx, ses, [a, c])
    assert ctx.stats()["evictions"] == 1
    # nothing left to evict: all-or-nothing ENOMEM
    with pytest.raises(jev.JevError) as e:
        ctx.prefill_prefix([a], [list(range(64, 96))])
    assert e.value.code == jev.JEV_ENOMEM
    same_state(ctx, ses, [a, c])


def test_switching_back_to_release_frees_the_cache():
    ctx, ses = dry(40), op.Session(40, keep=True)
    hs = ctx.prefill_prefix([0, 0], [list(range(40)), list(range(100, 130))])
    assert hs == ses.prefill([(0, list(range(40))), (0, list(range(100, 130)))])
    (k,) = ctx.prefill_prefix([hs[0]], [list(range(40, 60))])
    assert [k] == ses.prefill([(hs[0], list(range(40, 60)))])
    ctx.free_pages([hs[0], hs[1]]); ses.release([hs[0], hs[1]])
    same_state(ctx, ses, [k])
    ctx.set_cache_policy(jev.JEV_CACHE_RELEASE); ses.set_keep(False)
    same_state(ctx, ses, [k])
    st = ctx.stats()
    assert st["cached_prefixes"] == 1 and st["resident_prefixes"] == 2   # hs[0] stays under k
    with pytest.raises(jev.JevError) as e:
        ctx.set_cache_policy(7)
    assert e.value.code == jev.JEV_EINVAL


@pytest.mark.parametrize("seed", range(40))
def test_random_call_sequences_match_the_oracle(seed):
    rng = np.random.default_rng(4000 + seed)
    n_pages = int(rng.integers(8, 60))
    mode = ["depth", "candidate_first"][seed % 2]
    ctx = dry(n_pages, mode=[jev.JEV_PLAN_DEPTH, jev.JEV_PLAN_CANDIDATE_FIRST][seed % 2])
    ses = op.Session(n_pages, mode=mode, keep=True)
    base = [int(x) for x in rng.integers(0, 4, 200)]
    live = []                 # caller references held (handles, with repeats)
    for step in range(40):
        op_kind = int(rng.integers(0, 4))
        if op_kind <= 1:      # prefill one or two segments
            items = []
            for _ in range(int(rng.integers(1, 3))):
                parent = live[int(rng.integers(0, len(live)))] if live and rng.random() < 0.5 else 0
                cut = int(rng.integers(1, 60))
                start = int(rng.integers(0, 3)) * 16
                items.append((parent, base[start:start + cut]))
            try:
                want = ses.prefill(items)
            except op.PoolExhausted:
                with pytest.raises(jev.JevError) as e:
                    ctx.prefill_prefix([p for p, _ in items], [t for _, t in items])
                assert e.value.code == jev.JEV_ENOMEM
                continue
            got = ctx.prefill_prefix([p for p, _ in items], [t for _, t in items])
            assert got == want
            live += got
        elif op_kind == 2 and live:   # release one reference
            h = live.pop(int(rng.integers(0, len(live))))
            ctx.free_pages([h])
            ses.release([h])
        else:                 # plan a few candidates (changes nothing)
            seqs = [base[:int(rng.integers(10, 120))] + [int(x) for x in rng.integers(0, 4, int(rng.integers(1, 30)))]
                    for _ in range(int(rng.integers(1, 5)))]
            try:
                want = ses.plan(seqs).serialize()
            except op.PoolExhausted:
                with pytest.raises(jev.JevError) as e:
                    ctx.plan(seqs)
                assert e.value.code == jev.JEV_ENOMEM
                continue
            assert ctx.plan(seqs) == want
        same_state(ctx, ses, sorted(set(live)))
