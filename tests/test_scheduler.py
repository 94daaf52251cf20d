"""Round-level continuous batching (jev_sched_*) on planning-only contexts:
plans, tree state and request states compared bit for bit with the oracle's
Scheduler model, plus invariants that hold whatever the model says."""
import threading

import numpy as np
import pytest

from oracle import plan as op
from shared_prefix_kv_amd import jev
from synth import workload

VOCAB = workload(1).model.vocab


def dry(n_pages=256, max_pos=1024):
    m = workload(1).model
    d = jev.make_desc(m.n_layers, m.d, m.hq, m.hkv, m.dh, m.vocab, m.dtype, m.rope_theta, m.eps, max_pos, max_pos)
    return jev.Context(d, n_pages)


def labels(n):
    return [[1, 2]] * n


def stats_view(st):
    return {k: st[k] for k in ("pages_in_use", "resident_prefixes", "cached_prefixes", "cached_pages", "evictions")}


def random_request(rng, bases):
    """Candidates continuing one of the shared bases (some shared inside the
    request, some across requests)."""
    base = bases[rng.integers(len(bases))]
    mid = [int(t) for t in rng.integers(0, VOCAB, int(rng.integers(0, 40)))]
    out = []
    for _ in range(int(rng.integers(1, 5))):
        tail = [int(t) for t in rng.integers(0, VOCAB, int(rng.integers(1, 20)))]
        out.append(base + (mid if rng.random() < 0.7 else []) + tail)
    return out


def run_both(script, n_pages, keep, counts):
    """script: list of lists of requests submitted before each step.  Refusals
    (submission, or a step that cannot fit) must agree too."""
    ctx = dry(n_pages)
    if keep:
        ctx.set_cache_policy(jev.JEV_CACHE_LRU)
    sch = jev.Scheduler(ctx)
    sess = op.Session(n_pages, keep=keep)
    ref = op.Scheduler(sess)
    tickets = []
    for reqs in script:
        for r in reqs:
            try:
                t = sch.submit(r, labels(len(r)))
            except jev.JevError as e:
                assert e.code == jev.JEV_ENOMEM
                with pytest.raises(op.PoolExhausted):
                    ref.submit(r)
                counts["refused"] += 1
                continue
            assert ref.submit(r) == t
            tickets.append(t)
        try:
            got = sch.step(want_plan=True)
        except jev.JevError as e:
            assert e.code == jev.JEV_ENOMEM
            with pytest.raises(op.PoolExhausted):
                ref.step()
            counts["failed_steps"] += 1
            return ctx, sch, tickets, False
        want = ref.step()
        assert got == (want.serialize() if want is not None else [])
        assert stats_view(ctx.stats()) == sess.stats()
        waiting = [t for t in tickets if ref.status(t) == 1 and not
                   next(r for r in ref.active if r["ticket"] == t)["started"]]
        counts["deferred"] += len(waiting)
        for t in tickets:
            assert sch.status(t) == ref.status(t)
    return ctx, sch, tickets, True


@pytest.mark.parametrize("keep", [False, True])
def test_random_request_streams_match_the_oracle(keep):
    rng = np.random.default_rng(1234 + keep)
    counts = {"refused": 0, "failed_steps": 0, "deferred": 0, "finished": 0}
    for trial in range(40):
        bases = [[int(t) for t in rng.integers(0, VOCAB, int(rng.integers(0, 50)))] for _ in range(3)]
        steps = int(rng.integers(2, 7))
        script = [[random_request(rng, bases) for _ in range(int(rng.integers(0, 3)))] for _ in range(steps)]
        script += [[] for _ in range(16)]       # drain
        n_pages = int(rng.integers(3, 100))
        ctx, sch, tickets, ok = run_both(script, n_pages, keep, counts)
        if ok:
            assert all(sch.status(t) == jev.JEV_SCHED_FINISHED for t in tickets)
            counts["finished"] += len(tickets)
            st = ctx.stats()
            if not keep:
                assert st["pages_in_use"] == 0 and st["resident_prefixes"] == 0
            else:
                assert st["resident_prefixes"] == st["cached_prefixes"]
        sch.close()
    # the streams exercised refusals, deferrals and completions
    assert counts["refused"] > 0 and counts["deferred"] > 0 and counts["finished"] > 50, counts


def test_one_request_takes_one_step_per_tree_level_and_computes_each_node_once():
    P = list(range(100, 140))                      # 40 shared tokens
    Q = list(range(200, 220))                      # 20 more shared by two of them
    seqs = [P + Q + [1], P + Q + [2, 3], P + [4], P + [5, 6, 7]]
    ctx = dry()
    sch = jev.Scheduler(ctx)
    t = sch.submit(seqs, labels(4))
    computed, steps = 0, 0
    while sch.status(t) != jev.JEV_SCHED_FINISHED:
        sch.step()
        computed += ctx.stats()["computed_tokens"]
        steps += 1
    assert steps == 3                              # P, then Q and the two leaves under P, then Q's leaves
    trie_tokens = len(P) + len(Q) + 1 + 2 + 1 + 3
    assert computed == trie_tokens
    assert ctx.stats()["pages_in_use"] == 0


def test_a_late_request_joins_the_running_round_and_shares_its_prefix():
    P = list(range(300, 348))                      # 3 pages
    first = [P + [1, 2], P + [3]]
    late = [P + [9], [7] * 30 + [1], [7] * 30 + [2]]
    ctx = dry()
    sch = jev.Scheduler(ctx)
    t1 = sch.submit(first, labels(2))
    sch.step()                                     # computes P, held
    assert ctx.stats()["computed_tokens"] == len(P)
    t2 = sch.submit(late, labels(3))
    plan = sch.step(want_plan=True)
    # one round: first's two leaves and late's leaf under P (P not recomputed),
    # and late's shared [7]*30 node
    st = ctx.stats()
    assert st["computed_tokens"] == 2 + 1 + 1 + 30
    assert sch.status(t1) == jev.JEV_SCHED_FINISHED and sch.status(t2) == jev.JEV_SCHED_ACTIVE
    assert plan[0] == 2                            # the plan has two rounds; only the first ran
    sch.step()
    assert sch.status(t2) == jev.JEV_SCHED_FINISHED
    assert ctx.stats()["pages_in_use"] == 0 and ctx.stats()["resident_prefixes"] == 0


def test_total_compute_equals_one_call_over_all_candidates():
    rng = np.random.default_rng(7)
    for _ in range(20):
        bases = [[int(t) for t in rng.integers(0, VOCAB, int(rng.integers(16, 60)))] for _ in range(2)]
        reqs = [random_request(rng, bases) for _ in range(4)]
        ctx = dry(512)
        sch = jev.Scheduler(ctx)
        tickets = [sch.submit(r, labels(len(r))) for r in reqs]
        total = 0
        while any(sch.status(t) != jev.JEV_SCHED_FINISHED for t in tickets):
            sch.step()
            total += ctx.stats()["computed_tokens"]
        allc = [s for r in reqs for s in r]
        plan = op.plan_candidates(op.ResidentTree(op.PagePool(512)), allc)
        assert total == sum(x.b - x.a for rnd in plan.rounds for x in rnd)


def test_errors_leave_the_scheduler_unchanged():
    ctx = dry(8)
    sch = jev.Scheduler(ctx)
    with pytest.raises(jev.JevError) as e:
        sch.submit([[1, 2]], [[1]])                # one label
    assert e.value.code == jev.JEV_EINVAL
    with pytest.raises(jev.JevError) as e:
        sch.submit([[VOCAB]], [[1, 2]])            # token out of range
    assert e.value.code == jev.JEV_EINVAL
    with pytest.raises(jev.JevError) as e:
        sch.status(99)
    assert e.value.code == jev.JEV_EHANDLE
    big = [list(range(1, 200)) + [5], list(range(1, 200)) + [6]]   # 13 pages: cannot fit 8 even alone
    with pytest.raises(jev.JevError) as e:
        sch.submit(big, labels(2))
    assert e.value.code == jev.JEV_ENOMEM
    t = sch.submit([list(range(1, 60)) + [5], list(range(1, 60)) + [6]], labels(2))   # 4 + 1 + 1 pages
    with pytest.raises(jev.JevError) as e:
        sch.result(t)
    assert e.value.code == jev.JEV_EPENDING
    n = np.zeros(1, dtype=np.int64)
    buf = np.zeros(1, dtype=np.int32)
    import ctypes
    rc = jev.lib().jev_sched_step(sch.s, None, jev._ptr(buf, ctypes.c_int32), 1, jev._ptr(n, ctypes.c_int64))
    assert rc == jev.JEV_EINVAL                                     # plan_out too small: nothing ran
    assert sch.status(t) == jev.JEV_SCHED_ACTIVE and ctx.stats()["pages_in_use"] == 0
    sch.step()
    sch.step()
    assert sch.status(t) == jev.JEV_SCHED_FINISHED and ctx.stats()["pages_in_use"] == 0


def test_a_request_that_does_not_fit_next_to_running_ones_waits():
    ctx = dry(12)
    sch = jev.Scheduler(ctx)
    A = [list(range(1, 100)) + [5], list(range(1, 100)) + [6, 7]]     # 7 pages held, then 1 + 1
    B = [list(range(200, 280)) + [5], list(range(200, 280)) + [6]]    # 5 + 1 + 1 pages
    ta = sch.submit(A, labels(2))
    sch.step()                                                         # A's shared node held (7 pages)
    tb = sch.submit(B, labels(2))
    sch.step()                                                         # A's leaves; B does not fit beside A
    assert sch.status(ta) == jev.JEV_SCHED_FINISHED
    assert sch.status(tb) == jev.JEV_SCHED_ACTIVE and ctx.stats()["computed_tokens"] == 3
    sch.step()
    sch.step()
    assert sch.status(tb) == jev.JEV_SCHED_FINISHED and ctx.stats()["pages_in_use"] == 0


def test_concurrent_submitters():
    ctx = dry(1024)
    sch = jev.Scheduler(ctx)
    got = [[] for _ in range(4)]

    def worker(k):
        rng = np.random.default_rng(100 + k)
        for _ in range(25):
            r = [[int(t) for t in rng.integers(0, VOCAB, 5)] + [k, i] for i in range(2)]
            got[k].append(sch.submit(r, labels(2)))

    th = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
    for x in th:
        x.start()
    for _ in range(3):
        sch.step()
    for x in th:
        x.join()
    tickets = [t for g in got for t in g]
    assert sorted(tickets) == list(range(1, 101))
    for _ in range(10):
        sch.step()
    assert all(sch.status(t) == jev.JEV_SCHED_FINISHED for t in tickets)
    assert ctx.stats()["pages_in_use"] == 0


def test_repeated_state_is_checkpointed_under_the_cache_policy():
    """A state shared by a request's candidates stays cached after the request
    (cache policy on): a later request over the same state computes only its
    own tokens, in one step.  With the policy off it is recomputed."""
    S = [int(t) for t in np.random.default_rng(3).integers(0, VOCAB, 70)]
    for keep in (True, False):
        ctx = dry(64)
        if keep:
            ctx.set_cache_policy(jev.JEV_CACHE_LRU)
        sch = jev.Scheduler(ctx)
        a = sch.submit([S + [1, 2], S + [3]], labels(2))
        sch.step()
        sch.step()
        assert sch.status(a) == jev.JEV_SCHED_FINISHED
        b = sch.submit([S + [4, 5, 6], S + [7]], labels(2))
        sch.step()
        if keep:
            assert sch.status(b) == jev.JEV_SCHED_FINISHED
            assert ctx.stats()["computed_tokens"] == 3 + 1
            assert ctx.stats()["cached_prefixes"] == 1 and ctx.stats()["cached_pages"] == 5
        else:
            assert sch.status(b) == jev.JEV_SCHED_ACTIVE
            assert ctx.stats()["computed_tokens"] == len(S)


def test_closing_the_context_first_closes_its_schedulers():
    ctx = dry(64)
    sch = jev.Scheduler(ctx)
    t = sch.submit([[1, 2, 3], [1, 2, 4]], labels(2))
    sch.step()
    ctx.close()                                   # destroys the scheduler first
    assert not sch.s
    sch.close()                                   # no-op
    ctx2 = dry(64)
    sch2 = jev.Scheduler(ctx2)
    t2 = sch2.submit([[5, 6]], labels(1))
    sch2.step()
    assert sch2.status(t2) == jev.JEV_SCHED_FINISHED
    with pytest.raises(jev.JevError) as e:
        sch2.result(t2)                           # planning-only context: no scores
    assert e.value.code == jev.JEV_ESTATE
    with pytest.raises(jev.JevError) as e:
        sch2.status(t + 100)
    assert e.value.code == jev.JEV_EHANDLE


def test_destroying_the_context_first_detaches_its_schedulers():
    """A context destroyed before its scheduler (as a garbage collector may
    finalise them in either order) detaches it: later calls fail with
    JEV_ESTATE instead of reading freed memory, and destroying the scheduler
    still works.  Raw C ABI calls, so the binding's own ordering cannot help."""
    import ctypes
    L = jev.lib()
    ctx = dry(64)
    sch = jev.Scheduler(ctx)
    t = sch.submit([[1, 2, 3, 4]], labels(1))
    raw_ctx, raw_s = ctx.ctx, sch.s
    assert L.jev_destroy(raw_ctx) == jev.JEV_OK
    ctx.ctx = ctypes.c_void_p()              # the binding no longer owns it
    state = ctypes.c_int32()
    assert L.jev_sched_status(raw_s, t, ctypes.byref(state)) == jev.JEV_OK
    tk = ctypes.c_int64()
    flat = np.array([1, 2, 3], np.int32)
    off = np.array([0, 3], np.int64)
    lab = np.array([1, 2], np.int32)
    loff = np.array([0, 2], np.int64)
    P = lambda a, t_: a.ctypes.data_as(ctypes.POINTER(t_))
    rc = L.jev_sched_submit(raw_s, 1, P(flat, ctypes.c_int32), P(off, ctypes.c_int64), P(lab, ctypes.c_int32),
                            P(loff, ctypes.c_int64), ctypes.byref(tk))
    assert rc == jev.JEV_ESTATE
    n = ctypes.c_int64()
    assert L.jev_sched_step(raw_s, None, None, 0, ctypes.byref(n)) == jev.JEV_ESTATE
    assert L.jev_sched_destroy(raw_s) == jev.JEV_OK
    sch.s = ctypes.c_void_p()
